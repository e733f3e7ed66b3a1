"""Host logic of the group records: the binding's inverse permutation
(records_to_arrays), which the GPU parity tests use to compare a device
cache with the oracle's per-array layout, must be a bijection between the
record's bytes and the per-array bytes of one group, for both bit widths and
both scale/zero formats, and must put each K piece where the decode lanes
read it; the record holds the same number of bytes as the per-array layout
(no padding)."""
import numpy as np
import pytest

from decode_attention_channel_amd import kivi


def _ids(bits, meta):
    rec_bytes = 1024 * (bits + (1 if meta else 2))
    pos = np.arange(rec_bytes)
    lo = kivi.records_to_arrays((pos & 0xFF).astype(np.uint8)[None], bits, meta)
    hi = kivi.records_to_arrays((pos >> 8).astype(np.uint8)[None], bits, meta)
    out = {}
    for name in lo:
        a = np.ascontiguousarray(lo[name]).view(np.uint8).reshape(-1).astype(np.int64)
        b = np.ascontiguousarray(hi[name]).view(np.uint8).reshape(-1).astype(np.int64)
        out[name] = a | (b << 8)
    return rec_bytes, out


@pytest.mark.parametrize("bits,meta", [(2, 0), (4, 0), (2, 1), (4, 1)])
def test_record_inverse_is_a_bijection(bits, meta):
    rec_bytes, ids = _ids(bits, meta)
    D, G, mb = 128, 32, 2 if meta else 4
    sizes = {"k_codes": G * D * bits // 8, "k_scale": D * mb, "k_zero": D * mb,
             "v_codes": G * D * bits // 8, "v_scale": D * mb, "v_zero": D * mb}
    for name, n in sizes.items():
        assert ids[name].size == n, name
    allids = np.concatenate([ids[n] for n in sizes])
    assert allids.size == rec_bytes
    assert np.array_equal(np.sort(allids), np.arange(rec_bytes))


@pytest.mark.parametrize("bits", [2, 4])
def test_key_pieces_follow_the_lane_roles(bits):
    # lane 16 j + 4 (t >> 3) + (t & 3), for t with (t >> 2) & 1 == 0, reads
    # the 32-channel block j of token rows t and t + 4 (the two MFMA tiles):
    # 2-bit, 8 bytes each in plane 0; 4-bit, 16 bytes each in planes 0, 1
    _, ids = _ids(bits, 0)
    piece = 4 * bits
    k = ids["k_codes"].reshape(32, 4, piece)   # [row][block j][bytes]
    for t in range(32):
        if (t >> 2) & 1:
            continue
        for j in range(4):
            lane = 16 * j + 4 * (t >> 3) + (t & 3)
            for tile, row in enumerate((t, t + 4)):
                got = k[row, j]
                if bits == 2:
                    want = lane * 16 + 8 * tile + np.arange(8)
                else:
                    want = tile * 1024 + lane * 16 + np.arange(16)
                assert np.array_equal(got, want), (t, j, tile)
