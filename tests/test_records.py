"""Host logic of the group records: the binding's inverse permutation
(records_to_arrays), which the GPU parity tests use to compare a device
cache with the oracle's per-array layout, must be a bijection between the
record's bytes and the per-array bytes of one group, for both K lane roles,
both bit widths and both scale/zero formats; and the record must hold the
same number of bytes as the per-array layout (no padding)."""
import numpy as np
import pytest

from decode_attention_channel_amd import kivi


def _ids(bits, meta, valu_k):
    rec_bytes = 1024 * (bits + (1 if meta else 2))
    pos = np.arange(rec_bytes)
    lo = kivi.records_to_arrays((pos & 0xFF).astype(np.uint8)[None], bits, meta, valu_k)
    hi = kivi.records_to_arrays((pos >> 8).astype(np.uint8)[None], bits, meta, valu_k)
    out = {}
    for name in lo:
        a = np.ascontiguousarray(lo[name]).view(np.uint8).reshape(-1).astype(np.int64)
        b = np.ascontiguousarray(hi[name]).view(np.uint8).reshape(-1).astype(np.int64)
        out[name] = a | (b << 8)
    return rec_bytes, out


@pytest.mark.parametrize("valu_k", [False, True])
@pytest.mark.parametrize("bits,meta", [(2, 0), (4, 0), (2, 1), (4, 1)])
def test_record_inverse_is_a_bijection(bits, meta, valu_k):
    rec_bytes, ids = _ids(bits, meta, valu_k)
    D, G, mb = 128, 32, 2 if meta else 4
    sizes = {"k_codes": G * D * bits // 8, "k_scale": D * mb, "k_zero": D * mb,
             "v_codes": G * D * bits // 8, "v_scale": D * mb, "v_zero": D * mb}
    for name, n in sizes.items():
        assert ids[name].size == n, name
    allids = np.concatenate([ids[n] for n in sizes])
    assert allids.size == rec_bytes
    assert np.array_equal(np.sort(allids), np.arange(rec_bytes))


@pytest.mark.parametrize("bits", [2, 4])
def test_key_roles_differ_only_in_the_key_planes(bits):
    # both K lane roles share the V and scale/zero planes; their K codes are
    # two permutations of the same code planes
    _, mfma = _ids(bits, 0, False)
    _, valu = _ids(bits, 0, True)
    for name in ("k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        assert np.array_equal(mfma[name], valu[name]), name
    assert not np.array_equal(mfma["k_codes"], valu["k_codes"])
    assert np.array_equal(np.sort(mfma["k_codes"]), np.sort(valu["k_codes"]))
    assert mfma["k_codes"].max() < 1024 * bits // 2


def test_valu_key_pieces_follow_the_lane_roles():
    # q_per_kv = 1 readers: lane 8 k + c reads, at its 16 bytes of each K
    # plane, channels 16 c .. 16 c + 15 of token rows 4 k .. 4 k + 3
    _, ids = _ids(2, 0, True)
    k = ids["k_codes"].reshape(32, 32)         # [row][byte], 4 channels per byte
    for t in range(32):
        for c in range(8):
            lane = 8 * (t // 4) + c
            got = k[t, 4 * c:4 * c + 4]
            assert np.all(got // 16 == lane) and np.all(got < 1024), (t, c)
    _, ids = _ids(4, 0, True)
    k = ids["k_codes"].reshape(32, 64)         # 2 channels per byte
    for t in range(32):
        for c in range(8):
            got = k[t, 8 * c:8 * c + 8]
            assert np.all((got % 1024) // 16 == 8 * (t // 4) + c), (t, c)
            assert np.all(got // 1024 == (t % 4) // 2), (t, c)
