// quantize.hip -- KIVI group quantiser for prefill and residual flush, plus
// the bf16 row copies that fill the residual ring.
//
// Method ("KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache",
// method paragraph; catalog record kivi-2bit-llama3-8b-gqa-8k, Methodology):
// keys are grouped along the token axis of each channel (per-channel), values
// along 32 channels of each token (per-token), G = 32, asymmetric min-max
// scale/zero, 2- or 4-bit codes.  Every float operation of the quantiser is a
// single IEEE fp32 operation, rounded to nearest even, nothing fused:
//     s = (max - min) / L ;  inv = s >= FLT_MIN ? 1 / s : 0 ;
//     code = clamp(rint((x - min) * inv), 0, L) ;  scale = s, zero = min.
// With the 16-bit scale/zero format the scale is first rounded to fp16 and
// the codes use the rounded value; the zero is stored as bf16 (exact).
//
// Each workgroup takes `gpw` consecutive groups (one by default) of one unit:
// two waves quantise the keys (one channel half each), two waves the values
// (one token half each), independently (see quantize_keys / quantize_values).  Codes
// are staged as bytes in a per-wave LDS tile and re-read in the order of the
// packed layout, so the global stores are coalesced.
#pragma clang fp contract(off)

#include <float.h>
#include <stdlib.h>

#include "kivi_internal.h"

namespace kivi {
namespace {

template <int BITS>
struct Q {
  static constexpr float kLevels = (float)((1 << BITS) - 1);
};

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// Scale and reciprocal of one group.  META == 1 (fp16 scale): the scale is
// rounded to fp16 (nearest even; clamping to 65504 first makes overflow
// saturate) and the codes are computed from the rounded value; s_bits gets
// the fp16 bits.
template <int BITS, int META>
__device__ __forceinline__ void group_params(float mn, float mx, float &s, float &inv,
                                             uint32_t &s_bits) {
  s = __fdiv_rn(__fsub_rn(mx, mn), Q<BITS>::kLevels);
  s_bits = 0;
  if constexpr (META == 1) {
    const _Float16 h = (_Float16)fminf(s, 65504.0f);
    s_bits = __builtin_bit_cast(uint16_t, h);
    s = (float)h;
  }
  inv = (s >= FLT_MIN) ? __fdiv_rn(1.0f, s) : 0.0f;
}

// The quantiser reads each bf16 input byte once and writes each record byte
// once, nothing in the same launch reading it back, so both go through the
// non-temporal path.  8K GQA prefill on MI355X: 5.62-5.65 TB/s with cached
// loads and stores, 5.77-5.86 with non-temporal stores only, 5.47-5.50 with
// non-temporal loads only, 6.22-6.30 with both.
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(uint8_t *p, uint32_t x, uint32_t y) {
  __builtin_nontemporal_store(u32x2_nt{x, y}, reinterpret_cast<u32x2_nt *>(p));
}
__device__ __forceinline__ void store_nt(uint8_t *p, uint32_t x, uint32_t y, uint32_t z,
                                         uint32_t w) {
  __builtin_nontemporal_store(u32x4_nt{x, y, z, w}, reinterpret_cast<u32x4_nt *>(p));
}
__device__ __forceinline__ void store_nt(uint8_t *p, uint32_t x) {
  __builtin_nontemporal_store(x, reinterpret_cast<uint32_t *>(p));
}
__device__ __forceinline__ void store_nt(uint8_t *p, uint16_t x) {
  __builtin_nontemporal_store(x, reinterpret_cast<uint16_t *>(p));
}

// bf16 bits of a group minimum (a widened bf16 value: exact)
__device__ __forceinline__ uint32_t zero_bits(float mn) { return __float_as_uint(mn) >> 16; }

template <int BITS>
__device__ __forceinline__ uint32_t code_of(float x, float mn, float inv) {
  float y = rintf(__fmul_rn(__fsub_rn(x, mn), inv));
  y = fminf(fmaxf(y, 0.0f), Q<BITS>::kLevels);
  return (uint32_t)y;
}

// four byte-codes (one per byte, each < 4) -> one byte of 2-bit codes
__device__ __forceinline__ uint32_t pack4x2(uint32_t x) {
  const uint32_t y = x | (x >> 6);
  return (y & 0xFu) | ((y >> 12) & 0xF0u);
}
// four byte-codes (each < 16) -> 16 bits of 4-bit codes
__device__ __forceinline__ uint32_t pack4x4(uint32_t x) {
  const uint32_t y = x | (x >> 4);
  return (y & 0xFFu) | ((y >> 8) & 0xFF00u);
}

// min / max of x over lanes l and l ^ 32.  permlane32_swap of x with itself
// returns, in lanes 0-31, (x[l], x[l + 32]) and, in lanes 32-63,
// (x[l - 32], x[l]): the pair always holds both values.
__device__ __forceinline__ float min_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Byte offsets inside a group record (kivi_internal.h).  K piece: token row
// t, 32-channel block j; V cell: octet o, channels 4 c4 .. 4 c4 + 3; scale /
// zero value v (0..127) of array i (0 k_scale, 1 k_zero, 2 v_scale, 3 v_zero).
template <int BITS>
__device__ __forceinline__ int rec_k_piece(int t, int j) {
  const int lane = 16 * j + 4 * (t >> 3) + (t & 3), tile = (t >> 2) & 1;
  return BITS == 2 ? lane * 16 + tile * 8 : tile * kPlaneBytes + lane * 16;
}
template <int BITS>
__device__ __forceinline__ int rec_v_cell(int o, int c4) {
  const int lane = 16 * o + (c4 >> 1);
  return BITS == 2 ? kPlaneBytes + lane * 16 + (c4 & 1) * 8
                   : (2 + (c4 & 1)) * kPlaneBytes + lane * 16;
}
template <int BITS, int META>
__device__ __forceinline__ int rec_meta(int i, int v) {
  const int lane = v >> 1, e = v & 1;
  return META == 1 ? BITS * kPlaneBytes + lane * 16 + i * 4 + e * 2
                   : (BITS + (i >> 1)) * kPlaneBytes + lane * 16 + (i & 1) * 8 + e * 4;
}

// One wave quantises the keys of one half of the channels (64) of each of
// its groups.  Lane (pair p, row half h) owns channels cb+2p, cb+2p+1 of rows
// 16h..16h+15: the per-channel min/max over 32 tokens is 16 values in
// registers plus one exchange with lane ^ 32.  Byte codes go through the
// wave's LDS tile ([row][64 channels]) and come back in packed row order.
template <int BITS, int META>
__device__ __forceinline__ void key_group(const QuantizeArgs &a, int u, int gl,
                                          const uint32_t (&raw)[16], int cb, int lane,
                                          uint8_t *tile) {
  const int p = lane & 31, h = lane >> 5;
  const long long slot = group_slot(a.pages, a.kv_heads, a.n_groups_cap, u, a.dst_g0 + gl);
  if (slot < 0) return;   // paged: no page for this group
  float x0[16], x1[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x0[i] = bf16_lo(raw[i]);
    x1[i] = bf16_hi(raw[i]);
  }
  float mn0 = x0[0], mx0 = x0[0], mn1 = x1[0], mx1 = x1[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    mn0 = fminf(mn0, x0[i]); mx0 = fmaxf(mx0, x0[i]);
    mn1 = fminf(mn1, x1[i]); mx1 = fmaxf(mx1, x1[i]);
  }
  // the other row half of the same channels sits in lane ^ 32
  mn0 = min_x32(mn0); mx0 = max_x32(mx0);
  mn1 = min_x32(mn1); mx1 = max_x32(mx1);
  float sc0, inv0, sc1, inv1;
  uint32_t sb0, sb1;
  group_params<BITS, META>(mn0, mx0, sc0, inv0, sb0);
  group_params<BITS, META>(mn1, mx1, sc1, inv1, sb1);
  if (h == 0) {
    uint8_t *rec = a.records + slot * rec_bytes(BITS, META);
    const int c = cb + 2 * p;   // channels c, c + 1: one lane's value pair
    if constexpr (META == 1) {
      store_nt(rec + rec_meta<BITS, META>(0, c), sb0 | (sb1 << 16));
      store_nt(rec + rec_meta<BITS, META>(1, c), zero_bits(mn0) | (zero_bits(mn1) << 16));
    } else {
      store_nt(rec + rec_meta<BITS, META>(0, c), __float_as_uint(sc0), __float_as_uint(sc1));
      store_nt(rec + rec_meta<BITS, META>(1, c), __float_as_uint(mn0), __float_as_uint(mn1));
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t c = code_of<BITS>(x0[i], mn0, inv0) | (code_of<BITS>(x1[i], mn1, inv1) << 8);
    reinterpret_cast<uint16_t *>(tile + (16 * h + i) * 64)[p] = (uint16_t)c;
  }
  __builtin_amdgcn_wave_barrier();
  // pack: lane -> (row lane/2, 32 channels)
  const int row = lane >> 1, c32 = 32 * (lane & 1);
  const uint4 b0 = *reinterpret_cast<const uint4 *>(tile + row * 64 + c32);
  const uint4 b1 = *reinterpret_cast<const uint4 *>(tile + row * 64 + c32 + 16);
  // the packed row piece: 32 channels of token `row`
  uint8_t *dst = a.records + slot * rec_bytes(BITS, META) + rec_k_piece<BITS>(row, (cb + c32) / 32);
  if constexpr (BITS == 2) {
    const uint32_t w0 = pack4x2(b0.x) | (pack4x2(b0.y) << 8) | (pack4x2(b0.z) << 16) |
                        (pack4x2(b0.w) << 24);
    const uint32_t w1 = pack4x2(b1.x) | (pack4x2(b1.y) << 8) | (pack4x2(b1.z) << 16) |
                        (pack4x2(b1.w) << 24);
    store_nt(dst, w0, w1);
  } else {
    store_nt(dst, pack4x4(b0.x) | (pack4x4(b0.y) << 16), pack4x4(b0.z) | (pack4x4(b0.w) << 16),
             pack4x4(b1.x) | (pack4x4(b1.y) << 16), pack4x4(b1.z) | (pack4x4(b1.w) << 16));
  }
  __builtin_amdgcn_wave_barrier();   // tile reads done before the next group's writes
}

template <int BITS, int META>
__device__ __forceinline__ void quantize_keys(const QuantizeArgs &a, int u, int gl0, int gl1,
                                              int half, int lane, uint8_t *tile) {
  constexpr int D = kHeadDim, G = kGroup;
  const int p = lane & 31, h = lane >> 5, cb = 64 * half;
  const uint32_t *src = reinterpret_cast<const uint32_t *>(
      a.src_k + (long long)u * a.src_unit_stride + (long long)a.src_tok0 * D);
  const int col = cb / 2 + p;   // 32-bit column of this lane's channel pair
  auto load = [&](int gl, uint32_t (&x)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      x[i] = __builtin_nontemporal_load(&src[((long long)gl * G + 16 * h + i) * (D / 2) + col]);
  };
  // software pipeline: the loop always loads the next group (the last group
  // is peeled off), so each step waits only for its own rows
  uint32_t cur[16], nxt[16];
  load(gl0, nxt);
  for (int gl = gl0; gl + 1 < gl1; ++gl) {
#pragma unroll
    for (int i = 0; i < 16; ++i) cur[i] = nxt[i];
    load(gl + 1, nxt);
    key_group<BITS, META>(a, u, gl, cur, cb, lane, tile);
  }
  key_group<BITS, META>(a, u, gl1 - 1, nxt, cb, lane, tile);
}

// One wave quantises the values of 16 tokens (two octets) of each of its
// groups.  Lane (row r, quarter q) owns channels 32q..32q+31 of token r: one
// whole value group, min/max in registers.  Byte codes go through the wave's
// LDS tile ([row][128 channels]) and are regathered as octet x channel cells.
template <int BITS, int META>
__device__ __forceinline__ void value_group(const QuantizeArgs &a, int u, int gl,
                                            const uint4 (&raw)[4], int part, int lane,
                                            uint8_t *tile) {
  constexpr int D = kHeadDim, G = kGroup;
  const int r = lane >> 2, q = lane & 3;
  const long long slot = group_slot(a.pages, a.kv_heads, a.n_groups_cap, u, a.dst_g0 + gl);
  if (slot < 0) return;   // paged: no page for this group
  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * i + 2 * e] = bf16_lo(w[e]);
      x[8 * i + 2 * e + 1] = bf16_hi(w[e]);
    }
  }
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
  float sc, inv;
  uint32_t sb;
  group_params<BITS, META>(mn, mx, sc, inv, sb);
  {
    uint8_t *rec = a.records + slot * rec_bytes(BITS, META);
    const int v = q * G + 16 * part + r;   // value index within the group
    if constexpr (META == 1) {
      store_nt(rec + rec_meta<BITS, META>(2, v), (uint16_t)sb);
      store_nt(rec + rec_meta<BITS, META>(3, v), (uint16_t)zero_bits(mn));
    } else {
      store_nt(rec + rec_meta<BITS, META>(2, v), __float_as_uint(sc));
      store_nt(rec + rec_meta<BITS, META>(3, v), __float_as_uint(mn));
    }
  }
  uint32_t cw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    cw[i] = code_of<BITS>(x[4 * i], mn, inv) | (code_of<BITS>(x[4 * i + 1], mn, inv) << 8) |
            (code_of<BITS>(x[4 * i + 2], mn, inv) << 16) |
            (code_of<BITS>(x[4 * i + 3], mn, inv) << 24);
  uint4 *t = reinterpret_cast<uint4 *>(tile + r * D + 32 * q);
  t[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
  t[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
  __builtin_amdgcn_wave_barrier();
  // cells: lane -> (octet o, channels 4c4..4c4+3), 8 tokens each
  const int o = lane >> 5, c4 = lane & 31;
  uint32_t cell[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(tile + (8 * o + k) * D + 4 * c4);
#pragma unroll
    for (int i = 0; i < 4; ++i) cell[i] |= ((w >> (8 * i)) & 0xFFu) << (BITS * k);
  }
  uint8_t *dst = a.records + slot * rec_bytes(BITS, META) + rec_v_cell<BITS>(2 * part + o, c4);
  if constexpr (BITS == 2) {
    store_nt(dst, cell[0] | (cell[1] << 16), cell[2] | (cell[3] << 16));
  } else {
    store_nt(dst, cell[0], cell[1], cell[2], cell[3]);
  }
  __builtin_amdgcn_wave_barrier();
}

// Row stride of the value staging tile, in 16-byte units: 17 (one unit of
// padding) keeps both its row-wise writes and the (row r, channel group q)
// reads free of bank conflicts.
constexpr int kStageStride = kHeadDim / 8 + 1;

// In place: x holds load i's piece (row 4i + lr, channels 8 lc .. + 7) on
// entry and the lane's value group (row r, channels 32q + 8i .. + 7) on exit.
__device__ __forceinline__ void regather_values(uint4 (&x)[4], uint4 *stage, int lr, int lc, int r,
                                                int q) {
#pragma unroll
  for (int i = 0; i < 4; ++i) stage[(4 * i + lr) * kStageStride + lc] = x[i];
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = stage[r * kStageStride + 4 * q + i];
  __builtin_amdgcn_wave_barrier();   // reads done before the next group's writes
}

// The 16 token rows of a half group are contiguous in the source, so each
// load covers one contiguous KiB of them (load i, lane l: row 4i + l/16,
// channels 8 (l % 16) .. + 7); the wave's staging tile in LDS hands each lane
// its value group (row r, channels 32q .. 32q + 31).
template <int BITS, int META>
__device__ __forceinline__ void quantize_values(const QuantizeArgs &a, int u, int gl0, int gl1,
                                                int part, int lane, uint8_t *tile, uint4 *stage) {
  constexpr int D = kHeadDim, G = kGroup;
  const int r = lane >> 2, q = lane & 3;
  const int lr = lane >> 4, lc = lane & 15;
  const uint16_t *src = a.src_v + (long long)u * a.src_unit_stride + (long long)a.src_tok0 * D;
  auto load = [&](int gl, uint4 (&x)[4]) {
    const uint4 *base =
        reinterpret_cast<const uint4 *>(src + ((long long)gl * G + 16 * part + lr) * D) + lc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // row 4i + lr
      const u32x4_nt t =
          __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(base + i * (4 * D / 8)));
      x[i] = make_uint4(t.x, t.y, t.z, t.w);
    }
  };
  uint4 cur[4], nxt[4];
  load(gl0, nxt);
  for (int gl = gl0; gl + 1 < gl1; ++gl) {
#pragma unroll
    for (int i = 0; i < 4; ++i) cur[i] = nxt[i];
    load(gl + 1, nxt);
    regather_values(cur, stage, lr, lc, r, q);
    value_group<BITS, META>(a, u, gl, cur, part, lane, tile);
  }
  regather_values(nxt, stage, lr, lc, r, q);
  value_group<BITS, META>(a, u, gl1 - 1, nxt, part, lane, tile);
}

// One 16-byte piece of the row copy: piece `idx` of unit u, the K rows'
// pieces first, then the V rows'.
__device__ __forceinline__ void copy_row_piece(const CopyRowsArgs &a, int idx, int u) {
  constexpr int CH = kHeadDim / 8;   // 16-byte pieces per row
  const int per = a.n_rows * CH;
  if (idx >= 2 * per) return;
  const bool is_v = idx >= per;
  const int i = (idx - (is_v ? per : 0)) / CH, c = idx % CH;
  const uint16_t *src = is_v ? a.src_v : a.src_k;
  uint16_t *dst = is_v ? a.dst_v : a.dst_k;
  const uint4 v = *reinterpret_cast<const uint4 *>(
      src + (long long)u * a.src_unit_stride + (long long)(a.src_tok0 + i) * kHeadDim + 8 * c);
  *reinterpret_cast<uint4 *>(dst + (long long)u * a.dst_unit_stride +
                             (long long)(a.dst_row0 + i) * kHeadDim + 8 * c) = v;
}

// Grid (ceil(n_groups / gpw) + residual blocks, n_units): waves 0-1 take the keys (channel
// halves), waves 2-3 the values (token halves) of `gpw` consecutive groups
// (one by default).  The waves share nothing and never wait for each other.
template <int BITS, int META>
__global__ __launch_bounds__(256) void quantize_kernel(QuantizeArgs a) {
  __shared__ __align__(16) uint8_t s_tile[4][16 * kHeadDim];
  __shared__ uint4 s_stage[2][16 * kStageStride];   // value waves' bf16 staging
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int u = blockIdx.y;
  const int n_gblocks = (a.n_groups + a.gpw - 1) / a.gpw;
  if ((int)blockIdx.x >= n_gblocks) {
    // a prefill's residual rows, beside its groups: one piece per thread
    copy_row_piece(a.res, ((int)blockIdx.x - n_gblocks) * 256 + (int)threadIdx.x, u);
    return;
  }
  const int gl0 = blockIdx.x * a.gpw;
  int gl1 = min(gl0 + a.gpw, a.n_groups);
  if (a.seq_lens) {
    // mixed-length prefill: this sequence's own quantised groups
    int n_q, r;
    if (!seq_split(a.seq_lens[u / a.kv_heads], a.stride, kGroup, a.residual, a.max_tokens, n_q, r))
      return;
    gl1 = min(gl1, n_q / kGroup);
    if (gl0 >= gl1) return;
  } else if (a.state) {
    // mixed-length flush: only sequences whose ring fills with this step's
    // append, and that have room for one more group
    const int4 st = reinterpret_cast<const int4 *>(a.state)[u / a.kv_heads];
    if (!state_ok(st.x, st.y, st.z, st.w, kGroup, a.slots, a.max_tokens) || st.w != 0 ||
        st.y + 1 != a.slots || st.x + kGroup > a.max_tokens)
      return;
    a.dst_g0 = st.x / kGroup;
    a.src_tok0 = st.z;   // a multiple of G: the G oldest ring tokens are contiguous
  }
  if (wave < 2)
    quantize_keys<BITS, META>(a, u, gl0, gl1, wave, lane, s_tile[wave]);
  else
    quantize_values<BITS, META>(a, u, gl0, gl1, wave - 2, lane, s_tile[wave], s_stage[wave - 2]);
}

__global__ __launch_bounds__(256) void copy_rows_kernel(CopyRowsArgs a) {
  copy_row_piece(a, blockIdx.x * blockDim.x + threadIdx.x, blockIdx.y);
}

__global__ __launch_bounds__(256) void ragged_residual_kernel(RaggedResidualArgs a) {
  constexpr int CH = kHeadDim / 8;   // 16-byte chunks per row
  const int u = blockIdx.y, b = u / a.kv_heads;
  int n_q, r;
  bool ok = seq_split(a.seq_lens[b], a.stride, a.group, a.residual, a.max_tokens, n_q, r);
  if (blockIdx.x == 0 && blockIdx.z == 0 && u % a.kv_heads == 0) {
    // the state block: with pages, every history group needs its page
    // (the quantiser skips groups without one)
    bool missing = false;
    if (ok && a.pages.table) {
      const int n_pages = ((n_q / a.group) + (1 << a.pages.shift) - 1) >> a.pages.shift;
      for (int i = threadIdx.x; i < n_pages; i += blockDim.x)
        missing |= group_slot(a.pages, a.kv_heads, 0, u, i << a.pages.shift) < 0;
    }
    ok = ok && !__syncthreads_or(missing);
    if (threadIdx.x == 0)
      reinterpret_cast<int4 *>(a.state)[b] = ok ? make_int4(n_q, r, 0, 0)
                                               : make_int4(0, 0, 0, kSeqBadLength);
  }
  if (!ok) return;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= r * CH) return;
  const int i = idx / CH, c = idx % CH;
  const uint16_t *src = blockIdx.z == 0 ? a.src_k : a.src_v;
  uint16_t *dst = blockIdx.z == 0 ? a.dst_k : a.dst_v;
  const uint4 v = *reinterpret_cast<const uint4 *>(
      src + ((long long)u * a.stride + n_q + i) * kHeadDim + 8 * c);
  *reinterpret_cast<uint4 *>(dst + ((long long)u * a.slots + i) * kHeadDim + 8 * c) = v;
}

}  // namespace

hipError_t launch_ragged_residual(const RaggedResidualArgs &a, hipStream_t s) {
  if (a.n_units <= 0) return hipSuccess;
  const int chunks = a.slots * (kHeadDim / 8);
  const dim3 grid((chunks + 255) / 256, a.n_units, 2);
  hipLaunchKernelGGL(ragged_residual_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize(int bits, int meta, const QuantizeArgs &a_in, hipStream_t s) {
  if (a_in.n_groups <= 0 || a_in.n_units <= 0) return hipSuccess;
  // groups per workgroup: one.  Short independent workgroups keep the most
  // loads in flight; on MI355X at the 8K GQA prefill (16 x 8 units, 252
  // groups each) 1 group per workgroup runs at 5.4 TB/s, 2 at 5.2, 4 at 4.8,
  // 8 at 4.5.  KIVI_QGPW sets another count (sweeps; read once per process).
  QuantizeArgs a = a_in;
  static const long long gpw = [] {
    const char *env = getenv("KIVI_QGPW");
    return env ? atoll(env) : 1ll;
  }();
  a.gpw = (int)(gpw < 1 ? 1 : gpw > 8 ? 8 : gpw);
  // workgroups of the residual copy: 2 * n_rows rows of 16 pieces, 256 a block
  const int res_blocks = a.res.n_rows > 0 ? (2 * a.res.n_rows * (kHeadDim / 8) + 255) / 256 : 0;
  const dim3 grid((a.n_groups + a.gpw - 1) / a.gpw + res_blocks, a.n_units), block(256);
  if (bits == 2 && meta == 0)
    hipLaunchKernelGGL((quantize_kernel<2, 0>), grid, block, 0, s, a);
  else if (bits == 2)
    hipLaunchKernelGGL((quantize_kernel<2, 1>), grid, block, 0, s, a);
  else if (meta == 0)
    hipLaunchKernelGGL((quantize_kernel<4, 0>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((quantize_kernel<4, 1>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const CopyRowsArgs &a, hipStream_t s) {
  if (a.n_rows <= 0 || a.n_units <= 0) return hipSuccess;
  const int pieces = 2 * a.n_rows * (kHeadDim / 8);   // K rows, then V rows
  const dim3 grid((pieces + 255) / 256, a.n_units);
  hipLaunchKernelGGL(copy_rows_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kivi
