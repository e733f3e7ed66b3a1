// quantize_group.h -- the per-wave group quantiser, shared by the
// quantise kernels (prefill, flush) and the decode kernel (a flush folded
// into a decode launch).
//
// Method ("KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache",
// method paragraph; catalog record kivi-2bit-llama3-8b-gqa-8k, Methodology):
// keys are grouped along the token axis of each channel (per-channel), values
// along 32 channels of each token (per-token), G = 32, asymmetric min-max
// scale/zero, 2- or 4-bit codes.  Every float operation of the quantiser is a
// single IEEE fp32 operation, rounded to nearest even, nothing fused (the
// rounding-explicit intrinsics below):
//     s = (max - min) / L ;  inv = s >= FLT_MIN ? 1 / s : 0 ;
//     code = clamp(rint((x - min) * inv), 0, L) ;  scale = s, zero = min.
// With the 16-bit scale/zero format the scale is first rounded to fp16 and
// the codes use the rounded value; the zero is stored as bf16 (exact).
//
// quantize_keys quantises one channel half of the keys of its groups and
// quantize_values one token half of the values, one wave each, with wave
// barriers only: four waves (or one wave four times) cover a group.
#pragma once

#include <float.h>

#include "kivi_internal.h"

namespace kivi {
namespace qgroup {

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
#pragma clang fp contract(off)
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
#pragma clang fp contract(off)
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

}  // namespace qgroup
}  // namespace kivi
