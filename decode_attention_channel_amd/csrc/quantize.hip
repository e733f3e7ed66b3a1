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
//
// One workgroup of 256 threads quantises one group of one unit; blockIdx.z
// selects K (0) or V (1).
//  K: thread (wave w, lane) owns channels 2*lane, 2*lane+1 of rows 8w..8w+7:
//     min/max in registers, across the 4 waves through LDS.
//  V: thread (row r, chunk q) owns channels 16q..16q+15 of row r; the 32
//     channels of a value group sit in two adjacent lanes.
// Codes are staged as bytes in LDS ([token][channel]) and re-read in the
// order of the packed layout, so every global store is a coalesced dword.
#pragma clang fp contract(off)

#include <float.h>

#include "kivi_internal.h"

namespace kivi {
namespace {

template <int BITS>
struct Q {
  static constexpr float kLevels = (float)((1 << BITS) - 1);
};

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

template <int BITS>
__device__ __forceinline__ void group_params(float mn, float mx, float &s, float &inv) {
  s = __fdiv_rn(__fsub_rn(mx, mn), Q<BITS>::kLevels);
  inv = (s >= FLT_MIN) ? __fdiv_rn(1.0f, s) : 0.0f;
}

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

template <int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(QuantizeArgs a) {
  constexpr int D = kHeadDim, G = kGroup;
  __shared__ __align__(16) uint8_t s_code[G][D];
  __shared__ float s_mn[4][D], s_mx[4][D];

  const int gl = blockIdx.x, u = blockIdx.y, t = threadIdx.x;
  const int g = a.dst_g0 + gl;
  const long long unit_grp = (long long)u * a.n_groups_cap + g;

  if (blockIdx.z == 0) {
    // ------------------------------------------------------------- keys
    const int lane = t & 63, w = t >> 6;
    const uint32_t *src = reinterpret_cast<const uint32_t *>(
        a.src_k + (long long)u * a.src_unit_stride + (long long)(a.src_tok0 + gl * G) * D);
    float x0[8], x1[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t x = src[(8 * w + r) * (D / 2) + lane];
      x0[r] = bf16_lo(x);
      x1[r] = bf16_hi(x);
    }
    float mn0 = x0[0], mx0 = x0[0], mn1 = x1[0], mx1 = x1[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) {
      mn0 = fminf(mn0, x0[r]); mx0 = fmaxf(mx0, x0[r]);
      mn1 = fminf(mn1, x1[r]); mx1 = fmaxf(mx1, x1[r]);
    }
    s_mn[w][2 * lane] = mn0; s_mn[w][2 * lane + 1] = mn1;
    s_mx[w][2 * lane] = mx0; s_mx[w][2 * lane + 1] = mx1;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mn0 = fminf(mn0, s_mn[i][2 * lane]); mn1 = fminf(mn1, s_mn[i][2 * lane + 1]);
      mx0 = fmaxf(mx0, s_mx[i][2 * lane]); mx1 = fmaxf(mx1, s_mx[i][2 * lane + 1]);
    }
    float sc0, inv0, sc1, inv1;
    group_params<BITS>(mn0, mx0, sc0, inv0);
    group_params<BITS>(mn1, mx1, sc1, inv1);
    if (w == 0) {
      reinterpret_cast<float2 *>(a.k_scale + unit_grp * D)[lane] = make_float2(sc0, sc1);
      reinterpret_cast<float2 *>(a.k_zero + unit_grp * D)[lane] = make_float2(mn0, mn1);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t c = code_of<BITS>(x0[r], mn0, inv0) | (code_of<BITS>(x1[r], mn1, inv1) << 8);
      reinterpret_cast<uint16_t *>(s_code[8 * w + r])[lane] = (uint16_t)c;
    }
    __syncthreads();
    // pack: thread -> (row, 16 consecutive channels)
    const int row = t >> 3, ch0 = 16 * (t & 7);
    const uint4 x = *reinterpret_cast<const uint4 *>(&s_code[row][ch0]);
    uint8_t *dst = a.k_codes + ((long long)u * a.max_tokens + (long long)g * G + row) * (D * BITS / 8);
    if (BITS == 2) {
      const uint32_t word = pack4x2(x.x) | (pack4x2(x.y) << 8) | (pack4x2(x.z) << 16) |
                            (pack4x2(x.w) << 24);
      reinterpret_cast<uint32_t *>(dst)[t & 7] = word;
    } else {
      const uint2 word = make_uint2(pack4x4(x.x) | (pack4x4(x.y) << 16),
                                    pack4x4(x.z) | (pack4x4(x.w) << 16));
      reinterpret_cast<uint2 *>(dst)[t & 7] = word;
    }
  } else {
    // ----------------------------------------------------------- values
    const int row = t >> 3, q = t & 7, j = q >> 1;
    const uint4 *src = reinterpret_cast<const uint4 *>(
        a.src_v + (long long)u * a.src_unit_stride + (long long)(a.src_tok0 + gl * G + row) * D +
        16 * q);
    const uint4 p0 = src[0], p1 = src[1];
    const uint32_t wv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float x[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = bf16_lo(wv[i]);
      x[2 * i + 1] = bf16_hi(wv[i]);
    }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
    mn = fminf(mn, __shfl_xor(mn, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    float sc, inv;
    group_params<BITS>(mn, mx, sc, inv);
    if ((q & 1) == 0) {
      const long long mi = (unit_grp * (D / G) + j) * G + row;
      a.v_scale[mi] = sc;
      a.v_zero[mi] = mn;
    }
    uint32_t cw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      cw[i] = code_of<BITS>(x[4 * i], mn, inv) | (code_of<BITS>(x[4 * i + 1], mn, inv) << 8) |
              (code_of<BITS>(x[4 * i + 2], mn, inv) << 16) |
              (code_of<BITS>(x[4 * i + 3], mn, inv) << 24);
    *reinterpret_cast<uint4 *>(&s_code[row][16 * q]) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    __syncthreads();
    // pack: thread -> (octet o, channels 2cp, 2cp+1): two cells of 8 tokens
    const int o = t >> 6, cp = t & 63;
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t pair = reinterpret_cast<const uint16_t *>(s_code[8 * o + k])[cp];
      c0 |= (pair & 0xFFu) << (BITS * k);
      c1 |= (pair >> 8) << (BITS * k);
    }
    const long long cell = ((unit_grp * (G / 8) + o) * D) / 2 + cp;   // in channel pairs
    if (BITS == 2) {
      reinterpret_cast<uint32_t *>(a.v_codes)[cell] = c0 | (c1 << 16);
    } else {
      reinterpret_cast<uint2 *>(a.v_codes)[cell] = make_uint2(c0, c1);
    }
  }
}

__global__ __launch_bounds__(256) void copy_rows_kernel(CopyRowsArgs a) {
  constexpr int CH = kHeadDim / 8;   // 16-byte chunks per row
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.n_rows * CH) return;
  const int i = idx / CH, c = idx % CH, u = blockIdx.y;
  const uint16_t *src = blockIdx.z == 0 ? a.src_k : a.src_v;
  uint16_t *dst = blockIdx.z == 0 ? a.dst_k : a.dst_v;
  const uint4 v = *reinterpret_cast<const uint4 *>(
      src + (long long)u * a.src_unit_stride + (long long)(a.src_tok0 + i) * kHeadDim + 8 * c);
  *reinterpret_cast<uint4 *>(dst + (long long)u * a.dst_unit_stride +
                             (long long)(a.dst_row0 + i) * kHeadDim + 8 * c) = v;
}

}  // namespace

hipError_t launch_quantize(int bits, const QuantizeArgs &a, hipStream_t s) {
  if (a.n_groups <= 0 || a.n_units <= 0) return hipSuccess;
  const dim3 grid(a.n_groups, a.n_units, 2);
  if (bits == 2)
    hipLaunchKernelGGL(quantize_kernel<2>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(quantize_kernel<4>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const CopyRowsArgs &a, hipStream_t s) {
  if (a.n_rows <= 0 || a.n_units <= 0) return hipSuccess;
  const int chunks = a.n_rows * (kHeadDim / 8);
  const dim3 grid((chunks + 255) / 256, a.n_units, 2);
  hipLaunchKernelGGL(copy_rows_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kivi
