// decode_attn.hip -- decode-step attention over the KIVI mixed cache.
//
// For every query head: score_t = sigma * q . k_t over the dequantised
// history (per-channel K groups, per-token V groups; "KIVI: A Tuning-Free
// Asymmetric 2bit Quantization for KV Cache", method paragraph) and the bf16
// residual (catalog record kivi-2bit-llama3-8b-gqa-8k, KV bytes basis);
// p = softmax(score); out = sum_t p_t v_t, fp32 accumulation.
//
// Split-K flash decoding.  Grid (split, unit): splits 0..n_split_q-1 take
// `gps` consecutive groups of 32 quantised tokens each (4 waves, one group per
// wave at a time, each wave with its own online-softmax state, merged in LDS
// at the end); split n_split_q takes the bf16 residual.  Each split writes
// (m, l, o[128]) per query head; combine_kernel merges the splits.
//
// Dequantisation is folded into the products, which is algebraically the
// same as dequantise-then-dot:
//   q . k_t = sum_c (q_c s^K_c) code_tc + sum_c q_c z^K_c          (per group)
//   sum_t p_t v_tc = sum_t (p_t s^V_t,j) code_tc + sum_t p_t z^V_t,j
// so the codes enter the arithmetic as exact small integers.  They are
// unpacked with the gfx950 microscaling converts: a 2-bit code placed in an
// FP4 (e2m1) nibble is exactly code/2, a 4-bit code in an FP8 (e4m3) byte is
// exactly code * 2^-9; the convert's power-of-two scale (2, 512) restores the
// integer exactly.
//
// GQA (q_per_kv >= 2): q.K^T and P.V run on v_mfma_f32_16x16x32_bf16 with the
// codes as the A operand (16 tokens x 32 channels for q.K^T, 16 channels x 32
// tokens for P.V) and the scaled queries / probabilities as the B operand.
// The B operand is split into bf16 hi + lo parts (relative error ~2^-16), the
// parts occupying different MFMA columns (q.K^T) or two MFMAs (P.V), so the
// result carries close to fp32 precision.  MHA (q_per_kv == 1) stays on VALU
// with fp32 FMAs: one query row is not a dense contraction.
#include <float.h>
#include <math.h>

#include "kivi_internal.h"

namespace kivi {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

union Op8 {
  bf16x8_t v;
  uint32_t u[4];
};

constexpr int D = kHeadDim;
constexpr int G = kGroup;
constexpr float kNegInf = -INFINITY;
constexpr float kRescaleSlack = 8.0f;   // running max may lag the true max by 8 (log2)

// MFMA slot s of an 8-slot operand group <-> element P8[s] of a block of 8
// consecutive channels (q.K^T) or tokens (P.V): the order in which the
// converts below deliver codes.
constexpr int P8[8] = {0, 2, 1, 3, 4, 6, 5, 7};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 2.0f, SEL));
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, HI));
}
template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 2.0f, SEL);
}
template <bool HI>
__device__ __forceinline__ f32x2_t fp8x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 512.0f, HI);
}

// 16 two-bit codes of one word -> two 8-slot bf16 operands (codes 0..7 and
// 8..15), each in P8 order.
__device__ __forceinline__ void unpack2(uint32_t w, Op8 &lo8, Op8 &hi8) {
  const uint32_t a = w & 0x33333333u, b = (w >> 2) & 0x33333333u;
  lo8.u[0] = fp4x2_to_bf16x2<0>(a);
  lo8.u[1] = fp4x2_to_bf16x2<0>(b);
  lo8.u[2] = fp4x2_to_bf16x2<1>(a);
  lo8.u[3] = fp4x2_to_bf16x2<1>(b);
  hi8.u[0] = fp4x2_to_bf16x2<2>(a);
  hi8.u[1] = fp4x2_to_bf16x2<2>(b);
  hi8.u[2] = fp4x2_to_bf16x2<3>(a);
  hi8.u[3] = fp4x2_to_bf16x2<3>(b);
}
// 8 four-bit codes of one word -> one 8-slot bf16 operand in P8 order.
__device__ __forceinline__ void unpack4(uint32_t w, Op8 &o) {
  const uint32_t a = w & 0x0F0F0F0Fu, b = (w >> 4) & 0x0F0F0F0Fu;
  o.u[0] = fp8x2_to_bf16x2<false>(a);
  o.u[1] = fp8x2_to_bf16x2<false>(b);
  o.u[2] = fp8x2_to_bf16x2<true>(a);
  o.u[3] = fp8x2_to_bf16x2<true>(b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): two packed words for a pair
__device__ __forceinline__ void split_bf16(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(x0, x1);
  const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xFFFF0000u);
  lo = pack_bf16x2(x0 - h0, x1 - h1);
}

__device__ __forceinline__ float dpp_ror4(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124,
                                                             0xF, 0xF, false));
}
__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m)); }
__device__ __forceinline__ float xor_sum(float x, int m) { return x + __shfl_xor(x, m); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void ld8(const float *p, float (&x)[8]) {
  const float4 a = ld4(p), b = ld4(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void ld16(const float *p, float (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = ld4(p + 4 * i);
    x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
  }
}

// ---------------------------------------------------------------- merge ---
// Each wave contributes (m, l, o[128]) per head; the workgroup writes one
// partial per head: M = max m_w, l = sum 2^(m_w - M) l_w, o likewise.
template <int HMAX>
struct MergeSmem {
  float m[4][HMAX];
  float l[4][HMAX];
  float o[4][HMAX][D];
};

template <int HMAX>
__device__ void merge_and_store(MergeSmem<HMAX> &sm, const DecodeArgs &a, int u, int split) {
  __syncthreads();
  const int qpk = a.qpk;
  float *part = a.part + ((long long)u * a.n_split + split) * qpk * kPartStride;
  for (int idx = threadIdx.x; idx < qpk * D; idx += blockDim.x) {
    const int hh = idx / D, c = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm.m[w][hh]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = sm.m[w][hh] == kNegInf ? 0.f : fast_exp2(sm.m[w][hh] - M);
      l += f * sm.l[w][hh];
      o += f * sm.o[w][hh][c];
    }
    part[hh * kPartStride + 4 + c] = o;
    if (c == 0) {
      part[hh * kPartStride + 0] = M;
      part[hh * kPartStride + 1] = l;
    }
  }
}

// ------------------------------------------------------- residual split ---
// The bf16 residual of one unit: one token per thread for q.k, then one
// (head, channel pair) per thread for P.V, 256 tokens at a time.
template <int HMAX>
struct ResidSmem {
  float q[HMAX][D];
  float s[HMAX][256];
  float mx[HMAX];
};

template <int HMAX>
__device__ void residual_split(ResidSmem<HMAX> &sm, const DecodeArgs &a, int u, int split) {
  const int tid = threadIdx.x, qpk = a.qpk;
  const int b = u / a.kv_heads, h = u % a.kv_heads;
  const uint16_t *qrow = a.q + ((long long)b * a.kv_heads * qpk + (long long)h * qpk) * D;
  for (int i = tid; i < qpk * D; i += 256) sm.q[i / D][i % D] = bf16_bits_to_f32(qrow[i]) * a.qscale;

  constexpr int ITEMS = (HMAX * (D / 2) + 255) / 256;
  float m_h[HMAX], oacc[ITEMS][2], lacc[ITEMS];
#pragma unroll
  for (int hh = 0; hh < HMAX; ++hh) m_h[hh] = kNegInf;
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) { oacc[it][0] = oacc[it][1] = 0.f; lacc[it] = 0.f; }

  const long long ring = (long long)u * a.slots;
  for (int t0 = 0; t0 < a.n_res; t0 += 256) {
    const int cn = min(256, a.n_res - t0);
    __syncthreads();   // q staged / previous chunk consumed
    if (tid < cn) {
      const int slot = (a.res_start + t0 + tid) % a.slots;
      const uint4 *krow = reinterpret_cast<const uint4 *>(a.k_res + (ring + slot) * D);
      float s[HMAX];
#pragma unroll
      for (int hh = 0; hh < HMAX; ++hh) s[hh] = 0.f;
      for (int c8 = 0; c8 < D / 8; ++c8) {
        const uint4 kv = krow[c8];
        const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
        float kf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[2 * e] = __uint_as_float(w[e] << 16);
          kf[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
#pragma unroll
        for (int hh = 0; hh < HMAX; ++hh) {
          if (hh < qpk) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s[hh] += sm.q[hh][8 * c8 + e] * kf[e];
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < HMAX; ++hh)
        if (hh < qpk) sm.s[hh][tid] = s[hh];
    }
    __syncthreads();
    // chunk max per head: wave w reduces heads w, w+4, ...
    {
      const int w = tid >> 6, lane = tid & 63;
      for (int hh = w; hh < qpk; hh += 4) {
        float mx = kNegInf;
        for (int i = lane; i < cn; i += 64) mx = fmaxf(mx, sm.s[hh][i]);
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1) mx = xor_max(mx, msk);
        if (lane == 0) sm.mx[hh] = mx;
      }
    }
    __syncthreads();
    float alpha[HMAX];
#pragma unroll
    for (int hh = 0; hh < HMAX; ++hh) {
      if (hh < qpk) {
        const float mnew = fmaxf(m_h[hh], sm.mx[hh]);
        alpha[hh] = m_h[hh] == kNegInf ? 0.f : fast_exp2(m_h[hh] - mnew);
        m_h[hh] = mnew;
      } else {
        alpha[hh] = 0.f;
      }
    }
    for (int i = tid; i < qpk * cn; i += 256) {
      const int hh = i / cn, tt = i % cn;
      sm.s[hh][tt] = fast_exp2(sm.s[hh][tt] - m_h[hh]);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int item = tid + 256 * it;
      if (item < qpk * (D / 2)) {
        const int hh = item / (D / 2), cp = item % (D / 2);
        float al = 0.f;
#pragma unroll
        for (int x = 0; x < HMAX; ++x)
          if (x == hh) al = alpha[x];
        float o0 = oacc[it][0] * al, o1 = oacc[it][1] * al, l = lacc[it] * al;
        for (int tt = 0; tt < cn; ++tt) {
          const int slot = (a.res_start + t0 + tt) % a.slots;
          const uint32_t vv = reinterpret_cast<const uint32_t *>(a.v_res + (ring + slot) * D)[cp];
          const float p = sm.s[hh][tt];
          o0 += p * __uint_as_float(vv << 16);
          o1 += p * __uint_as_float(vv & 0xFFFF0000u);
          l += p;
        }
        oacc[it][0] = o0; oacc[it][1] = o1; lacc[it] = l;
      }
    }
  }
  float *part = a.part + ((long long)u * a.n_split + split) * qpk * kPartStride;
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int item = tid + 256 * it;
    if (item < qpk * (D / 2)) {
      const int hh = item / (D / 2), cp = item % (D / 2);
      float mh = kNegInf;
#pragma unroll
      for (int x = 0; x < HMAX; ++x)
        if (x == hh) mh = m_h[x];
      reinterpret_cast<float2 *>(part + hh * kPartStride + 4)[cp] =
          make_float2(oacc[it][0], oacc[it][1]);
      if (cp == 0) {
        part[hh * kPartStride + 0] = mh;
        part[hh * kPartStride + 1] = lacc[it];
      }
    }
  }
}

// ------------------------------------------------------ MFMA (GQA) path ---
template <int NHB>
struct MfmaSmem {
  uint4 bq[4][NHB][2][4][4][4];   // [wave][head block][hi/lo][head][step][lane group]
};

template <int BITS, int NHB>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int HMAX = 4 * NHB;
  constexpr int KROW = D * BITS / 8;     // bytes per token row of K codes
  constexpr int CB = 32 * BITS / 8;      // bytes of 32 channels
  __shared__ __align__(16) union {
    MfmaSmem<NHB> mf;
    MergeSmem<HMAX> mg;
    ResidSmem<HMAX> rs;
  } sm;

  const int split = blockIdx.x, u = blockIdx.y;
  if (split >= a.n_split_q) {
    residual_split<HMAX>(sm.rs, a, u, split);
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, gq = lane >> 4;          // MFMA column / row, lane group
  const int ch = lane & 3, cm = (lane >> 2) & 3;    // cooperative q' role: head, step
  const int qpk = a.qpk;
  const int b = u / a.kv_heads, h = u % a.kv_heads;

  // scaled query values in slot order for the cooperative role
  float qv[NHB][8];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int hh = hb * 4 + ch;
    if (hh < qpk) {
      const uint4 raw = *reinterpret_cast<const uint4 *>(
          a.q + ((long long)b * a.kv_heads * qpk + (long long)h * qpk + hh) * D + 32 * gq + 8 * cm);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) qv[hb][s] = x[P8[s]] * a.qscale;
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) qv[hb][s] = 0.f;
    }
  }

  f32x4_t acc[NHB][8];
  float m_run[NHB], l_run[NHB], z_run[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[hb][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[hb] = kNegInf; l_run[hb] = 0.f; z_run[hb] = 0.f;
  }

  const int g_begin = split * a.gps;
  const int g_end = min(g_begin + a.gps, a.n_groups);
  const int kr0 = 8 * (n >> 2) + (n & 3);   // A-operand row n of tile 0 -> token; tile 1: +4
  const int jv = n >> 2;                      // V channel group of this column (P.V)
  const int hv = n & 3;                       // head (within block) of this column

  for (int g = g_begin + wave; g < g_end; g += 4) {
    const long long ug = (long long)u * a.n_groups_cap + g;
    // ---- loads
    const uint8_t *kb = a.k_codes + ((long long)u * a.max_tokens + (long long)g * G) * KROW + gq * CB;
    const uint8_t *vb = a.v_codes + ((ug * (G / 8) + gq) * D + 8 * n) * BITS;
    uint32_t kw[2][BITS];   // per tile: BITS words = 32 channels
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const uint8_t *p = kb + (kr0 + 4 * tile) * KROW;
      if constexpr (BITS == 2) {
        const uint2 x = *reinterpret_cast<const uint2 *>(p);
        kw[tile][0] = x.x; kw[tile][1] = x.y;
      } else {
        const uint4 x = *reinterpret_cast<const uint4 *>(p);
        kw[tile][0] = x.x; kw[tile][1] = x.y; kw[tile][2] = x.z; kw[tile][3] = x.w;
      }
    }
    uint32_t vw[2 * BITS];   // 8 channels x 8 tokens
    {
      const uint4 x = *reinterpret_cast<const uint4 *>(vb);
      vw[0] = x.x; vw[1] = x.y; vw[2] = x.z; vw[3] = x.w;
      if constexpr (BITS == 4) {
        const uint4 y = *reinterpret_cast<const uint4 *>(vb + 16);
        vw[4] = y.x; vw[5] = y.y; vw[6] = y.z; vw[7] = y.w;
      }
    }
    float sk[8], zk[8], sv[8], zv[8];
    ld8(a.k_scale + ug * D + 32 * gq + 8 * cm, sk);
    ld8(a.k_zero + ug * D + 32 * gq + 8 * cm, zk);
    ld8(a.v_scale + (ug * (D / G) + jv) * G + 8 * gq, sv);
    ld8(a.v_zero + (ug * (D / G) + jv) * G + 8 * gq, zv);

    // ---- A operands (exact codes)
    Op8 ak[2][4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      if constexpr (BITS == 2) {
        unpack2(kw[tile][0], ak[tile][0], ak[tile][1]);
        unpack2(kw[tile][1], ak[tile][2], ak[tile][3]);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) unpack4(kw[tile][m], ak[tile][m]);
      }
    }
    Op8 av[8];
    if constexpr (BITS == 2) {
#pragma unroll
      for (int d = 0; d < 4; ++d) unpack2(vw[d], av[2 * d], av[2 * d + 1]);
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) unpack4(vw[mt], av[mt]);
    }

#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      // ---- cooperative q' = q * s^K (hi/lo) and beta = q . z^K
      float beta = 0.f;
      {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int s = 0; s < 8; s += 2) {
          split_bf16(qv[hb][s] * sk[P8[s]], qv[hb][s + 1] * sk[P8[s + 1]], hi[s / 2], lo[s / 2]);
          beta += qv[hb][s] * zk[P8[s]];
          beta += qv[hb][s + 1] * zk[P8[s + 1]];
        }
        sm.mf.bq[wave][hb][0][ch][cm][gq] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        sm.mf.bq[wave][hb][1][ch][cm][gq] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
      beta = xor_sum(beta, 4);
      beta = xor_sum(beta, 8);
      beta = xor_sum(beta, 16);
      beta = xor_sum(beta, 32);   // every lane with (lane & 3) == head holds beta[head]
      __builtin_amdgcn_wave_barrier();

      // ---- scores: columns n = 4x + head, x in {hi, lo, hi, lo}
      f32x4_t sc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        Op8 bq;
        const uint4 x = sm.mf.bq[wave][hb][(n >> 2) & 1][n & 3][m][gq];
        bq.u[0] = x.x; bq.u[1] = x.y; bq.u[2] = x.z; bq.u[3] = x.w;
#pragma unroll
        for (int tile = 0; tile < 2; ++tile)
          sc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[tile][m].v, bq.v, sc[tile], 0, 0, 0);
      }
      // token 8gq + 4*tile + r  <->  p index 4*tile + r
      float s8[8];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
#pragma unroll
        for (int r = 0; r < 4; ++r) s8[4 * tile + r] = sc[tile][r] + dpp_ror4(sc[tile][r]) + beta;

      // ---- online softmax (log2 domain), lazily rescaled
      float mx = s8[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) mx = fmaxf(mx, s8[k]);
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32);
      const bool need = mx > m_run[hb] + kRescaleSlack;
      if (__any(need)) {
        const float mnew = need ? mx : m_run[hb];
        const float al = m_run[hb] == kNegInf ? 0.f : fast_exp2(m_run[hb] - mnew);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) acc[hb][mt] *= al;
        l_run[hb] *= al;
        z_run[hb] *= al;
        m_run[hb] = mnew;
      }
      float p[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        p[k] = fast_exp2(s8[k] - m_run[hb]);
        l_run[hb] += p[k];
        z_run[hb] += p[k] * zv[k];
      }
      // ---- P.V: columns n = 4j + head; B slot s <-> token 8gq + P8[s]
      Op8 bh, bl;
#pragma unroll
      for (int s = 0; s < 8; s += 2)
        split_bf16(p[P8[s]] * sv[P8[s]], p[P8[s + 1]] * sv[P8[s + 1]], bh.u[s / 2], bl.u[s / 2]);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        acc[hb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt].v, bh.v, acc[hb][mt], 0, 0, 0);
        acc[hb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt].v, bl.v, acc[hb][mt], 0, 0, 0);
      }
    }
  }

  // ---- per-wave totals, then the workgroup merge (the merge buffer aliases
  // the q' staging of the other waves: wait until every wave left the loop)
  __syncthreads();
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    float l = xor_sum(xor_sum(l_run[hb], 16), 32);
    float z = xor_sum(xor_sum(z_run[hb], 16), 32);
    // lane (n, gq) holds rows 4gq + r of M-tile mt = channel 32gq + 8r + mt,
    // for column n = 4j + head; the column is useful when j == gq.
    if (jv == gq) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float o8[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) o8[mt] = acc[hb][mt][r] + z;
        float *dst = &sm.mg.o[wave][hb * 4 + hv][32 * gq + 8 * r];
        *reinterpret_cast<float4 *>(dst) = make_float4(o8[0], o8[1], o8[2], o8[3]);
        *reinterpret_cast<float4 *>(dst + 4) = make_float4(o8[4], o8[5], o8[6], o8[7]);
      }
    }
    if (gq == 0 && n < 4) {
      sm.mg.m[wave][hb * 4 + n] = m_run[hb];
      sm.mg.l[wave][hb * 4 + n] = l;
    }
  }
  merge_and_store<HMAX>(sm.mg, a, u, split);
}

// ------------------------------------------------------- VALU (MHA) path ---
struct ValuSmem {
  float p[4][32];
};

template <int BITS>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  constexpr int KROW = D * BITS / 8;
  __shared__ __align__(16) union {
    ValuSmem vs;
    MergeSmem<1> mg;
    ResidSmem<1> rs;
  } sm;
  // `mg` and `vs` are live at different times except p[] during the loop;
  // the merge starts with a barrier after the loop.

  const int split = blockIdx.x, u = blockIdx.y;
  if (split >= a.n_split_q) {
    residual_split<1>(sm.rs, a, u, split);
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tb = lane >> 3, cb = lane & 7;    // q.k role: tokens 4tb.., channels 16cb..
  const int oc = lane >> 4, cq = lane & 15;   // P.V role: octet, channels 8cq..
  const int b = u / a.kv_heads, h = u % a.kv_heads;

  float qv[16];
  {
    const uint4 *qp = reinterpret_cast<const uint4 *>(
        a.q + ((long long)b * a.kv_heads + h) * D + 16 * cb);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 raw = qp[i];
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[8 * i + 2 * e] = __uint_as_float(w[e] << 16) * a.qscale;
        qv[8 * i + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u) * a.qscale;
      }
    }
  }
  float oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = 0.f;
  float m_run = kNegInf, l_run = 0.f, z_run = 0.f;

  const int g_begin = split * a.gps;
  const int g_end = min(g_begin + a.gps, a.n_groups);
  const int jv = cq >> 2;
  for (int g = g_begin + wave; g < g_end; g += 4) {
    const long long ug = (long long)u * a.n_groups_cap + g;
    const uint8_t *kb = a.k_codes + ((long long)u * a.max_tokens + (long long)g * G + 4 * tb) * KROW +
                        16 * cb * BITS / 8;
    uint32_t kw[4][BITS / 2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (BITS == 2) {
        kw[r][0] = *reinterpret_cast<const uint32_t *>(kb + r * KROW);
      } else {
        const uint2 x = *reinterpret_cast<const uint2 *>(kb + r * KROW);
        kw[r][0] = x.x;
        kw[r][1] = x.y;
      }
    }
    const uint8_t *vb = a.v_codes + ((ug * (G / 8) + oc) * D + 8 * cq) * BITS;
    uint32_t vw[2 * BITS];
    {
      const uint4 x = *reinterpret_cast<const uint4 *>(vb);
      vw[0] = x.x; vw[1] = x.y; vw[2] = x.z; vw[3] = x.w;
      if constexpr (BITS == 4) {
        const uint4 y = *reinterpret_cast<const uint4 *>(vb + 16);
        vw[4] = y.x; vw[5] = y.y; vw[6] = y.z; vw[7] = y.w;
      }
    }
    float sk[16], zk[16], sv[8], zv[8];
    ld16(a.k_scale + ug * D + 16 * cb, sk);
    ld16(a.k_zero + ug * D + 16 * cb, zk);
    ld8(a.v_scale + (ug * (D / G) + jv) * G + 8 * oc, sv);
    ld8(a.v_zero + (ug * (D / G) + jv) * G + 8 * oc, zv);

    float qs[16], beta = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      qs[c] = qv[c] * sk[c];
      beta += qv[c] * zk[c];
    }
    beta = xor_sum(xor_sum(xor_sum(beta, 1), 2), 4);

    float s4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float acc = 0.f;
      if constexpr (BITS == 2) {
        const uint32_t w = kw[r][0];
        const uint32_t x = w & 0x33333333u, y = (w >> 2) & 0x33333333u;
        // byte k of x: channels 4k, 4k+2 ; of y: 4k+1, 4k+3
        f32x2_t f;
        f = fp4x2_to_f32x2<0>(x); acc += qs[0] * f[0] + qs[2] * f[1];
        f = fp4x2_to_f32x2<0>(y); acc += qs[1] * f[0] + qs[3] * f[1];
        f = fp4x2_to_f32x2<1>(x); acc += qs[4] * f[0] + qs[6] * f[1];
        f = fp4x2_to_f32x2<1>(y); acc += qs[5] * f[0] + qs[7] * f[1];
        f = fp4x2_to_f32x2<2>(x); acc += qs[8] * f[0] + qs[10] * f[1];
        f = fp4x2_to_f32x2<2>(y); acc += qs[9] * f[0] + qs[11] * f[1];
        f = fp4x2_to_f32x2<3>(x); acc += qs[12] * f[0] + qs[14] * f[1];
        f = fp4x2_to_f32x2<3>(y); acc += qs[13] * f[0] + qs[15] * f[1];
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t w = kw[r][i];
          const uint32_t x = w & 0x0F0F0F0Fu, y = (w >> 4) & 0x0F0F0F0Fu;
          const float *q8 = qs + 8 * i;
          f32x2_t f;
          f = fp8x2_to_f32x2<false>(x); acc += q8[0] * f[0] + q8[2] * f[1];
          f = fp8x2_to_f32x2<false>(y); acc += q8[1] * f[0] + q8[3] * f[1];
          f = fp8x2_to_f32x2<true>(x); acc += q8[4] * f[0] + q8[6] * f[1];
          f = fp8x2_to_f32x2<true>(y); acc += q8[5] * f[0] + q8[7] * f[1];
        }
      }
      acc = xor_sum(xor_sum(xor_sum(acc, 1), 2), 4);
      s4[r] = acc + beta;
    }
    float mx = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
    mx = xor_max(xor_max(xor_max(mx, 8), 16), 32);
    const bool need = mx > m_run + kRescaleSlack;
    if (__any(need)) {
      const float mnew = need ? mx : m_run;
      const float al = m_run == kNegInf ? 0.f : fast_exp2(m_run - mnew);
#pragma unroll
      for (int i = 0; i < 8; ++i) oacc[i] *= al;
      l_run *= al;
      z_run *= al;
      m_run = mnew;
    }
    float p4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p4[r] = fast_exp2(s4[r] - m_run);
      l_run += p4[r];
    }
    // hand the 32 probabilities to the P.V layout through LDS (same wave)
    if (cb == 0) *reinterpret_cast<float4 *>(&sm.vs.p[wave][4 * tb]) = make_float4(p4[0], p4[1], p4[2], p4[3]);
    __builtin_amdgcn_wave_barrier();
    float p8[8];
    {
      const float4 x = *reinterpret_cast<const float4 *>(&sm.vs.p[wave][8 * oc]);
      const float4 y = *reinterpret_cast<const float4 *>(&sm.vs.p[wave][8 * oc + 4]);
      p8[0] = x.x; p8[1] = x.y; p8[2] = x.z; p8[3] = x.w;
      p8[4] = y.x; p8[5] = y.y; p8[6] = y.z; p8[7] = y.w;
    }
    __builtin_amdgcn_wave_barrier();
    float pp[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pp[k] = p8[k] * sv[k];
      z_run += p8[k] * zv[k];
    }
    if constexpr (BITS == 2) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t w = vw[d];
        const uint32_t x = w & 0x33333333u, y = (w >> 2) & 0x33333333u;
        // bytes 0,1: channel 2d (tokens (0,2),(4,6) / (1,3),(5,7)); bytes 2,3: channel 2d+1
        f32x2_t f;
        float o0 = oacc[2 * d], o1 = oacc[2 * d + 1];
        f = fp4x2_to_f32x2<0>(x); o0 += pp[0] * f[0] + pp[2] * f[1];
        f = fp4x2_to_f32x2<0>(y); o0 += pp[1] * f[0] + pp[3] * f[1];
        f = fp4x2_to_f32x2<1>(x); o0 += pp[4] * f[0] + pp[6] * f[1];
        f = fp4x2_to_f32x2<1>(y); o0 += pp[5] * f[0] + pp[7] * f[1];
        f = fp4x2_to_f32x2<2>(x); o1 += pp[0] * f[0] + pp[2] * f[1];
        f = fp4x2_to_f32x2<2>(y); o1 += pp[1] * f[0] + pp[3] * f[1];
        f = fp4x2_to_f32x2<3>(x); o1 += pp[4] * f[0] + pp[6] * f[1];
        f = fp4x2_to_f32x2<3>(y); o1 += pp[5] * f[0] + pp[7] * f[1];
        oacc[2 * d] = o0; oacc[2 * d + 1] = o1;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = vw[e];
        const uint32_t x = w & 0x0F0F0F0Fu, y = (w >> 4) & 0x0F0F0F0Fu;
        f32x2_t f;
        float o0 = oacc[e];
        f = fp8x2_to_f32x2<false>(x); o0 += pp[0] * f[0] + pp[2] * f[1];
        f = fp8x2_to_f32x2<false>(y); o0 += pp[1] * f[0] + pp[3] * f[1];
        f = fp8x2_to_f32x2<true>(x); o0 += pp[4] * f[0] + pp[6] * f[1];
        f = fp8x2_to_f32x2<true>(y); o0 += pp[5] * f[0] + pp[7] * f[1];
        oacc[e] = o0;
      }
    }
  }
  const float l = xor_sum(xor_sum(xor_sum(l_run, 8), 16), 32);
  const float z = xor_sum(xor_sum(z_run, 16), 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = xor_sum(xor_sum(oacc[i], 16), 32) + z;
  __syncthreads();   // p[] of every wave consumed before the merge buffer reuses it
  if (oc == 0) {
    float *dst = &sm.mg.o[wave][0][8 * cq];
    *reinterpret_cast<float4 *>(dst) = make_float4(oacc[0], oacc[1], oacc[2], oacc[3]);
    *reinterpret_cast<float4 *>(dst + 4) = make_float4(oacc[4], oacc[5], oacc[6], oacc[7]);
  }
  if (lane == 0) {
    sm.mg.m[wave][0] = m_run;
    sm.mg.l[wave][0] = l;
  }
  merge_and_store<1>(sm.mg, a, u, split);
}

// ---------------------------------------------------------- combine -----
__global__ __launch_bounds__(128) void combine_kernel(DecodeArgs a) {
  const int row = blockIdx.x, c = threadIdx.x;
  const int hq_count = a.kv_heads * a.qpk;
  const int b = row / hq_count, hq = row % hq_count;
  const int h = hq / a.qpk, j = hq % a.qpk;
  const long long u = (long long)b * a.kv_heads + h;
  const float *base = a.part + (u * a.n_split * a.qpk + j) * kPartStride;
  const long long stride = (long long)a.qpk * kPartStride;
  float M = kNegInf;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, base[s * stride]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < a.n_split; ++s) {
    const float *p = base + s * stride;
    const float f = p[0] == kNegInf ? 0.f : fast_exp2(p[0] - M);
    l += f * p[1];
    o += f * p[4 + c];
  }
  a.out[(long long)row * D + c] = o / l;
}

}  // namespace

hipError_t launch_decode(int bits, const DecodeArgs &a, hipStream_t s) {
  const dim3 grid(a.n_split, a.n_units), block(256);
  const int nhb = (a.qpk + 3) / 4;
#define KIVI_LAUNCH(BITS)                                                                 \
  do {                                                                                    \
    if (a.qpk == 1)                                                                       \
      hipLaunchKernelGGL((decode_valu_kernel<BITS>), grid, block, 0, s, a);               \
    else if (nhb == 1)                                                                    \
      hipLaunchKernelGGL((decode_mfma_kernel<BITS, 1>), grid, block, 0, s, a);            \
    else if (nhb == 2)                                                                    \
      hipLaunchKernelGGL((decode_mfma_kernel<BITS, 2>), grid, block, 0, s, a);            \
    else if (nhb == 3)                                                                    \
      hipLaunchKernelGGL((decode_mfma_kernel<BITS, 3>), grid, block, 0, s, a);            \
    else                                                                                  \
      hipLaunchKernelGGL((decode_mfma_kernel<BITS, 4>), grid, block, 0, s, a);            \
  } while (0)
  if (bits == 2)
    KIVI_LAUNCH(2);
  else
    KIVI_LAUNCH(4);
#undef KIVI_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(a.n_units * a.qpk), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace kivi
