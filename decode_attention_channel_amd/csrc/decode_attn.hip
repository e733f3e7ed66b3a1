// decode_attn.hip -- decode-step attention over the KIVI mixed cache.
//
// For every query head: score_t = sigma * q . k_t over the dequantised
// history (per-channel K groups, per-token V groups; "KIVI: A Tuning-Free
// Asymmetric 2bit Quantization for KV Cache", method paragraph) and the bf16
// residual (catalog record kivi-2bit-llama3-8b-gqa-8k, KV bytes basis);
// p = softmax(score); out = sum_t p_t v_t, fp32 accumulation.
//
// Split-K flash decoding.  Grid (unit, split): the workgroups of a unit (as
// many as fill the resident slots of the chip in one round) take byte shares
// of its work -- quantised groups of 32 tokens, then the bf16 residual in
// chunks of 32.  Within a workgroup each wave keeps its own online-softmax
// state over its part: a fixed quarter of the share (4 waves, several
// workgroups per compute unit), or, with one workgroup of 8 or 12 waves per
// compute unit, groups taken one at a time from an LDS counter (the default)
// or round-robin (bitwise-repeatable results).  The waves' states
// are merged in LDS at the end; each workgroup writes (m, l, o[128]) per
// query head, and the last workgroup of a unit to finish merges that unit's
// partials into `out` (arrival counter in the workspace).  A decode step
// whose ring is full also quantises the G oldest ring tokens into the new
// group inside the same launch (fold_flush), before any wave reads it.
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
// q.K^T and P.V run on v_mfma_f32_16x16x32_bf16.  The scores are computed
// transposed: the scaled queries of up to 4 query heads of the kv head are
// the A operand (rows head x {hi, lo, hi, lo}) and the codes the B operand
// (32 channels x 16 tokens), so each lane ends with the scores of two tokens
// of one head and the softmax is evaluated once per (token, head).  For P.V
// the codes are the A operand (16 channels x 32 tokens) and the scaled
// probabilities the B operand (columns channel block x head), reached through
// a per-wave LDS exchange.  MHA (one query head per kv head) leaves three
// heads idle.  The scaled queries and probabilities are split into bf16 hi +
// lo parts (relative error ~2^-16), occupying different MFMA rows (q.K^T) or
// two MFMAs (P.V), so the result carries close to fp32 precision.
#include <float.h>
#include <math.h>

#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

#include "kivi_internal.h"
#include "quantize_group.h"

namespace kivi {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

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


template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 2.0f, SEL));
}
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, HI));
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
// x ~= hi + lo with hi = x truncated to bf16 (its upper 16 bits) and
// lo = bf16(x - hi), x - hi being exact in fp32: two packed words for a pair,
// |x - hi - lo| <= 2^-16 |x|
__device__ __forceinline__ void split_bf16(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  const uint32_t b0 = __float_as_uint(x0), b1 = __float_as_uint(x1);
  hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u);   // upper halves of x0 (low word), x1
  lo = pack_bf16x2(x0 - __uint_as_float(b0 & 0xFFFF0000u), x1 - __uint_as_float(b1 & 0xFFFF0000u));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


// s_waitcnt operand that waits for vmcnt == 0 only: vmcnt bits [3:0] and
// [15:14] zero, expcnt [6:4] and lgkmcnt [11:8] at their maxima (no wait).
constexpr int kWaitVmcnt0 = 0x0F70;

// Split partials cross workgroups (and XCDs, whose L2 caches are not coherent
// with each other), so they are written and read with agent-scope atomic
// accesses, which are coherent without flushing or invalidating the L2.
__device__ __forceinline__ void st_shared_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_shared_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- merge ---
// Each wave contributes (m, l, o[128]) per head; the workgroup writes one
// partial per head: M = max m_w, l = sum 2^(m_w - M) l_w, o likewise.  A
// unit's only workgroup (n_split == 1) writes out = o / l itself instead,
// the value the combine would compute from its one partial (weight 2^0).
template <int HMAX, int NW>
struct MergeSmem {
  float m[NW][HMAX];
  float l[NW][HMAX];
  float o[NW][HMAX][D];
  int last;
};

template <int HMAX, int NW>
__device__ void merge_and_store(MergeSmem<HMAX, NW> &sm, const DecodeArgs &a, int u, int split,
                                int4 next_state) {
  __syncthreads();
  const int qpk = a.qpk;
  const bool direct = a.n_split == 1;
  float *part = a.part + ((long long)u * a.n_split + split) * qpk * kPartStride;
  for (int idx = threadIdx.x; idx < qpk * D; idx += 64 * NW) {
    const int hh = idx / D, c = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][hh]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = sm.m[w][hh] == kNegInf ? 0.f : fast_exp2(sm.m[w][hh] - M);
      l += f * sm.l[w][hh];
      o += f * sm.o[w][hh][c];
    }
    if (direct) {
      // a unit with no token (a flagged sequence of a mixed-length batch) gets 0
      a.out[((long long)u * qpk + hh) * D + c] = l > 0.f ? o / l : 0.f;
      continue;
    }
    st_shared_agent(part + hh * kPartStride + 4 + c, o);
    if (c == 0) {
      st_shared_agent(part + hh * kPartStride + 0, M);
      st_shared_agent(part + hh * kPartStride + 1, l);
    }
  }
  if (direct && threadIdx.x == 0 && a.state_out && u % a.kv_heads == 0)
    reinterpret_cast<int4 *>(a.state_out)[u / a.kv_heads] = next_state;
}

// ------------------------------------------------------------ combine -----
// Called by every workgroup after it stored its partials.  Arrivals are
// counted per unit; the last workgroup of the unit merges the n_split
// partials of each of its query heads,
//   M = max m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// writes `out`, and re-arms the counter to zero for the next call.
// NT: threads of the workgroup (a constant: blockDim would be a late scalar
// load from the dispatch packet)
template <int NT>
__device__ void finish_unit(const DecodeArgs &a, int u, int *s_last, int4 next_state) {
  // Every wave first waits until its own partial stores have completed
  // (vmcnt counts stores on this architecture; a completed agent-scope store
  // is visible to every compute unit).  The barrier alone would only wait for
  // LDS traffic, so without this wait the arrival could be counted while
  // another wave's stores are still in flight, and the last workgroup could
  // merge a stale partial left by an earlier launch on the same workspace.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(a.counters + u, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_last = prev == (unsigned)(a.n_split - 1);
  }
  __syncthreads();
  if (!*s_last) return;
  const int qpk = a.qpk;
  const long long stride = (long long)qpk * kPartStride;
  constexpr int kBatch = 8;   // splits whose partials are loaded together
  for (int idx = threadIdx.x; idx < qpk * D; idx += NT) {
    const int hh = idx / D, c = idx % D;
    const float *base = a.part + ((long long)u * a.n_split * qpk + hh) * kPartStride;
    float M = kNegInf, l = 0.f, o = 0.f;
    for (int s0 = 0; s0 < a.n_split; s0 += kBatch) {
      float mb[kBatch], lb[kBatch], ob[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int sp = min(s0 + k, a.n_split - 1);
        const float *pp = base + sp * stride;
        mb[k] = s0 + k < a.n_split ? ld_shared_agent(pp) : kNegInf;
        lb[k] = ld_shared_agent(pp + 1);
        ob[k] = ld_shared_agent(pp + 4 + c);
      }
      float Mn = M;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) Mn = fmaxf(Mn, mb[k]);
      const float al = M == kNegInf ? 0.f : fast_exp2(M - Mn);
      l *= al;
      o *= al;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const float f = mb[k] == kNegInf ? 0.f : fast_exp2(mb[k] - Mn);
        l += f * lb[k];
        o += f * ob[k];
      }
      M = Mn;
    }
    // a unit with no token (a flagged sequence of a mixed-length batch) gets 0
    a.out[((long long)u * qpk + hh) * D + c] = l > 0.f ? o / l : 0.f;
  }
  if (threadIdx.x == 0) {
    __hip_atomic_store(a.counters + u, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (a.state_out && u % a.kv_heads == 0)
      reinterpret_cast<int4 *>(a.state_out)[u / a.kv_heads] = next_state;
  }
}

// Mixed-length batches: this unit's counters from its sequence's state
// (DecodeArgs::state_in), with the step's flush and the fused append applied
// the same way as kivi_decode_step; the counters of `a` are replaced.  Returns
// the sequence's state after the step.  A sequence with a flag keeps its
// cache; one that needs a flush without room for another group gets
// kSeqFull and no append.  A state row out of range (state_ok) becomes an
// empty sequence with kSeqBadLength.
__device__ __forceinline__ int4 apply_unit_state(DecodeArgs &a, int u) {
  const int4 s = reinterpret_cast<const int4 *>(a.state_in)[u / a.kv_heads];
  int n_q = s.x, n_res = s.y, res_start = s.z, flags = s.w;
  if (!state_ok(n_q, n_res, res_start, flags, G, a.slots, a.max_tokens)) {
    n_q = n_res = res_start = 0;
    flags = kSeqBadLength;
  }
  bool append = flags == 0;
  a.flush_g = -1;
  if (append && n_res + 1 >= a.slots) {
    // the G oldest ring tokens go into group n_q / G, quantised in this
    // launch, iff there is room for it (and, paged, a page)
    if (n_res + 1 == a.slots && n_q + G <= a.max_tokens &&
        (!a.pages.table || group_slot(a.pages, a.kv_heads, 0, u, n_q / G) >= 0)) {
      a.flush_g = n_q / G;
      a.flush_src = res_start;
      n_q += G;
      n_res -= G;
      res_start = (res_start + G) % a.slots;
    } else {
      flags |= kSeqFull;
      append = false;
    }
  }
  if (flags & kSeqBadLength) n_res = 0;   // nothing valid to attend to
  a.n_groups = (flags & kSeqBadLength) ? 0 : n_q / G;
  a.res_start = res_start;
  a.new_idx = append ? n_res : -1;
  a.n_res = append ? n_res + 1 : n_res;
  return make_int4(n_q, a.n_res, res_start, flags);
}

// ------------------------------------------------------------ MFMA path ---
// ---- cross-lane sums / maxima without LDS round trips.  A wave is 4 rows of
// 16 lanes; permlane16/32 swaps exchange row pairs, so x + swap(x) is the
// sum over lanes l and l^16 (l^32) in every lane.
__device__ __forceinline__ float sum_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// IEEE maximum (NaN-propagating): one v_maximum3_f32, where fmaxf on
// values from a lane exchange would first quiet both operands
__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// sum over the 4 lanes n, n+-4, n+-8, n+-12 of each 16-lane row (DPP rotations)
__device__ __forceinline__ float sum_row_stride4(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true));
  return x;
}

typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2_t;

// Buffer descriptor of a workgroup-uniform range (values forced into SGPRs, so
// the loads need no per-lane descriptor loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  // readfirstlane returns int: go through uint32_t so that widening does not
  // sign-extend the low address word into the high one
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>((hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Raw bytes of one group as one lane of the MFMA path needs them: K codes of
// its two A-operand rows, V codes of its 8 channels x 8 tokens, and the
// scale/zero values its q' and P.V roles read.
template <int BITS>
struct GroupRaw {
  uint32_t kw[2][BITS];   // per tile: 32 channels of one token
  uint32_t vw[2 * BITS];  // 8 channels x 8 tokens
  uint32_t mw[4][2];      // this lane's 8 bytes of each of k_scale, k_zero, v_scale, v_zero
};

// Bytes of one scale or zero value: fp32, or fp16 / bf16 (META == 1).
template <int META>
constexpr int kMetaBytes = META == 1 ? 2 : 4;

// Page table entry read through the scalar cache (the table is read-only
// for the whole launch), so that it does not count among the vector loads
// of the group pipeline.
__device__ __forceinline__ int page_entry(const int32_t *table, long long i) {
  typedef __attribute__((address_space(4))) const int32_t *ConstPtr;
  return ((ConstPtr)table)[i];
}

// Group records (layout in kivi_internal.h): one buffer resource over the
// unit's records, or (PAGED) over the whole pool.  The host keeps a unit's
// records within kMaxUnitRecordBytes (2^30) and a pool below 2^31 bytes, so
// that kOutOfRange offsets stay out of range (see load_record).  Lane l reads bytes
// [16 l, 16 l + 16) of every plane, the group entering as a scalar offset.
struct RecView {
  __amdgpu_buffer_rsrc_t rec;
  uint32_t o_lane;
};

template <int BITS, int META, bool PAGED>
__device__ __forceinline__ RecView make_rec_view(const DecodeArgs &a, int u, int lane) {
  constexpr long long REC = rec_bytes(BITS, META);
  RecView v;
  if constexpr (PAGED) {
    const long long groups = (long long)a.pages.num_pages * a.kv_heads << a.pages.shift;
    v.rec = make_rsrc(a.records, (uint32_t)(groups * REC));
  } else {
    v.rec = make_rsrc(a.records + u * a.n_groups_cap * REC, (uint32_t)(a.n_groups_cap * REC));
  }
  v.o_lane = 16 * lane;
  return v;
}

// Loads of group g.  With live == false the same loads are issued with a
// per-lane offset beyond every buffer's range: they return zeros and touch
// no memory.  Issuing a fixed number of loads per pipeline step keeps the
// compiler's count of outstanding loads exact, so each step waits only for
// the group it computes and not for the prefetches behind it.
// 2^31: at least twice a unit's record range (kMaxUnitRecordBytes) and above
// any pool (< 2^31).  The scalar offset of a not-live contiguous group is at
// most a few records past the unit's range, so offset + kOutOfRange stays
// below 2^32 and above every range, whether or not the hardware adds the
// scalar offset before its range check.
constexpr uint32_t kOutOfRange = 0x80000000u;
static_assert(kOutOfRange >= 2u * (uint32_t)kMaxUnitRecordBytes, "sentinel inside a unit's range");
// cache policy of the history loads: non-temporal (each byte is read once per
// step), which keeps them from displacing other lines in the caches
constexpr int kStream = 2;

// Groups in flight per wave beyond the one being computed.  With 8-12 waves
// per compute unit one is enough to keep HBM busy, and fewer groups
// committed per wave end the launch with less imbalance between waves (it
// measured faster than two or three on both paths).
constexpr int kPrefetch = 1;


// The planes of group g as this lane's 16-byte pieces.  PAGED: the group's
// slot in the pool; a group without a page is loaded as not live.
template <int BITS, int META, bool PAGED>
__device__ __forceinline__ void load_record(u32x4_t (&q)[rec_planes(BITS, META)], const RecView &v,
                                            const DecodeArgs &a, int u, int g, bool live) {
  long long slot = g;   // contiguous: the view starts at the unit's records
  if constexpr (PAGED) {
    slot = -1;
    const int pi = g >> a.pages.shift;
    if (live && pi < a.pages.max_pages) {
      const int b = u / a.kv_heads, h = u - b * a.kv_heads;
      const int e = page_entry(a.pages.table, (long long)b * a.pages.max_pages + pi);
      if (e >= 0 && e < a.pages.num_pages)
        slot = (((long long)e * a.kv_heads + h) << a.pages.shift) + (g & ((1 << a.pages.shift) - 1));
    }
    live = slot >= 0;
    if (!live) slot = 0;
  }
  // wave-uniform: a scalar buffer offset
  const uint32_t sc = __builtin_amdgcn_readfirstlane((uint32_t)slot * (uint32_t)rec_bytes(BITS, META));
  const uint32_t o = v.o_lane + (live ? 0u : kOutOfRange);
#pragma unroll
  for (int p = 0; p < rec_planes(BITS, META); ++p)
    q[p] = __builtin_amdgcn_raw_buffer_load_b128(v.rec, o + p * kPlaneBytes, sc, kStream);
}

// Scale/zero pairs of this lane (values 2l, 2l + 1 of each array) from the
// meta plane(s) of a record.
template <int BITS, int META>
__device__ __forceinline__ void record_meta(uint32_t (&mw)[4][2],
                                            const u32x4_t (&q)[rec_planes(BITS, META)]) {
  if constexpr (META == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mw[i][0] = q[BITS][i];
      mw[i][1] = 0;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mw[i][0] = q[BITS + (i >> 1)][2 * (i & 1)];
      mw[i][1] = q[BITS + (i >> 1)][2 * (i & 1) + 1];
    }
  }
}

template <int BITS, int META, bool PAGED>
__device__ __forceinline__ void load_group(GroupRaw<BITS> &r, const RecView &v,
                                           const DecodeArgs &a, int u, int g, bool live) {
  u32x4_t q[rec_planes(BITS, META)];
  load_record<BITS, META, PAGED>(q, v, a, u, g, live);
  if constexpr (BITS == 2) {
    r.kw[0][0] = q[0][0]; r.kw[0][1] = q[0][1];
    r.kw[1][0] = q[0][2]; r.kw[1][1] = q[0][3];
#pragma unroll
    for (int i = 0; i < 4; ++i) r.vw[i] = q[1][i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.kw[0][i] = q[0][i]; r.kw[1][i] = q[1][i];
      r.vw[i] = q[2][i]; r.vw[4 + i] = q[3][i];
    }
  }
  record_meta<BITS, META>(r.mw, q);
}

// Write this lane's two values of each scale/zero array to the wave's LDS
// slot as floats (arrays: k_scale, k_zero, v_scale, v_zero).  META == 1:
// fp16 scales and bf16 zeros are widened exactly.
template <int META>
__device__ __forceinline__ void stage_meta(const uint32_t (&mw)[4][2], float (*meta)[D], int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint2 w;
    if constexpr (META == 1) {
      const uint32_t x = mw[i][0];
      float lo, hi;
      if (i == 0 || i == 2) {   // fp16 scale
        lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xFFFFu));
        hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
      } else {                  // bf16 zero
        lo = __uint_as_float(x << 16);
        hi = __uint_as_float(x & 0xFFFF0000u);
      }
      w = make_uint2(__float_as_uint(lo), __float_as_uint(hi));
    } else {
      w = make_uint2(mw[i][0], mw[i][1]);
    }
    *reinterpret_cast<uint2 *>(&meta[i][2 * lane]) = w;
  }
}

// Per-wave LDS staging.  A wave works on quantised groups and, after them,
// on residual chunks (vres), so the two share storage.  The groups use two
// buffer sets: while a group is computed from one set, the next group's
// scale/zero and q' operand are staged in the other.
template <int NHB>
union WaveSmem {
  struct {
    uint4 bq[NHB][128];    // q' operand chunks (8 bf16) per head block, indexed by bq_index
    float meta[4][D];      // the group's k_scale, k_zero, v_scale, v_zero
    float beta[NHB][4];    // q . z^K per head of each block
  } g[2];
  uint16_t vres[G][D];     // one residual chunk of V rows (bf16)
};
template <int NHB, int NW>
struct MfmaSmem {
  WaveSmem<NHB> w[NW];
  // probabilities of the current group or residual chunk, [head][token],
  // handed from the score lanes to the P.V lanes
  float pex[NW][NHB][4][G];
};

// LDS chunk of the q' operand for (hi/lo xx, head h, MFMA step m, lane group
// gq).  The low 3 bits pick the 16-byte bank group; (xx + h + 2gq) mod 8
// spreads both the stores (one xx at a time) and the loads (one m at a time)
// evenly over the 8 bank groups.
__device__ __forceinline__ int bq_index(int xx, int h, int m, int gq) {
  return (m * 4 + h) * 8 + ((xx + h + 2 * gq) & 7);
}

// Online-softmax state of one wave (per head block), in two lane roles.
// Score lanes (column = token slot lane & 15, row group = head lane >> 4):
// running max (log2 units), the partial sum of p over the lane's tokens, and
// the finite reference the quantised groups' scores are taken relative to
// (their MFMA accumulators start at beta - m_ref): m_run once it is finite,
// 0 before.  P.V lanes (column n = 4j + head, n = lane & 15): accumulators in
// the MFMA output layout and the partial sum of p * zero^V.
template <int NHB>
struct WaveState {
  f32x4_t acc[NHB][8];
  float z_run[NHB];
  float m_run[NHB], l_run[NHB], m_ref[NHB];
};

// Maximum / sum over the 16 lanes of a row (DPP rotations; every lane gets
// the result).  A row rotation reads every lane of the row, so bound_ctrl is
// moot; setting it lets the compiler fold the move into the operation that
// consumes it.
template <int CTRL>
__device__ __forceinline__ float dpp_rot(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                0xF, 0xF, true));
}
__device__ __forceinline__ float row_max16(float x) {
  x = max2(x, dpp_rot<0x128>(x));   // row_ror:8
  x = max2(x, dpp_rot<0x124>(x));   // row_ror:4
  x = max2(x, dpp_rot<0x122>(x));   // row_ror:2
  return max2(x, dpp_rot<0x121>(x));   // row_ror:1
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_rot<0x128>(x);
  x += dpp_rot<0x124>(x);
  x += dpp_rot<0x122>(x);
  return x + dpp_rot<0x121>(x);
}
// x is uniform within each row (a value per head, head = row); returns, in
// every lane, the value of head lane & 3 (the head of its P.V column)
__device__ __forceinline__ float head_value_for_pv(float x, int lane) {
  const int xi = __builtin_bit_cast(int, x);
  const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float a3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  const int h = lane & 3;
  return h == 0 ? a0 : h == 1 ? a1 : h == 2 ? a2 : a3;
}

// First half of a group: stage its scale/zero in buffer set `buf`, build the
// q' = q * s^K operand (hi/lo) of every head block there, and beta = q . z^K
// per head (into the set's beta).  A group past the end has all-zero loads:
// its q' and beta are zeros and the buffer set is not read.
template <int NHB, int META, int NW>
__device__ __forceinline__ void prep_group(const uint32_t (&mw)[4][2], MfmaSmem<NHB, NW> &smf,
                                           int buf, const float (&qv)[NHB][8], int wave, int lane,
                                           int gq, int ch, int cm) {
  auto &gs = smf.w[wave].g[buf];
  stage_meta<META>(mw, gs.meta, lane);
  __builtin_amdgcn_wave_barrier();
  float sk[8], zk[8];
  {
    const float *km = &gs.meta[0][32 * gq + 8 * cm];
    const float *kz = &gs.meta[1][32 * gq + 8 * cm];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sk[i] = km[i]; zk[i] = kz[i];
    }
  }
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    float bt = 0.f;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int s = 0; s < 8; s += 2) {
      split_bf16(qv[hb][s] * sk[P8[s]], qv[hb][s + 1] * sk[P8[s + 1]], hi[s / 2], lo[s / 2]);
      bt += qv[hb][s] * zk[P8[s]];
      bt += qv[hb][s + 1] * zk[P8[s + 1]];
    }
    gs.bq[hb][bq_index(0, ch, cm, gq)] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    gs.bq[hb][bq_index(1, ch, cm, gq)] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    // every lane with (lane & 3) == head holds the sum for that head
    gs.beta[hb][lane & 3] = sum_x32(sum_x16(sum_row_stride4(bt)));
  }
}

// Second half of a group, from buffer set `buf` (filled by prep_group): the
// scores on the MFMA, the online softmax and P.V.  `mid` runs once, after the
// first head block's score MFMAs are issued: the next group's prep_group goes
// there, so that its VALU and LDS work overlaps the matrix core.
//
// The scores are computed transposed: q' is the A operand (row 4 head + x,
// x = hi, lo, hi, lo) and the codes the B operand (column = token slot), so a
// score lane (column n, row group gq) holds the scores of its two tokens for
// head gq alone, and the softmax runs once per (token, head).  The
// probabilities reach the P.V lanes (column n = 4j + head, tokens 8gq ..
// 8gq + 7) through the wave's LDS exchange area.
template <int BITS, int NHB, int NW, class Mid>
__device__ __forceinline__ void attend_group(const GroupRaw<BITS> &raw, WaveState<NHB> &st,
                                             MfmaSmem<NHB, NW> &smf, int buf, int wave, int lane,
                                             Mid &&mid) {
  auto &gs = smf.w[wave].g[buf];
  const int n = lane & 15, gq = lane >> 4;
  // ---- A operands (exact codes).  With one head block they are unpacked
  // next to the MFMAs that read them (fewer live registers, and the
  // converts issue while the matrix core works); otherwise once, up front.
  constexpr bool kLazy = NHB == 1;
  Op8 ak[2][4];
  Op8 av[8];
  auto unpack_k = [&](int tile, int m) {   // fills ak[tile][m] (and its pair)
    if constexpr (BITS == 2) {
      if ((m & 1) == 0) unpack2(raw.kw[tile][m / 2], ak[tile][m], ak[tile][m + 1]);
    } else {
      unpack4(raw.kw[tile][m], ak[tile][m]);
    }
  };
  auto unpack_v = [&](int mt) {            // fills av[mt] (and its pair)
    if constexpr (BITS == 2) {
      if ((mt & 1) == 0) unpack2(raw.vw[mt / 2], av[mt], av[mt + 1]);
    } else {
      unpack4(raw.vw[mt], av[mt]);
    }
  };
  if constexpr (!kLazy) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      unpack_k(0, m);
      unpack_k(1, m);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) unpack_v(mt);
  }

#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    // ---- scores, transposed: this lane's rows 4gq + r are head gq, x = r;
    // relative to m_ref, beta - m_ref entering through the hi row (r = 0)
    f32x4_t sc[2];
    {
      const float bt = gs.beta[hb][gq] - st.m_ref[hb];
      sc[0] = f32x4_t{bt, 0.f, 0.f, 0.f};
      sc[1] = sc[0];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if constexpr (kLazy) {
        unpack_k(0, m);
        unpack_k(1, m);
      }
      // A row n = 4 head + x: q' of head n >> 2, hi / lo by x & 1
      Op8 aq;
      const uint4 x = gs.bq[hb][bq_index(n & 1, n >> 2, m, gq)];
      aq.u[0] = x.x; aq.u[1] = x.y; aq.u[2] = x.z; aq.u[3] = x.w;
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
        sc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq.v, ak[tile][m].v, sc[tile], 0, 0, 0);
    }
    if (hb == 0) mid();
    // this lane's V scale/zero: channel block n >> 2, tokens 8gq .. 8gq + 7
    float sv[8], zv[8];
    {
      const float *vm = &gs.meta[2][(n >> 2) * G + 8 * gq];
      const float *vz = &gs.meta[3][(n >> 2) * G + 8 * gq];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sv[i] = vm[i]; zv[i] = vz[i];
      }
    }
    // the lane's two scores: tile t holds token 8 (n >> 2) + (n & 3) + 4t
    float s2[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) s2[tile] = sc[tile][0] + sc[tile][1];

    // ---- online softmax (log2 domain), lazily rescaled; s2 is relative to
    // m_ref, which equals m_run except before the first rescale.  A rescale
    // is due for a head iff its maximum over the wave's 32 tokens passes the
    // bound, i.e. iff some lane's own maximum does: the lane-local test
    // decides, and the maximum across the row is taken only when it is due.
    float mx = fmaxf(s2[0], s2[1]);
    const float bound = st.m_run[hb] - st.m_ref[hb] + kRescaleSlack;
    if (__any(mx > bound)) {
      mx = row_max16(mx);
      const bool need = mx > bound;
      const float mnew = need ? mx + st.m_ref[hb] : st.m_run[hb];
      const float al = st.m_run[hb] == kNegInf ? 0.f : fast_exp2(st.m_run[hb] - mnew);
      st.l_run[hb] *= al;
      const float d = mnew - st.m_ref[hb];
      s2[0] -= d;
      s2[1] -= d;
      st.m_run[hb] = mnew;
      st.m_ref[hb] = mnew;
      // the P.V lanes of each head rescale by that head's factor
      const float alp = head_value_for_pv(al, lane);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) st.acc[hb][mt] *= alp;
      st.z_run[hb] *= alp;
    }
    {
      const float p0 = fast_exp2(s2[0]), p1 = fast_exp2(s2[1]);
      st.l_run[hb] += p0 + p1;
      float *pe = &smf.pex[wave][hb][gq][8 * (n >> 2) + (n & 3)];
      pe[0] = p0;
      pe[4] = p1;
    }
    __builtin_amdgcn_wave_barrier();
    // P.V lanes: p of head n & 3 for tokens 8gq .. 8gq + 7
    float p[8];
    {
      const float4 *pr = reinterpret_cast<const float4 *>(&smf.pex[wave][hb][n & 3][8 * gq]);
      const float4 a = pr[0], b = pr[1];
      p[0] = a.x; p[1] = a.y; p[2] = a.z; p[3] = a.w;
      p[4] = b.x; p[5] = b.y; p[6] = b.z; p[7] = b.w;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) st.z_run[hb] += p[k] * zv[k];
    // ---- P.V: columns n = 4j + head; B slot s <-> token 8gq + P8[s]
    Op8 bh, bl;
#pragma unroll
    for (int s = 0; s < 8; s += 2)
      split_bf16(p[P8[s]] * sv[P8[s]], p[P8[s + 1]] * sv[P8[s + 1]], bh.u[s / 2], bl.u[s / 2]);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      if constexpr (kLazy) unpack_v(mt);
      st.acc[hb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt].v, bh.v, st.acc[hb][mt], 0, 0, 0);
      st.acc[hb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt].v, bl.v, st.acc[hb][mt], 0, 0, 0);
    }
  }
}

// One residual chunk (32 ring slots, `valid` of them live) through the same
// MFMA pipeline as a quantised group: the transposed scores with the raw
// query as the A operand (the hi row of each head; the other rows zero; the
// softmax scale applied to the scores) and the bf16 K rows as B; P.V with the
// chunk's V rows transposed through LDS as the A operand and p (hi/lo) as B
// for every channel block, p handed over through the exchange area as for a
// group.
template <int NHB, int NW>
__device__ __forceinline__ void mfma_rchunk(const DecodeArgs &a, int u, int rc,
                                            WaveState<NHB> &st, MfmaSmem<NHB, NW> &smf, int wave,
                                            int lane, int n, int gq) {
  const int qpk = a.qpk;
  const int t0 = G * rc, valid = min(G, a.n_res - t0);
  const int slot0 = (a.res_start + t0) % a.slots;   // multiple of G: the chunk is contiguous
  const long long ring = (long long)u * a.slots + slot0;
  const uint16_t *krows = a.k_res + ring * D, *vrows = a.v_res + ring * D;

  // the appended token of a fused step, if it falls in this chunk
  const int new_row = a.new_idx - t0;   // row within the chunk; wave-uniform
  const bool has_new = new_row >= 0 && new_row < G;

  // All loads first, in one batch (one memory latency for the chunk): V rows
  // for the LDS transpose, one contiguous KiB of the chunk per load (load i,
  // lane l: row 4i + l/16, channels 8 (l % 16) .. + 7); K rows of the two
  // tiles as A operands of q.K^T, MFMA step m taking channels 32m + 8gq ..
  // + 7 so that the four lanes of a row read 64 contiguous bytes per load
  // (the query rows use the same order).  Ring rows past `valid` (stale or
  // never written slots, inside the ring) are loaded and then replaced by
  // zeros (V) or masked out of the softmax (K).
  const int vr0 = lane >> 4, vcol = 8 * (lane & 15);
  const int kr0 = 8 * (n >> 2) + (n & 3);
  bool k_new[2];
  const uint4 *ksrc[2];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    const int row = kr0 + 4 * tile;
    k_new[tile] = has_new && row == new_row;
    ksrc[tile] = reinterpret_cast<const uint4 *>(
        k_new[tile] ? a.k_new + (long long)u * D + 8 * gq : krows + (long long)row * D + 8 * gq);
  }
  const int b = u / a.kv_heads, h = u % a.kv_heads;
  // query rows as A operands of the transposed q.K^T (row n = 4 head + x; the
  // hi rows x = 0 take the query, the others zeros): every lane loads a
  // valid row; with one workgroup per compute unit (NW > 4, registers to
  // spare) those of head block 0 come with the chunk
  constexpr bool kQFirst = NW > 4;
  auto q_rows = [&](int hb) {
    const int hh = hb * 4 + (n >> 2);
    return reinterpret_cast<const uint4 *>(
        a.q + ((long long)b * a.kv_heads * qpk + (long long)h * qpk + (hh < qpk ? hh : 0)) * D +
        8 * gq);
  };
  uint4 xq[4];
  if constexpr (kQFirst) {
#pragma unroll
    for (int m = 0; m < 4; ++m) xq[m] = q_rows(0)[4 * m];
  }
  uint4 xv[8], xk[2][4];
  const uint4 *vbase = reinterpret_cast<const uint4 *>(vrows + (long long)vr0 * D + vcol);
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = vbase[i * (4 * D / 8)];   // row 4i + vr0
#pragma unroll
  for (int tile = 0; tile < 2; ++tile)
#pragma unroll
    for (int m = 0; m < 4; ++m) xk[tile][m] = ksrc[tile][4 * m];
  // the fused append (wave-uniform): the new token's V row comes from v_new
  // (load new_row / 4, lanes with vr0 == new_row % 4) and goes into its ring
  // slot
  if (has_new && vr0 == (new_row & 3)) {
    const uint4 x = *reinterpret_cast<const uint4 *>(a.v_new + (long long)u * D + vcol);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i == (new_row >> 2)) xv[i] = x;
    *reinterpret_cast<uint4 *>(a.v_res + (ring + new_row) * D + vcol) = x;
  }
  // stage V rows in LDS
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * i + vr0;
    *reinterpret_cast<uint4 *>(&smf.w[wave].vres[row][vcol]) =
        row < valid ? xv[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  Op8 ak[2][4];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    if (k_new[tile]) {
      uint4 *ring_row = reinterpret_cast<uint4 *>(a.k_res + (ring + kr0 + 4 * tile) * D + 8 * gq);
#pragma unroll
      for (int m = 0; m < 4; ++m) ring_row[4 * m] = xk[tile][m];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      ak[tile][m].u[0] = xk[tile][m].x; ak[tile][m].u[1] = xk[tile][m].y;
      ak[tile][m].u[2] = xk[tile][m].z; ak[tile][m].u[3] = xk[tile][m].w;
    }
  }
  __builtin_amdgcn_wave_barrier();
  // A operands of P.V: row i of M-tile mt = channel 8i + mt, k-slot s = token 8gq + s
  Op8 av[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const uint32_t lo = smf.w[wave].vres[8 * gq + 2 * s2][8 * n + mt];
      const uint32_t hi = smf.w[wave].vres[8 * gq + 2 * s2 + 1][8 * n + mt];
      av[mt].u[s2] = lo | (hi << 16);
    }
  }
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int hh = hb * 4 + (n >> 2);
    const bool hi_row = (n & 3) == 0 && hh < qpk;
    if (hb > 0 || !kQFirst) {
#pragma unroll
      for (int m = 0; m < 4; ++m) xq[m] = q_rows(hb)[4 * m];
    }
    f32x4_t sc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      Op8 aq;
      const uint4 x = hi_row ? xq[m] : make_uint4(0u, 0u, 0u, 0u);
      aq.u[0] = x.x; aq.u[1] = x.y; aq.u[2] = x.z; aq.u[3] = x.w;
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
        sc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq.v, ak[tile][m].v, sc[tile], 0, 0, 0);
    }
    // this lane: head gq, tokens 8 (n >> 2) + (n & 3) + 4 tile of the chunk
    const int tl = 8 * (n >> 2) + (n & 3);
    float s2[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
      s2[tile] = tl + 4 * tile < valid ? sc[tile][0] * a.qscale : kNegInf;
    float mx = fmaxf(s2[0], s2[1]);
    const float bound = st.m_run[hb] + kRescaleSlack;
    if (__any(mx > bound)) {
      mx = row_max16(mx);
      const bool need = mx > bound;
      const float mnew = need ? mx : st.m_run[hb];
      const float al = st.m_run[hb] == kNegInf ? 0.f : fast_exp2(st.m_run[hb] - mnew);
      st.l_run[hb] *= al;
      st.m_run[hb] = mnew;
      st.m_ref[hb] = mnew;
      const float alp = head_value_for_pv(al, lane);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) st.acc[hb][mt] *= alp;
      st.z_run[hb] *= alp;
    }
    {
      const float p0 = fast_exp2(s2[0] - st.m_run[hb]), p1 = fast_exp2(s2[1] - st.m_run[hb]);
      st.l_run[hb] += p0 + p1;
      float *pe = &smf.pex[wave][hb][gq][tl];
      pe[0] = p0;
      pe[4] = p1;
    }
    __builtin_amdgcn_wave_barrier();
    float p[8];
    {
      const float4 *pr = reinterpret_cast<const float4 *>(&smf.pex[wave][hb][n & 3][8 * gq]);
      const float4 a0 = pr[0], a1 = pr[1];
      p[0] = a0.x; p[1] = a0.y; p[2] = a0.z; p[3] = a0.w;
      p[4] = a1.x; p[5] = a1.y; p[6] = a1.z; p[7] = a1.w;
    }
    Op8 bh, bl;
#pragma unroll
    for (int k = 0; k < 8; k += 2) split_bf16(p[k], p[k + 1], bh.u[k / 2], bl.u[k / 2]);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      st.acc[hb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt].v, bh.v, st.acc[hb][mt], 0, 0, 0);
      st.acc[hb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt].v, bl.v, st.acc[hb][mt], 0, 0, 0);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// A flush folded into a decode launch (DecodeArgs::flush_g): waves 0-3 of
// the workgroup that holds the group quantise it from the ring, one quarter
// each (the quantise kernels' per-wave functions: channel halves of the keys,
// token halves of the values), using their own staging areas in LDS, which
// hold nothing yet.  Each then waits for its record stores to complete and
// counts itself in `done`; a wave that loads the group first waits until all
// four have counted (they wait on nothing, so the wait ends).  The ring
// tokens read here are neither the ones this launch attends to nor the slot
// the fused append writes (R >= G), and no other workgroup reads the group.
template <int BITS, int META>
__device__ __forceinline__ void fold_flush(const DecodeArgs &a, int u, int wave, int lane,
                                           uint8_t *stage_area, int *done) {
  QuantizeArgs q{};
  q.src_k = a.k_res;
  q.src_v = a.v_res;
  q.src_unit_stride = (long long)a.slots * D;
  q.src_tok0 = a.flush_src;
  q.dst_g0 = a.flush_g;
  q.n_groups_cap = a.n_groups_cap;
  q.records = const_cast<uint8_t *>(a.records);
  q.kv_heads = a.kv_heads;
  q.pages = a.pages;
  if (wave < 2)
    qgroup::quantize_keys<BITS, META>(q, u, 0, 1, wave, lane, stage_area);
  else
    qgroup::quantize_values<BITS, META>(q, u, 0, 1, wave - 2, lane, stage_area,
                                        reinterpret_cast<uint4 *>(stage_area + 16 * D));
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  if (lane == 0) __hip_atomic_fetch_add(done, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Before loading group g: if it is the folded flush's group, wait for it.
__device__ __forceinline__ void wait_fold(bool owner, int g, int flush_g, const int *done) {
  if (owner && g == flush_g)
    while (__hip_atomic_load(const_cast<int *>(done), __ATOMIC_ACQUIRE,
                             __HIP_MEMORY_SCOPE_WORKGROUP) < 4)
      __builtin_amdgcn_s_sleep(2);
}

// Byte range [lo, hi) of the unit's work for wave `wave` of workgroup
// (u, split): quantised groups cost `cq` units each, then residual chunks of
// G tokens `cr` each; the workgroup's share is weighted by its co-residency
// rank, split evenly over the 4 waves.
//
// Workgroups are dispatched in linear order s*n_units + u, one per compute
// unit per round, so that index / cus is the workgroup's rank among those
// sharing its compute unit.  Older workgroups win the arbitration for the
// memory pipeline, so the byte shares are weighted by rank; the weights are
// integers and every workgroup of a unit derives the same boundaries.
struct WorkRange {
  int g_begin, g_end, r_begin, r_end;
};

__device__ __forceinline__ WorkRange wave_work(const DecodeArgs &a, int u, int split, int wave,
                                               int nw, int cq, int cr) {
  const int n_rc = (a.n_res + G - 1) / G;
  const long long q0 = (long long)a.n_groups * cq, total = q0 + (long long)n_rc * cr;
  long long cum = 0, wsum = 0, wself = 0;
  for (int s = 0; s < a.n_split; ++s) {
    // a select chain, not an indexed load: the kernel's copy of the
    // arguments stays in registers (mixed-length batches rewrite its
    // counters, and an indexed member would move the whole copy to scratch)
    const int rank = (s * a.n_units + u) / a.cus;
    const int w = rank == 0 ? a.rank_w[0] : rank == 1 ? a.rank_w[1] : rank == 2 ? a.rank_w[2] : a.rank_w[3];
    cum += s < split ? w : 0;
    wself = s == split ? w : wself;
    wsum += w;
  }
  const long long wg_lo = total * cum / wsum, wg_hi = total * (cum + wself) / wsum;
  const long long lo = wg_lo + (wg_hi - wg_lo) * wave / nw, hi = wg_lo + (wg_hi - wg_lo) * (wave + 1) / nw;
  WorkRange r;
  r.g_begin = (int)min((lo + cq - 1) / cq, (long long)a.n_groups);
  r.g_end = (int)min((hi + cq - 1) / cq, (long long)a.n_groups);
  r.r_begin = (int)min(max(lo - q0 + cr - 1, 0ll) / cr, (long long)n_rc);
  r.r_end = (int)min(max(hi - q0 + cr - 1, 0ll) / cr, (long long)n_rc);
  return r;
}

// Decode attention, any number of query heads per kv head.  Grid (unit, wpu): the `wpu` workgroups of a unit
// split its work -- the quantised groups, then the residual in chunks of 32
// tokens -- into rank-weighted byte shares (wave_work).  Item costs are in
// KiB: a group (codes + scale/zero) is bits + 2, a residual chunk (32 bf16
// K and V rows) is 16.  NW == 4: each workgroup splits its share over its
// waves statically.  NW > 4 (one workgroup per compute unit): the waves take
// the share's groups one at a time from an LDS counter, so waves that the
// hardware issues less often take fewer groups and all finish together; the
// grouping of the online-softmax sums then depends on timing, so results may
// differ between launches in the last bits.
template <int BITS, int NHB, int META, bool PAGED, int NW, bool FIXED>
__global__ __launch_bounds__(64 * NW) void decode_gqa_kernel(DecodeArgs a) {
  constexpr int HMAX = 4 * NHB;
  // NW > 4: one workgroup per compute unit.  Its groups are handed out to
  // the waves one at a time from the LDS counter s_next (the first
  // kPrefetch + 1 of each wave fixed), or with FIXED round-robin (wave w
  // takes groups w, w + NW, ...), which makes every wave's groups, and so the
  // result, independent of timing.
  constexpr bool kDyn = NW > 4;
  static_assert(!FIXED || kDyn, "fixed round-robin claims are a form of the one-workgroup launch");
  // groups between a wave's consecutive claims
  constexpr int kClaimStride = FIXED ? NW : 1;
  // The merge buffer: with one workgroup per compute unit (NW > 4) there is
  // room for it beside the staging areas, and each wave writes its totals as
  // soon as it is done; with several workgroups per compute unit (NW == 4) it
  // aliases the staging areas, and the waves first wait for each other.
  struct Apart {
    MfmaSmem<NHB, NW> mf;
    MergeSmem<HMAX, NW> mg;
  };
  union Shared {
    MfmaSmem<NHB, NW> mf;
    MergeSmem<HMAX, NW> mg;
  };
  __shared__ __align__(16) std::conditional_t<kDyn, Apart, Shared> sm;
  constexpr int C = kPrefetch + 1;
  __shared__ int s_next;   // kDyn: the next group to hand out

  const int u = blockIdx.x, split = blockIdx.y;
  const int4 next_state = a.state_in ? apply_unit_state(a, u) : make_int4(0, 0, 0, 0);
  // wave index made visibly wave-uniform so that group offsets live in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, gq = lane >> 4;          // MFMA column / row, lane group
  const int ch = lane & 3, cm = (lane >> 2) & 3;    // cooperative q' role: head, step
  const int qpk = a.qpk;
  const int b = u / a.kv_heads, h = u % a.kv_heads;

  // this wave's byte share of the unit, and the items that start inside it
  // (kDyn: the workgroup's share; the waves take its groups dynamically and
  // its residual chunks round-robin, wave w the chunks w, w + NW, ...)
  const WorkRange wr = kDyn ? wave_work(a, u, split, 0, 1, BITS + kMetaBytes<META> / 2, 16)
                            : wave_work(a, u, split, wave, NW, BITS + kMetaBytes<META> / 2, 16);
  // A flush folded into this launch, if this workgroup's share holds its
  // group (workgroup-uniform)
  __shared__ int s_fold;   // quarters of the folded flush done
  bool fold = false;
  if (a.flush_g >= 0) {
    const WorkRange wg = kDyn ? wr : wave_work(a, u, split, 0, 1, BITS + kMetaBytes<META> / 2, 16);
    fold = a.flush_g >= wg.g_begin && a.flush_g < wg.g_end;
  }
  if (fold) {
    if (threadIdx.x == 0) s_fold = 0;
    __syncthreads();
    if (wave < 4)
      fold_flush<BITS, META>(a, u, wave, lane, reinterpret_cast<uint8_t *>(&sm.mf.w[wave]), &s_fold);
  }
  const int g_end = wr.g_end;
  const int g_begin = kDyn ? wr.g_begin + wave * (FIXED ? 1 : C) : wr.g_begin;
  const int r_begin = kDyn ? wr.r_begin + wave : wr.r_begin;
  const int r_end = wr.r_end;
  constexpr int r_step = kDyn ? NW : 1;

  // Order of the first loads: the query (needed first), then the first
  // groups, so that waiting for the query does not wait for the groups.
  uint4 qraw[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int hh = hb * 4 + ch;
    qraw[hb] = make_uint4(0u, 0u, 0u, 0u);
    if (hh < qpk)
      qraw[hb] = *reinterpret_cast<const uint4 *>(
          a.q + ((long long)b * a.kv_heads * qpk + (long long)h * qpk + hh) * D + 32 * gq + 8 * cm);
  }
  WaveState<NHB> st;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) st.acc[hb][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.m_run[hb] = kNegInf; st.l_run[hb] = 0.f; st.z_run[hb] = 0.f; st.m_ref[hb] = 0.f;
  }
  const RecView view = make_rec_view<BITS, META, PAGED>(a, u, lane);
  // register sets of the load pipeline: kPrefetch groups in flight
  GroupRaw<BITS> r[kPrefetch + 1];
#pragma unroll
  for (int i = 0; i < kPrefetch; ++i) {
    const int g = g_begin + i * kClaimStride;
    wait_fold(fold, g, a.flush_g, &s_fold);
    load_group<BITS, META, PAGED>(r[i], view, a, u, g, g < g_end);
    // keep the groups' loads in group order, as in the loop, so that the
    // wait counts at the loop head are the steady-state ones
    __builtin_amdgcn_sched_barrier(0);
  }

  // scaled query values in slot order for the cooperative role
  float qv[NHB][8];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const uint32_t w[4] = {qraw[hb].x, qraw[hb].y, qraw[hb].z, qraw[hb].w};
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) qv[hb][s] = x[P8[s]] * a.qscale;
  }


  // the buffer set that holds the q' operand and beta of the group between
  // prep_group and attend_group
  int buf = 0;
  if constexpr (kDyn) {
    if (threadIdx.x == 0) s_next = wr.g_begin + NW * C;
    __syncthreads();
    // gk[k]: the group in register set k; the wave's groups are its fixed
    // ones, then one claimed per step, claimed a step before it is loaded
    int gk[C];
#pragma unroll
    for (int k = 0; k < C; ++k) gk[k] = g_begin + k * kClaimStride;
    int to_load = g_begin + kPrefetch * kClaimStride;   // loaded at the next step
    int claim = g_begin + (kPrefetch + 1) * kClaimStride;
    if (!FIXED && lane == 0)
      claim = __hip_atomic_fetch_add(&s_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // the first group's prep; each step then preps the wave's next group
    // (in register set k + 1) while it attends to the current one
    prep_group<NHB, META, NW>(r[0].mw, sm.mf, 0, qv, wave, lane, gq, ch, cm);
    while (gk[0] < g_end) {
#pragma unroll
      for (int k = 0; k <= kPrefetch; ++k) {
        const int slot = (k + kPrefetch) % (kPrefetch + 1);
        gk[slot] = to_load;
        wait_fold(fold, to_load, a.flush_g, &s_fold);
        load_group<BITS, META, PAGED>(r[slot], view, a, u, to_load, to_load < g_end);
        if constexpr (FIXED) {
          to_load = claim;
          claim += NW;
        } else {
          to_load = __builtin_amdgcn_readfirstlane(claim);
          if (lane == 0)
            claim = __hip_atomic_fetch_add(&s_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        // issue priority from the live groups still in this wave's register
        // sets: the same for all waves while groups remain to be claimed; at
        // the end the waves with more left are served first, so that the
        // waves of a SIMD finish together instead of the oldest first (the
        // default tie-break)
        {
          int left = 0;
#pragma unroll
          for (int i = 0; i < C; ++i) left += gk[i] < g_end ? 1 : 0;
          if (left == C) __builtin_amdgcn_s_setprio(3);
          else if (left == C - 1) __builtin_amdgcn_s_setprio(2);
          else __builtin_amdgcn_s_setprio(1);
        }
        if (gk[k] < g_end) {
          attend_group<BITS, NHB, NW>(r[k], st, sm.mf, buf, wave, lane, [&] {
            prep_group<NHB, META, NW>(r[(k + 1) % (kPrefetch + 1)].mw, sm.mf, buf ^ 1, qv,
                                      wave, lane, gq, ch, cm);
          });
          buf ^= 1;
        }
      }
    }
  } else {
  // quantised groups: software pipeline over kPrefetch + 1 register sets
  // (unrolled, so the sets rotate without copies), the next kPrefetch groups
  // in flight while the current one is computed
  // Every pass issues the loads of kPrefetch + 1 groups, so that the
  // outstanding loads at the loop head are the same from either edge; the
  // last pass skips the groups past the end (a wave-uniform branch).
  prep_group<NHB, META, NW>(r[0].mw, sm.mf, 0, qv, wave, lane, gq, ch, cm);
  for (int g0 = g_begin; g0 < g_end; g0 += kPrefetch + 1) {
#pragma unroll
    for (int k = 0; k <= kPrefetch; ++k) {
      const int g = g0 + k;
      wait_fold(fold, g + kPrefetch, a.flush_g, &s_fold);
      load_group<BITS, META, PAGED>(r[(k + kPrefetch) % (kPrefetch + 1)], view, a, u,
                                    g + kPrefetch, g + kPrefetch < g_end);
      if (g < g_end) {
        attend_group<BITS, NHB, NW>(r[k], st, sm.mf, buf, wave, lane, [&] {
          prep_group<NHB, META, NW>(r[(k + 1) % (kPrefetch + 1)].mw, sm.mf, buf ^ 1, qv,
                                    wave, lane, gq, ch, cm);
        });
        buf ^= 1;
      }
    }
  }
  }
  // residual chunks
  for (int rc = r_begin; rc < r_end; rc += r_step)
    mfma_rchunk<NHB, NW>(a, u, rc, st, sm.mf, wave, lane, n, gq);

  // ---- per-wave totals, then the workgroup merge
  if constexpr (!kDyn) __syncthreads();
  const int jv = n >> 2, hv = n & 3;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const float l = row_sum16(st.l_run[hb]);                // score lanes: head gq
    const float z = sum_x32(sum_x16(st.z_run[hb]));         // P.V lanes: column n
    // lane (n, gq) holds rows 4gq + r of M-tile mt = channel 32gq + 8r + mt,
    // for column n = 4j + head; the column is useful when j == gq.
    if (jv == gq) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float o8[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) o8[mt] = st.acc[hb][mt][r] + z;
        float *dst = &sm.mg.o[wave][hb * 4 + hv][32 * gq + 8 * r];
        *reinterpret_cast<float4 *>(dst) = make_float4(o8[0], o8[1], o8[2], o8[3]);
        *reinterpret_cast<float4 *>(dst + 4) = make_float4(o8[4], o8[5], o8[6], o8[7]);
      }
    }
    if (n == 0) {
      sm.mg.m[wave][hb * 4 + gq] = st.m_run[hb];
      sm.mg.l[wave][hb * 4 + gq] = l;
    }
  }
  merge_and_store<HMAX, NW>(sm.mg, a, u, split, next_state);
  if (a.n_split > 1) finish_unit<64 * NW>(a, u, &sm.mg.last, next_state);
}

}  // namespace

namespace {

// Kernel variants, for each bit width and scale/zero format: 1-4 with 4, 8,
// 12 or 16 query-head columns per kv head (4 waves per workgroup, static
// shares); 5 up to 4 heads, one large workgroup per compute unit whose waves
// take groups dynamically (three waves per SIMD, 12 per workgroup, except
// 4-bit with fp32 scale/zero: 8).  The register allocator fits every
// variant into the 168 VGPRs of three waves per SIMD; at 4-bit with fp32
// scale/zero two waves per SIMD measured 0.6-0.9 us faster on the 8K and
// 32K GQA workloads, with 16-bit scale/zero three were 1.5 us faster.
// One query head per kv head (MHA) runs in the 4-column
// kernels with the other three columns idle: the matrix core has the time to
// spare, and its unpack-once path needs fewer vector instructions per group
// than fp32 FMAs would.
constexpr int kDynVariant = 5;
// 6: the same launch with fixed round-robin claims (bitwise repeatable).
// 8K GQA on one MI355X: 30.5-30.9 us per launch, against 29.3-30.0 us for 5
// and 33.5-34.2 us for 1 with its three-per-CU round.
constexpr int kDynFixedVariant = 6;
template <int BITS, int META>
constexpr int kDynWaves = BITS == 2 || META == 1 ? 12 : 8;
int variant_waves(int bits, int meta, int variant) {
  if (variant != kDynVariant && variant != kDynFixedVariant) return 4;
  return bits == 2 || meta == 1 ? 12 : 8;
}

template <int BITS, int META, bool PAGED>
void *kernel_fn_t(int variant) {
  switch (variant) {
    case 1: return (void *)&decode_gqa_kernel<BITS, 1, META, PAGED, 4, false>;
    case kDynVariant:
      return (void *)&decode_gqa_kernel<BITS, 1, META, PAGED, kDynWaves<BITS, META>, false>;
    case kDynFixedVariant:
      return (void *)&decode_gqa_kernel<BITS, 1, META, PAGED, kDynWaves<BITS, META>, true>;
    case 2: return (void *)&decode_gqa_kernel<BITS, 2, META, PAGED, 4, false>;
    case 3: return (void *)&decode_gqa_kernel<BITS, 3, META, PAGED, 4, false>;
    default: return (void *)&decode_gqa_kernel<BITS, 4, META, PAGED, 4, false>;
  }
}

template <bool PAGED>
void *kernel_fn_p(int bits, int meta, int variant) {
  if (bits == 2)
    return meta == 1 ? kernel_fn_t<2, 1, PAGED>(variant) : kernel_fn_t<2, 0, PAGED>(variant);
  return meta == 1 ? kernel_fn_t<4, 1, PAGED>(variant) : kernel_fn_t<4, 0, PAGED>(variant);
}
void *kernel_fn(int bits, int meta, int variant, bool paged) {
  return paged ? kernel_fn_p<true>(bits, meta, variant) : kernel_fn_p<false>(bits, meta, variant);
}

// Occupancy of a kernel variant on the current device: resident workgroups
// per compute unit and the number of compute units, cached per device and
// variant.
struct Residency {
  int per_cu, cus;
};

Residency residency(int bits, int meta, int variant, bool paged) {
  static int cache[16][2][2][2][7][2];   // 0 = not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int *slot = cache[dev & 15][bits == 4 ? 1 : 0][meta == 1 ? 1 : 0][paged ? 1 : 0][variant];
  Residency r{__atomic_load_n(&slot[0], __ATOMIC_RELAXED), __atomic_load_n(&slot[1], __ATOMIC_RELAXED)};
  if (r.per_cu > 0 && r.cus > 0) return r;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&r.per_cu, kernel_fn(bits, meta, variant, paged),
                                                   64 * variant_waves(bits, meta, variant),
                                                   0) != hipSuccess ||
      r.per_cu < 1)
    r.per_cu = 1;
  if (hipDeviceGetAttribute(&r.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || r.cus < 1)
    r.cus = 256;
  __atomic_store_n(&slot[0], r.per_cu, __ATOMIC_RELAXED);
  __atomic_store_n(&slot[1], r.cus, __ATOMIC_RELAXED);
  return r;
}

// Byte-share weights of co-resident ranks 0..3 (oldest first).  Measured on
// MI355X at the 8K GQA workload (2-bit, three workgroups per compute unit)
// with equal shares, the ranks finish their loops at about 19, 24 and 30 us;
// the defaults come from a sweep of the launch time there and at the 32K
// 4-bit workload (two per compute unit).  KIVI_RANK_WEIGHTS="w0,w1,w2,w3"
// (positive integers) overrides them, for sweeps; like every tuning variable
// of the library it is read once per process, at the first launch.
struct RankOverride {
  int n = 0;
  int w[4] = {0, 0, 0, 0};
};
RankOverride read_rank_override() {
  RankOverride r;
  if (const char *env = getenv("KIVI_RANK_WEIGHTS")) {
    int v[4];
    const int n = sscanf(env, "%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3]);
    for (int i = 0; i < n && i < 4; ++i)
      if (v[i] > 0 && v[i] <= 10000) r.w[r.n++] = v[i];
      else break;
  }
  return r;
}
void rank_weights(int per_cu, int (&w)[4]) {
  static const int k3[4] = {100, 75, 55, 55};
  static const int k2[4] = {100, 70, 70, 70};
  static const RankOverride ov = read_rank_override();   // once per process
  const int *src = per_cu == 3 ? k3 : per_cu == 2 ? k2 : nullptr;
  for (int i = 0; i < 4; ++i) w[i] = src ? src[i] : 100;
  for (int i = 0; i < 4 && ov.n > 0; ++i) w[i] = ov.w[i < ov.n ? i : ov.n - 1];
}

// Workgroups per unit.  Cost model in the work units of wave_work (KiB):
// a workgroup that takes K/w of a unit's cost K also pays a fixed kWgFixed
// (prologue loads, merge, partial stores, arrival count).  When all U*w
// workgroups are resident at once the launch takes one workgroup time;
// beyond that the dispatcher refills freed slots, and the launch takes about
// (U*w/slots + 1/2) workgroup times (half a workgroup of tail).  The count
// is capped so that every wave has at least two groups' worth of bytes and
// the workspace holds the partials.  MI355X sweeps: 6 per unit at the 8K GQA
// workload (one round), 1-2 at the 13B-shaped MHA memory wall (batch
// 64-316, many rounds).  KIVI_WPU fixes the count (sweeps; read once per
// process).
int choose_wpu(int group_cost, const DecodeArgs &a, int slots) {
  constexpr double kWgFixed = 40.0;
  const long long n_rc = (a.n_res + G - 1) / G;
  const long long total = (long long)a.n_groups * group_cost + n_rc * 16;
  // the bound the workspace is sized by (kivi_decode_workspace_bytes), and
  // the workspace's capacity in partials per unit
  long long cap = max_splits_for(a.n_groups, a.n_res, group_cost);
  if (cap > a.n_split) cap = a.n_split;
  static const long long env_wpu = [] {
    const char *env = getenv("KIVI_WPU");
    return env ? atoll(env) : 0ll;
  }();
  if (env_wpu >= 1) return (int)(env_wpu < cap ? env_wpu : cap);
  int best = 1;
  double best_t = 1e300;
  for (int w = 1; w <= cap; ++w) {
    const double rounds = (double)a.n_units * w / slots;
    const double t_wg = (double)total / w + kWgFixed;
    const double t = rounds <= 1.0 ? t_wg : (rounds + 0.5) * t_wg;
    if (t < best_t * 0.999) { best_t = t; best = w; }
  }
  return best;
}

}  // namespace

hipError_t launch_decode(int bits, int meta, const DecodeArgs &a_in, bool deterministic,
                         hipStream_t s) {
  int variant = (a_in.qpk + 3) / 4;   // 1..4
  DecodeArgs a = a_in;
  const bool paged = a_in.pages.table != nullptr;
  // Up to 4 query heads per kv head and at most one unit per compute unit:
  // the launch is a single round, whose end the slowest wave sets, so the
  // dynamic variant (one workgroup per compute unit, waves balanced by an
  // LDS counter) is used; a caller that asked for bitwise-repeatable results
  // gets the same launch with fixed round-robin claims (the counter's order
  // depends on timing).  Longer launches refill their slots as workgroups
  // finish and keep the static variant.
  if (variant == 1) {
    const int dyn = deterministic ? kDynFixedVariant : kDynVariant;
    const Residency rd = residency(bits, meta, dyn, paged);
    if ((long long)a_in.n_units <= (long long)rd.per_cu * rd.cus) variant = dyn;
  }
  const Residency res = residency(bits, meta, variant, paged);
  const int slots = res.per_cu * res.cus;
  // KiB per group: codes (bits) + scale/zero (2 fp32 or 1 16-bit)
  const int group_cost = bits + (meta == 1 ? 1 : 2);
  a.n_split = choose_wpu(group_cost, a_in, slots);   // a_in.n_split: capacity
  a.cus = res.cus;
  // rank weights only mean something when every workgroup is resident at once
  if ((long long)a.n_split * a.n_units <= slots) {
    rank_weights(res.per_cu, a.rank_w);
  } else {
    for (int i = 0; i < 4; ++i) a.rank_w[i] = 1;
  }
  const dim3 grid(a.n_units, a.n_split), block(64 * variant_waves(bits, meta, variant));
  hipLaunchKernelGGL(reinterpret_cast<void (*)(DecodeArgs)>(kernel_fn(bits, meta, variant, paged)), grid,
                     block, 0, s, a);
  return hipGetLastError();
}

}  // namespace kivi
