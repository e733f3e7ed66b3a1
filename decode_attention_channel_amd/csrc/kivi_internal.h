// kivi_internal.h -- declarations shared by the translation units of
// libkivi.so (host API, quantise kernels, decode kernels).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kivi.h"

namespace kivi {

constexpr int kHeadDim = 128;      // supported head_dim
constexpr int kGroup = 32;         // supported group size G
constexpr int kPartStride = 132;   // floats per split partial: m, l, pad, pad, o[128]
constexpr int kMaxSplits = 256;    // workgroups per unit of one decode launch, at most

// Largest byte range of one unit's group records (its NG records).  The
// decode kernel's out-of-range load offset (2^31) relies on it; the host
// refuses geometries beyond it.
constexpr long long kMaxUnitRecordBytes = 1ll << 30;

// Upper bound on the workgroups (split partials) per unit of a decode launch
// over n_groups quantised groups and n_res residual tokens, in the cost units
// of the launcher (KiB: a group costs group_cost, a residual chunk of 32
// tokens 16): every wave keeps at least two groups' worth of work.  The
// workspace is sized by this bound and the launcher never exceeds it.
__host__ __device__ inline int max_splits_for(long long n_groups, long long n_res,
                                              int group_cost) {
  const long long total = n_groups * group_cost + (n_res + 31) / 32 * 16;
  long long cap = total / (4 * 2 * group_cost);
  if (cap < 1) cap = 1;
  if (cap > kMaxSplits) cap = kMaxSplits;
  return (int)cap;
}

// Per-sequence state of a mixed-length batch (device memory): int32
// {n_q, n_res, res_start, flags} per sequence.  Flag bits (kivi.h):
constexpr int kSeqBadLength = 1;   // KIVI_SEQ_BAD_LENGTH
constexpr int kSeqFull = 2;        // KIVI_SEQ_FULL

// A state row that the mixed-length calls can have written: whole groups of
// history within capacity, a ring that is not yet full, a ring start on a
// group boundary, known flags.  Anything else is taken as a bad sequence, so
// that no launch indexes the cache with it.
__host__ __device__ inline bool state_ok(int n_q, int n_res, int res_start, int flags, int G,
                                         int slots, int T) {
  return n_q >= 0 && n_q <= T && n_q % G == 0 && n_res >= 0 && n_res < slots &&
         res_start >= 0 && res_start < slots && res_start % G == 0 && (flags & ~3) == 0;
}

// Prefill split of a sequence of S tokens (see kivi.h): false when S is out
// of [1, stride] or the quantised part does not fit T tokens.
__host__ __device__ inline bool seq_split(int S, int stride, int G, int R, int T, int &n_q,
                                          int &r) {
  n_q = 0;
  r = 0;
  if (S < 1 || S > stride) return false;
  n_q = S > R ? G * ((S - R) / G) : 0;
  r = S - n_q;
  return n_q <= T;
}

// Paged quantised history.  With table == nullptr every unit owns one
// contiguous block of n_groups_cap groups in each group-major array (group
// slot u * NG + g).  Otherwise the arrays are pools of pages; a page holds
// 2^shift consecutive groups of every kv head of one sequence, and group g of
// unit (b, h) has slot (table[b][g >> shift] * H + h) * 2^shift + g % 2^shift.
// Page entries outside [0, num_pages) map nothing.
struct PageMap {
  const int32_t *table;   // [B][max_pages]
  int shift, max_pages, num_pages;
};

// Group slot of group g of unit u (the multiplier of a group's bytes in the
// group-major arrays), or -1 when a paged unit has no page for it.
__host__ __device__ inline long long group_slot(const PageMap &p, int kv_heads, int n_groups_cap,
                                                int u, int g) {
  if (!p.table) return (long long)u * n_groups_cap + g;
  const int pi = g >> p.shift;
  if (g < 0 || pi >= p.max_pages) return -1;
  const int b = u / kv_heads, h = u % kv_heads;
  const int e = p.table[(long long)b * p.max_pages + pi];
  if (e < 0 || e >= p.num_pages) return -1;
  return (((long long)e * kv_heads + h) << p.shift) + (g & ((1 << p.shift) - 1));
}

// Group records (kivi.h): the quantised history of one group is one
// contiguous record of rec_planes() planes of 1 KiB; plane p holds 16 bytes
// for each lane l (0..63) of the decode wave at p * 1024 + 16 * l:
//   planes [0, b/2)      K codes: lane 16 j + 4 (t >> 3) + (t & 3) holds
//                        the 32-channel block j of token rows t and t + 4,
//                        (t >> 2) & 1 = 0 (2-bit: 8 bytes each in one plane;
//                        4-bit: one plane each)
//   planes [b/2, b)      V codes: lane 16 o + (c >> 3) holds channels
//                        8 (c >> 3) .. + 7 of octet o (b bytes per channel)
//   planes [b, b + 2)    fp32 scale/zero: values 2l, 2l + 1 of k_scale,
//                        k_zero (plane b) and v_scale, v_zero (plane b + 1)
//   plane b              16-bit scale/zero: value pairs 2l, 2l + 1 of
//                        k_scale, k_zero, v_scale, v_zero
// Each piece holds the bytes of the per-array layout (kivi.h), so a record
// is a fixed permutation of those bytes.
constexpr int kPlaneBytes = 1024;
__host__ __device__ constexpr int rec_planes(int bits, int meta) {
  return bits + (meta == 1 ? 1 : 2);
}
__host__ __device__ constexpr int rec_bytes(int bits, int meta) {
  return rec_planes(bits, meta) * kPlaneBytes;
}

// Copy `n_rows` bf16 rows of D channels per unit (K and V) from
// src + u*src_unit_stride + (src_tok0 + i)*D to dst + u*dst_unit_stride +
// (dst_row0 + i)*D.
struct CopyRowsArgs {
  const uint16_t *src_k, *src_v;
  long long src_unit_stride;
  int src_tok0;
  uint16_t *dst_k, *dst_v;
  long long dst_unit_stride;
  int dst_row0;
  int n_rows, n_units;
};
hipError_t launch_copy_rows(const CopyRowsArgs &a, hipStream_t s);

// One launch of the group quantiser: `n_groups` groups of G tokens for each
// of `n_units` units.  Source token i of local group gl of unit u is row
// (src_tok0 + gl*G + i) of a [rows][D] bf16 block starting at
// src + u*src_unit_stride.  Destination group is dst_g0 + gl.
struct QuantizeArgs {
  const uint16_t *src_k, *src_v;
  long long src_unit_stride;   // elements
  int src_tok0;
  int n_groups, n_units;
  int dst_g0;
  int max_tokens, n_groups_cap;  // T, NG
  uint8_t *records;   // group records
  int gpw;   // groups per workgroup (set by the launcher)
  // Mixed-length batches (null otherwise).  seq_lens (prefill): sequence b
  // quantises its own n_q tokens, n_groups being the largest count.  state
  // (flush): sequence b flushes iff its ring will be full after this step's
  // append, from its own ring start into its own next group.
  const int32_t *seq_lens, *state;
  int kv_heads, residual, slots, stride;
  PageMap pages;   // destination group slots (group_slot)
  // Prefill: residual rows copied by extra workgroups of the same launch
  // (res.n_rows 0: none); its unit count and source are those above.
  CopyRowsArgs res;
};
hipError_t launch_quantize(int bits, int meta, const QuantizeArgs &a, hipStream_t s);

// Mixed-length prefill: copy each sequence's residual tokens into ring slots
// 0.. and write its state.
struct RaggedResidualArgs {
  const uint16_t *src_k, *src_v;   // [B][H][stride][D]
  uint16_t *dst_k, *dst_v;         // [B][H][slots][D]
  const int32_t *seq_lens;         // [B]
  int32_t *state;                  // [B][4]
  int n_units, kv_heads, stride, group, residual, slots, max_tokens;
  PageMap pages;                   // a sequence whose history lacks a page is bad
};
hipError_t launch_ragged_residual(const RaggedResidualArgs &a, hipStream_t s);

struct DecodeArgs {
  const uint8_t *records;    // group records
  uint16_t *k_res, *v_res;   // written only for the fused append below
  // Fused append: logical residual token new_idx (-1: none) is taken from
  // k_new / v_new ([units][D] bf16) instead of the ring, and the one wave
  // that reads it also stores it into its ring slot.
  const uint16_t *k_new, *v_new;
  int new_idx;
  const uint16_t *q;
  unsigned *counters; // [units] arrival counters, zero between calls
  float *part;        // [units][n_split][QPK][kPartStride]
  float *out;         // [B][Hq][D]
  float qscale;       // softmax_scale * log2(e): scores come out in log2 units
  int kv_heads, qpk, max_tokens, n_groups_cap, slots;
  int n_units;
  int n_groups;       // quantised groups in the cache (n_q / G)
  int n_res, res_start;
  int n_split;        // workgroups per unit (the host passes the workspace capacity,
                      // at most kMaxSplits)
  // Mixed-length batches: with state_in set the counters above are upper
  // bounds (for the launch shape) and each sequence reads its own {n_q, n_res,
  // res_start, flags} from state_in, applies this step's flush (done by the
  // launch before) and the fused append, and the combining workgroup of kv
  // head 0 writes the result to state_out.
  const int32_t *state_in;
  int32_t *state_out;
  // paged history (table == nullptr: contiguous per unit); with pages, a
  // flush also needs a page for the new group
  PageMap pages;
  // A flush folded into this launch (flush_g -1: none): group flush_g of the
  // unit is quantised from the G ring tokens that start at slot flush_src,
  // by four waves of the workgroup whose share holds that group, before any
  // of its waves loads it.  Mixed-length batches set it per sequence
  // (from state_in); the counters above already include the flush.
  int flush_g, flush_src;
  // byte shares: workgroup (unit u, split s) has linear index s*n_units+u
  // and co-residency rank min(index / cus, 3) on its compute unit; its share
  // of the unit's bytes is proportional to rank_w[rank]
  int cus;
  int rank_w[4];
};
// deterministic: keep to the static launch variant, whose results are
// bitwise repeatable for the same inputs on the same device.
hipError_t launch_decode(int bits, int meta, const DecodeArgs &a, bool deterministic,
                         hipStream_t s);

}  // namespace kivi
