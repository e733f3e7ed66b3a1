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
constexpr int kMinGroupsPerSplit = 4;   // sizes the workspace: NG/4 + 1 partials per unit

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
  uint8_t *k_codes; void *k_scale, *k_zero;   // fp32, or fp16 / bf16 bits (meta)
  uint8_t *v_codes; void *v_scale, *v_zero;
  int gpw;   // groups per workgroup (set by the launcher)
};
hipError_t launch_quantize(int bits, int meta, const QuantizeArgs &a, hipStream_t s);

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

struct DecodeArgs {
  const uint8_t *k_codes; const void *k_scale, *k_zero;   // fp32, or fp16 / bf16 bits
  const uint8_t *v_codes; const void *v_scale, *v_zero;
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
  int n_split;        // workgroups per unit (the host passes the workspace capacity)
  // byte shares: workgroup (unit u, split s) has linear index s*n_units+u
  // and co-residency rank min(index / cus, 3) on its compute unit; its share
  // of the unit's bytes is proportional to rank_w[rank]
  int cus;
  int rank_w[4];
};
hipError_t launch_decode(int bits, int meta, const DecodeArgs &a, hipStream_t s);

}  // namespace kivi
