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
#include "quantize_group.h"

namespace kivi {
namespace {

using namespace qgroup;

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
