// kivi_api.hip -- the C ABI of libkivi.so (declared in include/kivi.h).
//
// Everything here runs on the host: argument validation (always before any
// HIP call, so that an error enqueues nothing and leaves the cache counters
// unchanged), buffer-size arithmetic, the choice of split-K partition for
// decode attention, and the kernel launches.  The method steps themselves
// are in quantize.hip (per-channel K / per-token V group quantiser, catalog
// record kivi-2bit-llama3-8b-gqa-8k "KV bytes basis" residual handling) and
// decode_attn.hip (decode attention over the mixed cache).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "kivi_internal.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

kivi_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KIVI_OK;
  g_last_hip_error = (int32_t)e;
  return KIVI_E_HIP;
}

kivi_status check_geom(const kivi_geom *g) {
  if (!g) return KIVI_E_NULL;
  if (g->batch <= 0 || g->kv_heads <= 0 || g->q_per_kv <= 0 || g->head_dim <= 0 ||
      g->bits <= 0 || g->group <= 0 || g->residual < 0 || g->max_tokens < 0)
    return KIVI_E_GEOMETRY;
  if (g->bits != 2 && g->bits != 4) return KIVI_E_UNSUPPORTED;
  if (g->meta_format != KIVI_META_FP32 && g->meta_format != KIVI_META_FP16_BF16)
    return KIVI_E_UNSUPPORTED;
  if (g->group != kivi::kGroup || g->head_dim != kivi::kHeadDim) return KIVI_E_UNSUPPORTED;
  if (g->residual % g->group != 0 || g->residual > 4096) return KIVI_E_UNSUPPORTED;
  if (g->q_per_kv > 16) return KIVI_E_UNSUPPORTED;
  if ((long long)g->batch * g->kv_heads > 65535) return KIVI_E_UNSUPPORTED;   // grid.y
  if ((g->flags & ~KIVI_FLAG_DETERMINISTIC) != 0) return KIVI_E_UNSUPPORTED;
  if (g->max_tokens % g->group != 0) return KIVI_E_UNSUPPORTED;
  // a unit's records are addressed with 32-bit offsets, and the decode
  // kernel's not-live offset (2^31) must lie beyond all of them
  if ((long long)(g->max_tokens / g->group) * kivi::rec_bytes(g->bits, g->meta_format) >
      kivi::kMaxUnitRecordBytes)
    return KIVI_E_UNSUPPORTED;
  // keep every byte offset of every buffer inside 2^62
  const double units = (double)g->batch * g->kv_heads;
  if (units * ((double)g->max_tokens + g->residual + g->group) * g->head_dim * 8.0 > 4.0e18)
    return KIVI_E_GEOMETRY;
  return KIVI_OK;
}

kivi_status check_cache(const kivi_geom *, const kivi_cache *c) {
  if (!c) return KIVI_E_NULL;
  if (!c->records || !c->k_res || !c->v_res) return KIVI_E_NULL;
  return KIVI_OK;
}

kivi_status check_state(const kivi_geom *g, const kivi_cache *c) {
  const int slots = g->residual + g->group;
  if (c->n_q < 0 || c->n_q % g->group != 0 || c->n_q > g->max_tokens) return KIVI_E_STATE;
  if (c->n_res < 0 || c->n_res > slots) return KIVI_E_STATE;
  if (c->res_start < 0 || c->res_start >= slots || c->res_start % g->group != 0)
    return KIVI_E_STATE;
  return KIVI_OK;
}

long long units_of(const kivi_geom *g) { return (long long)g->batch * g->kv_heads; }

// decode workspace: one arrival counter per unit (padded to 256 B), then the
// split partials, QPK of kPartStride floats per (unit, split)
size_t counters_bytes(const kivi_geom *g) {
  return ((size_t)units_of(g) * sizeof(unsigned) + 255) / 256 * 256;
}

size_t partial_bytes(const kivi_geom *g) {
  return (size_t)units_of(g) * (size_t)g->q_per_kv * kivi::kPartStride * sizeof(float);
}

// KiB per quantised group in the launcher's cost model: codes (bits) plus
// scale/zero (two fp32 arrays, or one 16-bit pair)
int group_cost(const kivi_geom *g) { return g->bits + (g->meta_format == KIVI_META_FP16_BF16 ? 1 : 2); }

// Workspace for a launch over n_q quantised and n_res residual tokens (the
// caller has validated the geometry).
size_t workspace_need(const kivi_geom *g, long long n_q, long long n_res) {
  return counters_bytes(g) +
         partial_bytes(g) * (size_t)kivi::max_splits_for(n_q / g->group, n_res, group_cost(g));
}

// Split partials per unit that a workspace of ws_bytes holds (the launcher's
// capacity), at most kMaxSplits.
int splits_capacity(const kivi_geom *g, size_t ws_bytes) {
  const size_t n = (ws_bytes - counters_bytes(g)) / partial_bytes(g);
  return n > (size_t)kivi::kMaxSplits ? kivi::kMaxSplits : (int)n;
}

// Quantise the G oldest residual tokens (ring slots res_start..+G-1, which
// are contiguous because res_start is a multiple of G) into group n_q/G and
// advance the counters.  The caller has validated everything.
kivi_status enqueue_flush(const kivi_geom *g, kivi_cache *c, hipStream_t s) {
  const int G = g->group, slots = g->residual + G;
  kivi::QuantizeArgs a{};
  a.src_k = c->k_res; a.src_v = c->v_res;
  a.src_unit_stride = (long long)slots * g->head_dim;
  a.src_tok0 = c->res_start;
  a.n_groups = 1; a.n_units = (int)units_of(g); a.dst_g0 = c->n_q / G;
  a.max_tokens = g->max_tokens; a.n_groups_cap = g->max_tokens / G;
  a.records = c->records;
  kivi_status st = hip_status(kivi::launch_quantize(g->bits, g->meta_format, a, s));
  if (st != KIVI_OK) return st;
  c->n_q += G;
  c->n_res -= G;
  c->res_start = (c->res_start + G) % slots;
  return KIVI_OK;
}

// Copy one token per unit into ring slot (res_start + n_res) mod (R+G).
kivi_status enqueue_append(const kivi_geom *g, kivi_cache *c, const uint16_t *k_new,
                           const uint16_t *v_new, hipStream_t s) {
  const int slots = g->residual + g->group;
  kivi::CopyRowsArgs a{};
  a.src_k = k_new; a.src_v = v_new;
  a.src_unit_stride = g->head_dim;
  a.src_tok0 = 0;
  a.dst_k = c->k_res; a.dst_v = c->v_res;
  a.dst_unit_stride = (long long)slots * g->head_dim;
  a.dst_row0 = (c->res_start + c->n_res) % slots;
  a.n_rows = 1; a.n_units = (int)units_of(g);
  kivi_status st = hip_status(kivi::launch_copy_rows(a, s));
  if (st != KIVI_OK) return st;
  c->n_res += 1;
  return KIVI_OK;
}

// Validation shared by the decode-attention calls: the launch will attend
// over (at most) n_q quantised and n_res residual tokens.
kivi_status check_attend_args(const kivi_geom *g, long long n_q, long long n_res,
                              const uint16_t *q, const float *out, float softmax_scale,
                              const void *ws, size_t ws_bytes) {
  if (!q || !out) return KIVI_E_NULL;
  if (!ws || ws_bytes < workspace_need(g, n_q, n_res)) return KIVI_E_WORKSPACE;
  if (!isfinite(softmax_scale)) return KIVI_E_GEOMETRY;
  return KIVI_OK;
}

// Launch decode attention over the cache state in `c`.  With k_new/v_new
// set, logical residual token c->n_res - 1 is read from them (and stored
// into its ring slot by the kernel) instead of from the ring.
kivi_status enqueue_attend(const kivi_geom *g, const kivi_cache *c, const uint16_t *k_new,
                           const uint16_t *v_new, const uint16_t *q, float *out,
                           float softmax_scale, void *ws, size_t ws_bytes, hipStream_t s,
                           int slots = 0,
                           const int32_t *state_in = nullptr, int32_t *state_out = nullptr,
                           const kivi::PageMap &pages = kivi::PageMap{}, int flush_g = -1,
                           int flush_src = 0) {
  kivi::DecodeArgs a{};
  a.pages = pages;
  a.flush_g = flush_g;
  a.flush_src = flush_src;
  a.records = c->records;
  a.k_res = c->k_res; a.v_res = c->v_res;
  a.k_new = k_new; a.v_new = v_new;
  a.new_idx = k_new ? c->n_res - 1 : -1;
  a.q = q; a.out = out;
  a.counters = (unsigned *)ws;
  a.part = (float *)((char *)ws + counters_bytes(g));
  a.qscale = softmax_scale * 1.4426950408889634f;
  a.kv_heads = g->kv_heads; a.qpk = g->q_per_kv; a.max_tokens = g->max_tokens;
  a.n_groups_cap = g->max_tokens / g->group;
  a.slots = slots > 0 ? slots : g->residual + g->group;
  a.n_units = (int)units_of(g);
  a.n_groups = c->n_q / g->group;
  a.n_res = c->n_res; a.res_start = c->res_start;
  a.state_in = state_in; a.state_out = state_out;
  // the launcher picks the workgroups per unit; pass the workspace capacity
  a.n_split = splits_capacity(g, ws_bytes);
  return hip_status(kivi::launch_decode(g->bits, g->meta_format, a,
                                        (g->flags & KIVI_FLAG_DETERMINISTIC) != 0, s));
}

// Arrival counters and split partials of kivi_decode_step_noalloc, for
// callers that cannot allocate (graph capture, tight serving loops,
// harnesses that forbid allocation).  Each device that runs the call holds
// its own copy of this array until the process ends.  In host code the
// array's name is only a host-side handle: its device address comes from
// hipGetSymbolAddress (static_scratch), per device.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
// the arrival counters that must start at zero: one per (sequence, kv head),
// at most 65535 of them
constexpr int kScratchCounterWords = 65536;
static_assert(kScratchCounterWords * 4 <= (int)kScratchBytes, "scratch too small");

__global__ void zero_words_kernel(uint32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device, once known

// Device address of `scratch` on the current device.  The first call on a
// device takes the address (hipGetSymbolAddress, with that device current)
// and zeroes the arrival counters with a small kernel on stream s (a kernel
// rather than a memset, so that a captured call records a kernel node); the
// decode launches return the counters to zero, so later calls reuse them.
kivi_status static_scratch(hipStream_t s, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return KIVI_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    hipLaunchKernelGGL(zero_words_kernel, dim3(kScratchCounterWords / 256), dim3(256), 0, s,
                       static_cast<uint32_t *>(p), kScratchCounterWords);
    if ((e = hipGetLastError()) != hipSuccess) return hip_status(e);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KIVI_OK;
}

// kivi_decode_step; with static_ws the workspace is the `scratch` array of
// the current device instead of (ws, ws_bytes).
kivi_status decode_step_impl(const kivi_geom *g, kivi_cache *c, const uint16_t *k_new,
                             const uint16_t *v_new, const uint16_t *q, float *out,
                             float softmax_scale, void *ws, size_t ws_bytes, int32_t *flushed,
                             hipStream_t s, bool static_ws) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  if ((st = check_cache(g, c)) != KIVI_OK) return st;
  if (!k_new || !v_new) return KIVI_E_NULL;
  if ((st = check_state(g, c)) != KIVI_OK) return st;
  const int G = g->group, slots = g->residual + G;
  if (c->n_res == slots) return KIVI_E_RESIDUAL_FULL;
  const bool flush = c->n_res + 1 == slots;
  if (flush && c->n_q + G > g->max_tokens) return KIVI_E_CAPACITY;
  // the attention runs over the counters after the step
  const long long nq_after = c->n_q + (flush ? G : 0), nres_after = c->n_res + 1 - (flush ? G : 0);
  if (static_ws) {
    if (!q || !out) return KIVI_E_NULL;
    if (!isfinite(softmax_scale)) return KIVI_E_GEOMETRY;
    if (workspace_need(g, nq_after, nres_after) > kScratchBytes) return KIVI_E_WORKSPACE;
    if ((st = static_scratch(s, &ws)) != KIVI_OK) return st;
    ws_bytes = kScratchBytes;
  }
  if ((st = check_attend_args(g, nq_after, nres_after, q, out, softmax_scale, ws, ws_bytes)) !=
      KIVI_OK)
    return st;
  if (flushed) *flushed = 0;

  if (flush && g->residual == 0) {
    // the ring holds exactly one group, which includes the new token: the
    // three steps run as separate launches
    if ((st = enqueue_append(g, c, k_new, v_new, s)) != KIVI_OK) return st;
    if ((st = enqueue_flush(g, c, s)) != KIVI_OK) return st;
    if (flushed) *flushed = 1;
    return enqueue_attend(g, c, nullptr, nullptr, q, out, softmax_scale, ws, ws_bytes, s);
  }
  // With R >= G the G oldest tokens of the full ring exclude the new one (the
  // newest of R+G), so quantising them before the append leaves the same
  // state as append-then-flush: the flush and the append both fold into the
  // attention launch, which quantises the group before any of its waves
  // reads it.
  kivi_cache next = *c;
  int flush_g = -1;
  if (flush) {
    flush_g = c->n_q / G;
    next.n_q += G;
    next.n_res -= G;
    next.res_start = (c->res_start + G) % slots;
  }
  // the new token is logical index n_res of the ring after the flush
  next.n_res += 1;
  if ((st = enqueue_attend(g, &next, k_new, v_new, q, out, softmax_scale, ws, ws_bytes, s, 0,
                           nullptr, nullptr, kivi::PageMap{}, flush_g, c->res_start)) != KIVI_OK)
    return st;
  c->n_q = next.n_q;
  c->n_res = next.n_res;
  c->res_start = next.res_start;
  if (flushed && flush) *flushed = 1;
  return KIVI_OK;
}

}  // namespace

extern "C" {

const char *kivi_status_string(kivi_status s) {
  // A C caller may pass any int; C++ gives an enum object only the values of
  // its enumerators' bit range, so the argument is read as the int it is.
  static_assert(sizeof(kivi_status) == sizeof(int), "kivi_status is int-sized");
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case KIVI_OK: return "ok";
    case KIVI_E_NULL: return "a required pointer is NULL";
    case KIVI_E_GEOMETRY: return "invalid geometry";
    case KIVI_E_UNSUPPORTED: return "geometry outside the supported set";
    case KIVI_E_SEQLEN: return "sequence length must be >= 1";
    case KIVI_E_CAPACITY: return "quantised history would exceed max_tokens";
    case KIVI_E_RESIDUAL_FULL: return "residual ring full: flush first";
    case KIVI_E_WORKSPACE: return "decode workspace NULL or too small";
    case KIVI_E_HIP: return "HIP error (see kivi_last_hip_error)";
    case KIVI_E_STATE: return "cache counters invalid";
  }
  return "unknown status";
}

int32_t kivi_last_hip_error(void) { return g_last_hip_error; }

kivi_status kivi_cache_layout(const kivi_geom *g, size_t bytes[KIVI_NUM_BUFS]) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  if (!bytes) return KIVI_E_NULL;
  const size_t U = (size_t)units_of(g), D = (size_t)g->head_dim;
  const size_t NG = (size_t)(g->max_tokens / g->group);
  const size_t slots = (size_t)(g->residual + g->group);
  bytes[KIVI_BUF_RECORDS] = U * NG * (size_t)kivi::rec_bytes(g->bits, g->meta_format);
  bytes[KIVI_BUF_K_RES] = U * slots * D * 2;
  bytes[KIVI_BUF_V_RES] = U * slots * D * 2;
  return KIVI_OK;
}

size_t kivi_decode_workspace_bytes(const kivi_geom *g, int32_t n_q, int32_t n_res) {
  if (check_geom(g) != KIVI_OK) return 0;
  if (n_q < 0 || n_q > g->max_tokens || n_q % g->group != 0 || n_res < 0) return 0;
  return workspace_need(g, n_q, n_res);
}

kivi_status kivi_quantize_prefill(const kivi_geom *g, kivi_cache *c, const uint16_t *k,
                                  const uint16_t *v, int32_t seq_len, void *stream) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  if ((st = check_cache(g, c)) != KIVI_OK) return st;
  if (!k || !v) return KIVI_E_NULL;
  if (seq_len < 1) return KIVI_E_SEQLEN;
  const int G = g->group, R = g->residual, slots = R + G;
  const int n_q = seq_len > R ? G * ((seq_len - R) / G) : 0;
  const int r = seq_len - n_q;
  if (n_q > g->max_tokens || r > slots) return KIVI_E_CAPACITY;
  hipStream_t s = (hipStream_t)stream;
  const int U = (int)units_of(g);
  // the r residual tokens go to ring slots 0.. (r >= 1 since seq_len >= 1)
  kivi::CopyRowsArgs res{};
  res.src_k = k; res.src_v = v;
  res.src_unit_stride = (long long)seq_len * g->head_dim;
  res.src_tok0 = n_q;
  res.dst_k = c->k_res; res.dst_v = c->v_res;
  res.dst_unit_stride = (long long)slots * g->head_dim;
  res.dst_row0 = 0; res.n_rows = r; res.n_units = U;
  if (n_q > 0) {
    // one launch: the groups, and the residual rows in extra workgroups
    kivi::QuantizeArgs a{};
    a.src_k = k; a.src_v = v;
    a.src_unit_stride = (long long)seq_len * g->head_dim;
    a.src_tok0 = 0;
    a.n_groups = n_q / G; a.n_units = U; a.dst_g0 = 0;
    a.max_tokens = g->max_tokens; a.n_groups_cap = g->max_tokens / G;
    a.records = c->records;
    a.res = res;
    if ((st = hip_status(kivi::launch_quantize(g->bits, g->meta_format, a, s))) != KIVI_OK) return st;
  } else if ((st = hip_status(kivi::launch_copy_rows(res, s))) != KIVI_OK) {
    return st;
  }
  c->n_q = n_q;
  c->n_res = r;
  c->res_start = 0;
  return KIVI_OK;
}

kivi_status kivi_append_token(const kivi_geom *g, kivi_cache *c, const uint16_t *k_new,
                              const uint16_t *v_new, void *stream) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  if ((st = check_cache(g, c)) != KIVI_OK) return st;
  if (!k_new || !v_new) return KIVI_E_NULL;
  if ((st = check_state(g, c)) != KIVI_OK) return st;
  if (c->n_res == g->residual + g->group) return KIVI_E_RESIDUAL_FULL;
  return enqueue_append(g, c, k_new, v_new, (hipStream_t)stream);
}

kivi_status kivi_flush_residual(const kivi_geom *g, kivi_cache *c, int32_t *flushed,
                                void *stream) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  if ((st = check_cache(g, c)) != KIVI_OK) return st;
  if ((st = check_state(g, c)) != KIVI_OK) return st;
  const int G = g->group, slots = g->residual + G;
  if (flushed) *flushed = 0;
  if (c->n_res != slots) return KIVI_OK;
  if (c->n_q + G > g->max_tokens) return KIVI_E_CAPACITY;
  if ((st = enqueue_flush(g, c, (hipStream_t)stream)) != KIVI_OK) return st;
  if (flushed) *flushed = 1;
  return KIVI_OK;
}

kivi_status kivi_decode_attention(const kivi_geom *g, const kivi_cache *c, const uint16_t *q,
                                  float *out, float softmax_scale, void *ws, size_t ws_bytes,
                                  void *stream) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  if ((st = check_cache(g, c)) != KIVI_OK) return st;
  if ((st = check_state(g, c)) != KIVI_OK) return st;
  if ((st = check_attend_args(g, c->n_q, c->n_res, q, out, softmax_scale, ws, ws_bytes)) != KIVI_OK)
    return st;
  if (c->n_q + c->n_res == 0) return KIVI_E_STATE;
  return enqueue_attend(g, c, nullptr, nullptr, q, out, softmax_scale, ws, ws_bytes,
                        (hipStream_t)stream);
}

kivi_status kivi_decode_step(const kivi_geom *g, kivi_cache *c, const uint16_t *k_new,
                             const uint16_t *v_new, const uint16_t *q, float *out,
                             float softmax_scale, void *ws, size_t ws_bytes, int32_t *flushed,
                             void *stream) {
  return decode_step_impl(g, c, k_new, v_new, q, out, softmax_scale, ws, ws_bytes, flushed,
                          (hipStream_t)stream, false);
}

kivi_status kivi_decode_step_noalloc(const kivi_geom *g, kivi_cache *c, const uint16_t *k_new,
                                     const uint16_t *v_new, const uint16_t *q, float *out,
                                     float softmax_scale, int32_t *flushed, void *stream) {
  return decode_step_impl(g, c, k_new, v_new, q, out, softmax_scale, nullptr, 0, flushed,
                          (hipStream_t)stream, true);
}

kivi_status kivi_dense_decode_attention(const kivi_geom *g, const uint16_t *k, const uint16_t *v,
                                        int32_t seq_len, const uint16_t *q, float *out,
                                        float softmax_scale, void *ws, size_t ws_bytes,
                                        void *stream) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  if (!k || !v) return KIVI_E_NULL;
  if (seq_len < 1 || seq_len > g->max_tokens) return KIVI_E_SEQLEN;
  if ((st = check_attend_args(g, 0, seq_len, q, out, softmax_scale, ws, ws_bytes)) != KIVI_OK)
    return st;
  // the dense cache is read as a residual of seq_len tokens in a "ring" of
  // max_tokens slots starting at slot 0; there is no quantised history
  kivi_cache c{};
  c.k_res = const_cast<uint16_t *>(k);
  c.v_res = const_cast<uint16_t *>(v);
  c.n_q = 0;
  c.n_res = seq_len;
  c.res_start = 0;
  return enqueue_attend(g, &c, nullptr, nullptr, q, out, softmax_scale, ws, ws_bytes,
                        (hipStream_t)stream, g->max_tokens);
}

}  // extern "C"

namespace {

// Mixed-length prefill and decode step over a contiguous (pages.table ==
// nullptr) or paged history; the caller has validated the geometry, the
// cache pointers and the page map.
kivi_status ragged_prefill_impl(const kivi_geom *g, const kivi_cache *c, const kivi::PageMap &pm,
                                const uint16_t *k, const uint16_t *v, int32_t stride,
                                const int32_t *seq_lens, int32_t *state, hipStream_t s) {
  kivi_status st = KIVI_OK;
  if (!k || !v || !seq_lens || !state) return KIVI_E_NULL;
  if (stride < 1 || stride > (1 << 24)) return KIVI_E_SEQLEN;
  const int G = g->group, R = g->residual, slots = R + G;
  // the longest possible quantised part sizes the quantiser's grid
  int nq_max = 0, r_max = 0;
  if (!kivi::seq_split(stride, stride, G, R, 1 << 30, nq_max, r_max)) return KIVI_E_SEQLEN;
  if (nq_max > g->max_tokens) nq_max = g->max_tokens / G * G;
  if (nq_max > 0) {
    kivi::QuantizeArgs a{};
    a.src_k = k; a.src_v = v;
    a.src_unit_stride = (long long)stride * g->head_dim;
    a.src_tok0 = 0;
    a.n_groups = nq_max / G; a.n_units = (int)units_of(g); a.dst_g0 = 0;
    a.max_tokens = g->max_tokens; a.n_groups_cap = g->max_tokens / G;
    a.records = c->records;
      a.seq_lens = seq_lens;
    a.kv_heads = g->kv_heads; a.residual = R; a.slots = slots; a.stride = stride;
    a.pages = pm;
    if ((st = hip_status(kivi::launch_quantize(g->bits, g->meta_format, a, s))) != KIVI_OK)
      return st;
  }
  kivi::RaggedResidualArgs r{};
  r.src_k = k; r.src_v = v;
  r.dst_k = c->k_res; r.dst_v = c->v_res;
  r.seq_lens = seq_lens; r.state = state;
  r.n_units = (int)units_of(g); r.kv_heads = g->kv_heads; r.stride = stride;
  r.group = G; r.residual = R; r.slots = slots; r.max_tokens = g->max_tokens;
  r.pages = pm;
  return hip_status(kivi::launch_ragged_residual(r, s));
}

kivi_status ragged_step_impl(const kivi_geom *g, const kivi_cache *c, const kivi::PageMap &pm,
                             const int32_t *state_in, int32_t *state_out, const uint16_t *k_new,
                             const uint16_t *v_new, const uint16_t *q, float *out,
                             float softmax_scale, void *ws, size_t ws_bytes, hipStream_t s) {
  kivi_status st = KIVI_OK;
  if (!state_in || !state_out || !k_new || !v_new) return KIVI_E_NULL;
  if (state_in == state_out) return KIVI_E_STATE;
  if ((st = check_attend_args(g, g->max_tokens, g->residual + g->group, q, out, softmax_scale, ws,
                              ws_bytes)) != KIVI_OK)
    return st;
  // the flush runs before the fused append, which needs R >= G (see
  // kivi_decode_step)
  if (g->residual < g->group) return KIVI_E_UNSUPPORTED;
  const int G = g->group, slots = g->residual + G;
  // One launch: every sequence's counters come from state_in, the launch
  // shape from the capacity; a sequence whose ring fills with this step's
  // append has its G oldest ring tokens quantised into its next group inside
  // the launch (the flush), then takes the fused append.
  kivi_cache bound = *c;
  bound.n_q = g->max_tokens / G * G;
  bound.n_res = slots;
  bound.res_start = 0;
  return enqueue_attend(g, &bound, k_new, v_new, q, out, softmax_scale, ws, ws_bytes, s, 0,
                        state_in, state_out, pm);
}

// Page map of a paged cache; KIVI_E_NULL / KIVI_E_UNSUPPORTED when the pool
// description is unusable (see kivi_paged_layout).
kivi_status paged_map(const kivi_geom *g, const kivi_paged_cache *pc, kivi::PageMap &pm,
                      kivi_cache &c) {
  if (!pc) return KIVI_E_NULL;
  if (!pc->records || !pc->k_res || !pc->v_res || !pc->block_table) return KIVI_E_NULL;
  size_t bytes[KIVI_NUM_BUFS];
  int32_t max_pages = 0;
  kivi_status st = kivi_paged_layout(g, pc->page_groups, pc->num_pages, bytes, &max_pages);
  if (st != KIVI_OK) return st;
  int shift = 0;
  while ((1 << shift) < pc->page_groups) ++shift;
  pm.table = pc->block_table;
  pm.shift = shift;
  pm.max_pages = max_pages;
  pm.num_pages = pc->num_pages;
  c = kivi_cache{};
  c.records = pc->records;
  c.k_res = pc->k_res; c.v_res = pc->v_res;
  return KIVI_OK;
}

}  // namespace

extern "C" {

kivi_status kivi_ragged_prefill(const kivi_geom *g, const kivi_cache *c, const uint16_t *k,
                                const uint16_t *v, int32_t stride, const int32_t *seq_lens,
                                int32_t *state, void *stream) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  if ((st = check_cache(g, c)) != KIVI_OK) return st;
  return ragged_prefill_impl(g, c, kivi::PageMap{}, k, v, stride, seq_lens, state,
                             (hipStream_t)stream);
}

kivi_status kivi_ragged_decode_step(const kivi_geom *g, const kivi_cache *c,
                                    const int32_t *state_in, int32_t *state_out,
                                    const uint16_t *k_new, const uint16_t *v_new,
                                    const uint16_t *q, float *out, float softmax_scale, void *ws,
                                    size_t ws_bytes, void *stream) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  if ((st = check_cache(g, c)) != KIVI_OK) return st;
  return ragged_step_impl(g, c, kivi::PageMap{}, state_in, state_out, k_new, v_new, q, out,
                          softmax_scale, ws, ws_bytes, (hipStream_t)stream);
}

kivi_status kivi_paged_layout(const kivi_geom *g, int32_t page_groups, int32_t num_pages,
                              size_t bytes[KIVI_NUM_BUFS], int32_t *max_pages) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  if (!bytes) return KIVI_E_NULL;
  if (page_groups < 1 || page_groups > (1 << 20) || (page_groups & (page_groups - 1)) != 0 ||
      num_pages < 1)
    return KIVI_E_UNSUPPORTED;
  const size_t D = (size_t)g->head_dim;
  const size_t slots = (size_t)(g->residual + g->group);
  const double groups = (double)num_pages * g->kv_heads * page_groups;
  // the pool is addressed with 32-bit offsets that must stay below 2^31
  const size_t rec = (size_t)kivi::rec_bytes(g->bits, g->meta_format);
  if (groups * rec >= 2147483648.0) return KIVI_E_UNSUPPORTED;
  const size_t n = (size_t)groups;
  bytes[KIVI_BUF_RECORDS] = n * rec;
  bytes[KIVI_BUF_K_RES] = (size_t)units_of(g) * slots * D * 2;
  bytes[KIVI_BUF_V_RES] = (size_t)units_of(g) * slots * D * 2;
  if (max_pages) {
    const int ng = g->max_tokens / g->group;
    *max_pages = (ng + page_groups - 1) / page_groups;
  }
  return KIVI_OK;
}

kivi_status kivi_paged_prefill(const kivi_geom *g, const kivi_paged_cache *pc, const uint16_t *k,
                               const uint16_t *v, int32_t stride, const int32_t *seq_lens,
                               int32_t *state, void *stream) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  kivi::PageMap pm{};
  kivi_cache c{};
  if ((st = paged_map(g, pc, pm, c)) != KIVI_OK) return st;
  return ragged_prefill_impl(g, &c, pm, k, v, stride, seq_lens, state, (hipStream_t)stream);
}

kivi_status kivi_paged_decode_step(const kivi_geom *g, const kivi_paged_cache *pc,
                                   const int32_t *state_in, int32_t *state_out,
                                   const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q,
                                   float *out, float softmax_scale, void *ws, size_t ws_bytes,
                                   void *stream) {
  kivi_status st = check_geom(g);
  if (st != KIVI_OK) return st;
  kivi::PageMap pm{};
  kivi_cache c{};
  if ((st = paged_map(g, pc, pm, c)) != KIVI_OK) return st;
  return ragged_step_impl(g, &c, pm, state_in, state_out, k_new, v_new, q, out, softmax_scale,
                          ws, ws_bytes, (hipStream_t)stream);
}

}  // extern "C"
