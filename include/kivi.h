/*
 * kivi.h -- C ABI of libkivi.so: KIVI asymmetric low-bit KV cache
 * (keys per-channel, values per-token, min-max scale/zero, bf16 residual)
 * and the decode-step attention that reads it, as HIP kernels for gfx950.
 *
 * Sources of the method (web pages):
 *  [card]    "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
 *            (paper card) -- method paragraph: keys grouped along the channel
 *            dimension, values per token, each with a group size, no tuning;
 *            the channel/token split matches how attention reads memory.
 *  [article] "KV cache quantization squeezes 5GB down to fit longer LLM
 *            generations" -- asymmetry paragraph: outlier channels in keys,
 *            asymmetric 2-bit quantization.
 *  [record]  catalog record "kv-efficiency/kivi-2bit-llama3-8b-gqa-8k" --
 *            "KV bytes basis" (grouped 2-bit history, group 32, bf16 residual
 *            of the most recent R=128 tokens), "Methodology" (group size 32
 *            and residual 128 for both 2- and 4-bit), "notes" (4-bit rate).
 *
 * Where the pages leave a step open, this header fixes one reading; every
 * such reading is marked READING below.
 *
 * ------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ------------------------------------------------------------------------
 *  - Pointers named "device" must point to device memory of the current HIP
 *    device; the caller allocates every buffer and keeps it alive until the
 *    work enqueued on `stream` has finished.  The library never allocates
 *    and never synchronises.  Its only global state is a thread-local copy
 *    of the last HIP error and, per device, the resident-workgroup count of
 *    each decode kernel (queried once from the HIP occupancy API and reused;
 *    safe to share between threads).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *  - All arguments are validated on the host before anything is enqueued.
 *    On any error nothing is enqueued and the counters in kivi_cache are
 *    left unchanged.  No exception crosses the ABI.  KIVI_E_HIP is returned
 *    when a launch fails; kivi_last_hip_error() then gives the hipError_t.
 *  - Supported set (v1): bits in {2,4}; group == 32; head_dim == 128;
 *    meta_format in {KIVI_META_FP32, KIVI_META_FP16_BF16}; flags a
 *    combination of KIVI_FLAG_*; residual a multiple of group with
 *    0 <= residual <= 4096; 1 <= q_per_kv <= 16; max_tokens a multiple of
 *    group whose records take at most 2^30 bytes per (sequence, kv head),
 *    i.e. (max_tokens / 32) * record bytes <= 2^30 (max_tokens <= 8,388,608
 *    at 2-bit with fp32 scale/zero, 5,592,384 at 4-bit); batch, kv_heads >= 1
 *    with batch * kv_heads <= 65535.  Anything else: KIVI_E_UNSUPPORTED (or
 *    KIVI_E_GEOMETRY for non-positive sizes).
 *  - Repeatability.  With KIVI_FLAG_DETERMINISTIC in geom.flags every
 *    decode-attention launch (kivi_decode_attention, kivi_decode_step, the
 *    dense, mixed-length and paged calls) splits its work the same way each
 *    time and sums in a fixed order: the same inputs on the same device give
 *    bitwise the same output.  Without it, a launch of at most 4 query heads
 *    per kv head and at most one (sequence, kv head) per compute unit (the
 *    Llama-3-8B-shaped batch of 16 at 8K tokens is one) lets the waves of a
 *    workgroup take token groups as they become free; the grouping of the
 *    fp32 online-softmax sums then depends on timing, and two calls on the
 *    same inputs can differ in the last bits (measured: up to 3.5e-5 of the
 *    row's largest output at that batch, none at small ones; the bound of
 *    the accuracy target, 1e-3, holds for both).  With the flag such a
 *    launch keeps its shape but hands the groups out round-robin (measured
 *    about 3% slower at that batch).  Quantised codes and scale/zero bytes
 *    never depend on the flag.
 *  - The whole batch moves in lockstep: one (n_q, n_res, res_start) triple
 *    describes every sequence of the batch.
 *  - Numbers: bf16 tensors are passed as uint16_t bit patterns.  Inputs must
 *    be finite (NaN/Inf are not checked).
 *
 * ------------------------------------------------------------------------
 * Symbols
 * ------------------------------------------------------------------------
 *  B = batch, H = kv_heads, QPK = q_per_kv, Hq = H*QPK, D = head_dim,
 *  b = bits, L = 2^b - 1, G = group, R = residual, T = max_tokens,
 *  NG = T / G, u = b*H + h  (a "unit" = one sequence and one kv head).
 *  Query head hq = h*QPK + j reads kv head h (READING: consecutive query
 *  heads share a kv head; the record gives only the head counts).
 *
 * ------------------------------------------------------------------------
 * Quantiser (READING of "asymmetric min-max, fp scale/zero", [card] method,
 * [article] asymmetry paragraph; the pages give no formula)
 * ------------------------------------------------------------------------
 *  For one group of G values x_i (bf16 widened exactly to fp32), every
 *  operation in IEEE single precision, round-to-nearest-even, nothing fused:
 *      mn = min x_i ; mx = max x_i
 *      s   = (mx - mn) / L                      (correctly rounded divide)
 *      inv = (s >= FLT_MIN) ? 1 / s : 0         (correctly rounded divide)
 *      c_i = min(max(rint((x_i - mn) * inv), 0), L)
 *      scale = s ; zero = mn ;  dequantised value = c_i * s + mn
 *  A K group is G consecutive tokens of one channel (per-channel keys); a V
 *  group is G consecutive channels of one token (per-token values).
 *
 * ------------------------------------------------------------------------
 * 16-bit scale/zero (geom.meta_format = KIVI_META_FP16_BF16; READING: no page
 * fixes a metadata format, and the record's byte basis counts none)
 * ------------------------------------------------------------------------
 *  The zero, the group minimum, is a bf16 input value and is stored exactly
 *  as bf16.  The scale s = (mx - mn) / L is rounded to fp16 (nearest even;
 *  values above 65504 saturate to 65504) and the codes are computed from
 *  that rounded scale with the formula above.  Scale and zero then take 4
 *  bytes per group instead of 8: at 2-bit, 96 instead of 128 bytes per
 *  quantised token and kv head.  The error bound is half a step of the
 *  rounded scale while it is a normal fp16 number (group range >= L * 2^-14);
 *  below that the scale's own rounding adds up to L times its error.
 *
 * ------------------------------------------------------------------------
 * Byte layout of the cache buffers (part of the contract: packed codes and
 * scale/zero are compared byte for byte with an independent CPU oracle)
 * ------------------------------------------------------------------------
 *  The quantised history of a group is defined in the per-array form
 *  below; the cache stores each group as one record (further below), a
 *  fixed permutation of those bytes.
 *  k_codes  uint8 [G][D*b/8]   token row t of the group holds channel c at
 *           byte c*b/8, bits [(c*b)%8, (c*b)%8 + b)  (LSB first).
 *  k_scale, k_zero  [D]              (channel c)
 *  v_codes  uint8 [G/8][D][b]        octet o (tokens 8o..8o+7 of the group),
 *           channel c: b bytes holding the 8 codes of that channel, token
 *           8o+k at bits [k*b, k*b + b) (LSB first).
 *  v_scale, v_zero  [D/G][G]         (channel group j, token i of the group)
 *           Element type by geom.meta_format: KIVI_META_FP32 -- fp32 scale and
 *           fp32 zero; KIVI_META_FP16_BF16 -- fp16 scale bits and bf16 zero
 *           bits (uint16_t), see "16-bit scale/zero" below.
 *  Group records: the six arrays above are not stored as six buffers.  The
 *           quantised history is one buffer, `records`, of one record per
 *           group: uint8 [B][H][NG][P * 1024], P = b + 2 (fp32 scale/zero)
 *           or b + 1 (16-bit).  Bytes are laid out in the order one 64-lane
 *           wave of the decode kernel reads them: plane p (1024 bytes) holds
 *           16 bytes for each lane l at p*1024 + 16*l.
 *             K codes, planes [0, b/2): lane 16*j + 4*(t>>3) + (t&3) holds
 *               bytes [j*4*b, (j+1)*4*b) of k_codes token rows t (first) and
 *               t+4 (second) of the group, t with (t>>2)&1 == 0 (b = 2: 8
 *               bytes each, one plane; b = 4: one plane each).
 *             V codes, planes [b/2, b): lane 16*o + c/8 holds the 8*b bytes
 *               of octet o, channels c..c+7 (c a multiple of 8); b = 4: the
 *               first 16 bytes in plane 2, the other 16 in plane 3.
 *             fp32 scale/zero, planes b and b+1: lane l holds values 2l, 2l+1
 *               of k_scale then of k_zero (plane b) and of v_scale then of
 *               v_zero (plane b+1), value index = channel (K) or
 *               j*G + token (V).
 *             16-bit scale/zero, plane b: lane l holds the pairs 2l, 2l+1 of
 *               k_scale, k_zero, v_scale, v_zero (4 bytes each).
 *           The record keeps every group's bytes contiguous (one 1 KiB load
 *           per plane per wave, from one place in memory) instead of spread
 *           over six arrays.  Paged pools (kivi_paged_layout) hold records the
 *           same way, one per pool slot.
 *  k_res, v_res  bf16 [B][H][R+G][D]        residual ring of R+G slots.
 *           Logical residual token i (0 = oldest) lives in slot
 *           (res_start + i) mod (R+G).  res_start is always a multiple of G.
 *  Packing runs along the contraction axis of the product that reads the
 *  codes (channels for q.K^T, tokens for P.V), orthogonal to the group.
 *
 * ------------------------------------------------------------------------
 * Cache state machine (READING of [record] KV bytes basis: a bf16 residual of
 * the latest R tokens sits beside the grouped history, which alone is
 * quantised; the pages do not say when tokens leave the residual)
 * ------------------------------------------------------------------------
 *  prefill(S):  n_q = G*floor((S-R)/G) if S > R else 0;  n_res = S - n_q
 *               (so R <= n_res < R+G once S >= R);  res_start = 0.
 *  per decode step: append (n_res += 1) -> flush iff n_res == R+G (the G
 *               oldest residual tokens become quantised group n_q/G) ->
 *               attend over all n_q + n_res tokens.
 *  Appending N tokens after prefill(S) leaves exactly the state (quantised
 *  bytes and logical residual) that prefill(S+N) produces.
 */
#ifndef KIVI_H_
#define KIVI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KIVI_OK = 0,
  KIVI_E_NULL = 1,           /* a required pointer is NULL                   */
  KIVI_E_GEOMETRY = 2,       /* a size is zero/negative or inconsistent      */
  KIVI_E_UNSUPPORTED = 3,    /* valid geometry outside the supported set     */
  KIVI_E_SEQLEN = 4,         /* prefill seq_len < 1                          */
  KIVI_E_CAPACITY = 5,       /* quantised history would exceed max_tokens    */
  KIVI_E_RESIDUAL_FULL = 6,  /* append with n_res == R+G (flush first)       */
  KIVI_E_WORKSPACE = 7,      /* decode workspace NULL or too small           */
  KIVI_E_HIP = 8,            /* a HIP launch failed (see kivi_last_hip_error)*/
  KIVI_E_STATE = 9           /* cache counters invalid (e.g. empty cache)    */
} kivi_status;

/* Element types of the scale/zero buffers (kivi_geom.meta_format). */
enum {
  KIVI_META_FP32 = 0,        /* fp32 scale, fp32 zero                        */
  KIVI_META_FP16_BF16 = 1    /* fp16 scale, bf16 zero (uint16_t bit patterns) */
};

/* Launch options (kivi_geom.flags). */
enum {
  KIVI_FLAG_DETERMINISTIC = 1   /* bitwise-repeatable decode attention (see
                                 * "Repeatability" above)                    */
};

/* Problem statement: batch, kv heads, query heads per kv head (GQA),
 * head_dim, bits, group size G, residual length R, the capacity of the
 * quantised history in tokens, the scale/zero format (KIVI_META_*), and
 * launch options (KIVI_FLAG_*, 0 for none). */
typedef struct {
  int32_t batch;
  int32_t kv_heads;
  int32_t q_per_kv;
  int32_t head_dim;
  int32_t bits;
  int32_t group;
  int32_t residual;
  int32_t max_tokens;
  int32_t meta_format;
  int32_t flags;
} kivi_geom;

/* The cache: three caller-owned device buffers laid out as described above
 * (the group records and the two residual rings), plus three host-side
 * counters that the calls below update. */
typedef struct {
  uint8_t  *records;    /* group records [B][H][NG][record bytes]          */
  uint16_t *k_res;      /* bf16 ring [B][H][R+G][D]                        */
  uint16_t *v_res;      /* bf16 ring [B][H][R+G][D]                        */
  int32_t   n_q;        /* tokens in the quantised history (multiple of G) */
  int32_t   n_res;      /* tokens in the residual ring                     */
  int32_t   res_start;  /* ring slot of the oldest residual token          */
} kivi_cache;

/* Order of the sizes written by kivi_cache_layout and kivi_paged_layout. */
enum { KIVI_BUF_RECORDS = 0, KIVI_BUF_K_RES, KIVI_BUF_V_RES, KIVI_NUM_BUFS };

/* Byte sizes of the KIVI_NUM_BUFS cache buffers for `geom`, in the order of
 * the KIVI_BUF_* enum.  Host-only, touches no device.
 * Errors: KIVI_E_NULL, KIVI_E_GEOMETRY, KIVI_E_UNSUPPORTED. */
kivi_status kivi_cache_layout(const kivi_geom *geom, size_t bytes_out[KIVI_NUM_BUFS]);

/* Bytes of decode workspace that a decode-attention launch needs for `geom`
 * over a cache of n_q quantised and n_res residual tokens.  The need grows
 * with both counts, so a workspace of that size also serves every smaller
 * state: n_q = max_tokens, n_res = R+G gives one for every state of the
 * cache (the mixed-length and paged calls need that one; the dense baseline
 * needs n_q = 0, n_res = seq_len).  Host-only.  The size is
 *   256 * ceil(4 * B * H / 256) + B * H * QPK * 528 * S,
 *   S = min(max(floor((n_q / G * c + ceil(n_res / 32) * 16) / (8 * c)), 1), 256),
 * c = bits + 2 (fp32 scale/zero) or bits + 1 (16-bit): one arrival counter
 * per (sequence, kv head), then up to S split partials of 132 floats per
 * query head (S bounds the workgroups a launch gives one (sequence, kv
 * head)).
 * Returns 0 when geom is NULL or outside the supported set, or when n_q is
 * not a multiple of G in [0, max_tokens] or n_res < 0. */
size_t kivi_decode_workspace_bytes(const kivi_geom *geom, int32_t n_q, int32_t n_res);

/* Prefill: quantise the first n_q tokens of k and v into the grouped
 * history ([card] method: per-channel K, per-token V; [record] Methodology:
 * G = 32) and copy the last n_res tokens, unchanged, into ring slots
 * 0..n_res-1 ([record] KV bytes basis: bf16 residual of the most recent R).
 * k, v: device bf16 [B][H][seq_len][D], read only.
 * Resets the cache: sets n_q, n_res, res_start (= 0).
 * Errors: KIVI_E_NULL, KIVI_E_GEOMETRY, KIVI_E_UNSUPPORTED,
 *         KIVI_E_SEQLEN (seq_len < 1), KIVI_E_CAPACITY (n_q > max_tokens),
 *         KIVI_E_HIP. */
kivi_status kivi_quantize_prefill(const kivi_geom *geom, kivi_cache *cache,
                                  const uint16_t *k, const uint16_t *v,
                                  int32_t seq_len, void *stream);

/* Append one decoded token per sequence and kv head to the residual ring
 * ([record] KV bytes basis: the newest tokens are kept unquantised in bf16):
 * slot (res_start + n_res) mod (R+G); then n_res += 1.
 * k_new, v_new: device bf16 [B][H][D].
 * Errors: KIVI_E_NULL, KIVI_E_GEOMETRY, KIVI_E_UNSUPPORTED,
 *         KIVI_E_RESIDUAL_FULL (n_res == R+G: flush first), KIVI_E_STATE,
 *         KIVI_E_HIP. */
kivi_status kivi_append_token(const kivi_geom *geom, kivi_cache *cache,
                              const uint16_t *k_new, const uint16_t *v_new,
                              void *stream);

/* Flush ([record] KV bytes basis: only the grouped history is quantised, in
 * groups of G = 32 tokens, while the latest R stay in bf16; READING: a group
 * leaves the residual as soon as R tokens remain without it): iff
 * n_res == R+G, quantise the G oldest residual tokens into group n_q/G with
 * the same quantiser as prefill ([card] method: per-channel K, per-token
 * V), then n_q += G, n_res -= G,
 * res_start = (res_start + G) mod (R+G), and *flushed = 1; otherwise do
 * nothing and set *flushed = 0.  `flushed` is a host pointer (may be NULL).
 * Errors: KIVI_E_NULL, KIVI_E_GEOMETRY, KIVI_E_UNSUPPORTED,
 *         KIVI_E_CAPACITY (n_q + G > max_tokens), KIVI_E_STATE, KIVI_E_HIP. */
kivi_status kivi_flush_residual(const kivi_geom *geom, kivi_cache *cache,
                                int32_t *flushed, void *stream);

/* Decode-step attention over the mixed cache ([card] method: the attention
 * kernel reads per-channel K and per-token V; [record] KV bytes basis:
 * grouped history plus bf16 residual).  For every query head hq of every
 * sequence: score_t = softmax_scale * q . k_t over all n_q + n_res cached
 * tokens (dequantised history and bf16 residual; no mask, no position
 * handling), p = softmax(score), out = sum_t p_t v_t, accumulated in fp32.
 * q:   device bf16 [B][Hq][D];  out: device fp32 [B][Hq][D] (written fully).
 * ws:  device workspace of at least kivi_decode_workspace_bytes(geom, n_q,
 *      n_res) bytes for the cache's counters, filled with zero bytes before
 *      its first use.  It holds one arrival counter per
 *      (sequence, kv head) and the split-K partials; every call returns the
 *      counters to zero, so a workspace is reusable by later calls ordered on
 *      the same stream.  Calls that overlap in time on one workspace race.
 * Errors: KIVI_E_NULL, KIVI_E_GEOMETRY, KIVI_E_UNSUPPORTED, KIVI_E_STATE
 *         (n_q + n_res == 0 or counters out of range), KIVI_E_WORKSPACE,
 *         KIVI_E_HIP. */
kivi_status kivi_decode_attention(const kivi_geom *geom, const kivi_cache *cache,
                                  const uint16_t *q, float *out,
                                  float softmax_scale, void *ws, size_t ws_bytes,
                                  void *stream);

/* One decode step of one layer in a single launch (R >= G): append
 * k_new/v_new, flush iff the ring is then full, and attend with q -- the
 * same cache bytes, counters and `out` as kivi_append_token,
 * kivi_flush_residual and kivi_decode_attention called in that order (the
 * step order of the cache state machine above).
 * How: when the append would fill the ring (n_res == R+G-1) the G oldest
 * tokens are quantised first; with R >= G they cannot include the new
 * token, so the state is the same.  The attention launch does both: the
 * workgroup whose share holds the new group quantises it from the ring
 * before any of its waves reads it, and the new token is read from
 * k_new/v_new and stored into its ring slot by the kernel.  With R == 0 a
 * flush step runs as three launches.
 * k_new, v_new: device bf16 [B][H][D]; q, out, softmax_scale, ws, ws_bytes
 * as for kivi_decode_attention, the workspace sized for the counters after
 * the step (kivi_decode_workspace_bytes(geom, n_q, n_res + 1) serves every
 * step, a flush only moving tokens from the residual to the history);
 * flushed: host pointer (may be NULL), set to 1 if a group was flushed, else
 * 0.
 * Errors (checked before anything is enqueued): those of the three calls,
 * i.e. KIVI_E_NULL, KIVI_E_GEOMETRY, KIVI_E_UNSUPPORTED, KIVI_E_STATE,
 * KIVI_E_RESIDUAL_FULL (n_res == R+G on entry), KIVI_E_CAPACITY (a flush is
 * due and n_q + G > max_tokens), KIVI_E_WORKSPACE; KIVI_E_HIP if a launch
 * fails, with the counters reflecting the launches that were enqueued. */
kivi_status kivi_decode_step(const kivi_geom *geom, kivi_cache *cache,
                             const uint16_t *k_new, const uint16_t *v_new,
                             const uint16_t *q, float *out, float softmax_scale,
                             void *ws, size_t ws_bytes, int32_t *flushed,
                             void *stream);

/* kivi_decode_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same launches, cache bytes, counters and output as
 * kivi_decode_step, with the decode workspace taken from a static device
 * array of the library (16 MiB per device that runs the call, held until
 * the process ends) instead of (ws, ws_bytes); the call allocates nothing.
 * The first call on a device takes the array's address and zeroes its
 * arrival counters with a kernel on `stream`; every call leaves them at zero.
 * All calls on one device share the array, so calls that overlap in time on
 * one device (other streams, other threads) race; order them on one stream.
 * Errors: those of kivi_decode_step, and KIVI_E_WORKSPACE when the step
 * needs more than the array holds, i.e. kivi_decode_workspace_bytes(geom,
 * n_q, n_res + 1) > 16 MiB (at 4 query heads per kv head and 8K tokens:
 * about 72 KB per (sequence, kv head), so at most 233 of them; the
 * Llama-3-8B-shaped batch of 16 x 8 kv heads needs 9.2 MB);
 * KIVI_E_UNSUPPORTED for a device index of 64 or more. */
kivi_status kivi_decode_step_noalloc(const kivi_geom *geom, kivi_cache *cache,
                                     const uint16_t *k_new, const uint16_t *v_new,
                                     const uint16_t *q, float *out, float softmax_scale,
                                     int32_t *flushed, void *stream);

/* Baseline: decode attention over an uncompressed bf16 KV cache, the
 * reference point of the pages' speed and memory claims ([card]: compared
 * with the FP16 cache; [record] Methodology: throughput over the FP16
 * baseline).  Same attention as kivi_decode_attention (no mask, fp32
 * accumulation, consecutive query heads per kv head), over the first
 * seq_len tokens of each (sequence, kv head).
 * geom: batch, kv_heads, q_per_kv and head_dim as usual; max_tokens is the
 *      token capacity T of the dense cache; bits, group and residual must be
 *      a supported combination but do not affect the result.
 * k, v: device bf16 [B][H][T][D], read only.  1 <= seq_len <= T.
 * q, out, softmax_scale, ws, ws_bytes: as for kivi_decode_attention, the
 *      workspace at least kivi_decode_workspace_bytes(geom, 0, seq_len).
 * Errors: KIVI_E_NULL, KIVI_E_GEOMETRY, KIVI_E_UNSUPPORTED, KIVI_E_SEQLEN,
 *         KIVI_E_WORKSPACE, KIVI_E_HIP. */
kivi_status kivi_dense_decode_attention(const kivi_geom *geom, const uint16_t *k,
                                        const uint16_t *v, int32_t seq_len,
                                        const uint16_t *q, float *out,
                                        float softmax_scale, void *ws, size_t ws_bytes,
                                        void *stream);

/* ------------------------------------------------------------------------
 * Mixed-length batches (per-sequence lengths).  The lockstep calls above
 * keep one (n_q, n_res, res_start) for the whole batch.  These two calls keep
 * it per sequence instead, in device memory, so that sequences of different
 * lengths share one cache and one launch per step, and so that a step's
 * launches take the same arguments every step (they can be captured in a
 * HIP graph; the state buffers alternate between two captured steps).
 *
 * State: int32 [B][4] per sequence: {n_q, n_res, res_start, flags}, with
 * the meaning of the kivi_cache counters.  flags: 0, or KIVI_SEQ_BAD_LENGTH
 * (the prefill length was out of range; the sequence is empty and its
 * output rows are 0) or KIVI_SEQ_FULL (a flush was due with no room for
 * another group; the sequence keeps its cache and takes no more tokens).
 * A state row that these calls cannot have written (history not whole
 * groups or beyond max_tokens, ring count or start out of range, unknown flag
 * bits) is taken as an empty KIVI_SEQ_BAD_LENGTH sequence.
 * The counters of kivi_cache are ignored by these calls.
 * ------------------------------------------------------------------------ */
enum { KIVI_SEQ_BAD_LENGTH = 1, KIVI_SEQ_FULL = 2 };

/* Prefill of a mixed-length batch: sequence b has seq_lens[b] tokens (device
 * int32 [B]), the first ones of each row block of k, v (device bf16
 * [B][H][stride][D]).  Each sequence is split and quantised exactly as
 * kivi_quantize_prefill splits a batch of that length; state (device int32
 * [B][4]) receives every sequence's counters.  A length outside
 * [1, stride], or one whose quantised part exceeds max_tokens, gives that
 * sequence KIVI_SEQ_BAD_LENGTH.
 * Errors: KIVI_E_NULL, KIVI_E_GEOMETRY, KIVI_E_UNSUPPORTED, KIVI_E_SEQLEN
 *         (stride < 1), KIVI_E_HIP. */
kivi_status kivi_ragged_prefill(const kivi_geom *geom, const kivi_cache *cache,
                                const uint16_t *k, const uint16_t *v, int32_t stride,
                                const int32_t *seq_lens, int32_t *state, void *stream);

/* One decode step of a mixed-length batch: for every sequence, append
 * k_new/v_new, flush iff its ring is then full, and attend with q -- per
 * sequence the same cache bytes and output as kivi_decode_step on a batch
 * of that sequence alone.  One launch with fixed arguments: decode
 * attention in which each sequence due to flush first quantises its G
 * oldest ring tokens into its next group, and the append is fused.  The
 * state is read from state_in and the state after
 * the step written to state_out (distinct device int32 [B][4] buffers; the
 * next step reads state_out).  Requires residual >= group.
 * k_new, v_new: device bf16 [B][H][D]; q, out, softmax_scale, ws, ws_bytes
 * as for kivi_decode_attention, the workspace at least
 * kivi_decode_workspace_bytes(geom, max_tokens, R+G).
 * Errors: KIVI_E_NULL, KIVI_E_GEOMETRY, KIVI_E_UNSUPPORTED, KIVI_E_STATE
 *         (state_in == state_out), KIVI_E_WORKSPACE, KIVI_E_HIP. */
kivi_status kivi_ragged_decode_step(const kivi_geom *geom, const kivi_cache *cache,
                                    const int32_t *state_in, int32_t *state_out,
                                    const uint16_t *k_new, const uint16_t *v_new,
                                    const uint16_t *q, float *out, float softmax_scale,
                                    void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Paged history (for serving: a pool of fixed-size pages shared by the
 * sequences of a batch, assigned by the caller through a block table).  The
 * quantised history is split into pages of page_groups consecutive groups
 * (page_groups * 32 tokens); one page holds those groups for every kv head
 * of one sequence.  Sequence b's group g lives in page block_table[b][g /
 * page_groups]; inside the pools, (page p, kv head h, group i of the page)
 * is group slot s = (p * H + h) * page_groups + i.  The history is one
 * pool, records [slots][record bytes] of group records (as in kivi_cache).
 * The residual rings are not paged:
 * k_res, v_res are [B][H][R+G][D] as in kivi_cache.  Lengths are per
 * sequence, in the same device state as the mixed-length calls above.
 *
 * block_table: device int32 [B][max_pages] (kivi_paged_layout gives
 * max_pages = ceil(max_tokens / G / page_groups)); entries outside
 * [0, num_pages) are unassigned.  The library only reads it; the caller
 * assigns pages (a page must not serve two sequences) and may add pages
 * between calls.  A prefill whose history needs an unassigned page gives the
 * sequence KIVI_SEQ_BAD_LENGTH; a flush into an unassigned page is treated
 * like a full cache (KIVI_SEQ_FULL: the sequence keeps its cache and takes
 * no more tokens), so assigning the next page before it is needed keeps a
 * sequence going.  A history group whose entry is changed to an unassigned
 * one after it was written reads as zeros.
 * ------------------------------------------------------------------------ */
typedef struct {
  uint8_t  *records;            /* record pool (kivi_paged_layout size)     */
  uint16_t *k_res;              /* [B][H][R+G][D] rings, as in kivi_cache  */
  uint16_t *v_res;
  const int32_t *block_table;   /* device [B][max_pages]                    */
  int32_t   page_groups;        /* groups per page: a power of two <= 2^20  */
  int32_t   num_pages;          /* pages in each pool                        */
} kivi_paged_cache;

/* Byte sizes of the buffers of a paged cache (in the order of the KIVI_BUF_*
 * enum: the record pool, the two rings) and the block table's row length.
 * The record pool must stay below 2 GiB (its offsets are 32-bit).
 * Errors: KIVI_E_NULL (bytes), KIVI_E_GEOMETRY, KIVI_E_UNSUPPORTED (geom
 *         outside the supported set, page_groups not a power of two in
 *         [1, 2^20], num_pages < 1, or a pool of 2 GiB or more). */
kivi_status kivi_paged_layout(const kivi_geom *geom, int32_t page_groups, int32_t num_pages,
                              size_t bytes[KIVI_NUM_BUFS], int32_t *max_pages);

/* kivi_ragged_prefill into a paged cache: the same split, codes and
 * scale/zero bytes per sequence, stored in the sequence's pages.
 * Errors: those of kivi_ragged_prefill and kivi_paged_layout; KIVI_E_NULL
 *         for a NULL pool (that the layout uses), ring or block table. */
kivi_status kivi_paged_prefill(const kivi_geom *geom, const kivi_paged_cache *cache,
                               const uint16_t *k, const uint16_t *v, int32_t stride,
                               const int32_t *seq_lens, int32_t *state, void *stream);

/* kivi_ragged_decode_step over a paged cache (flushes write the new group
 * into its page).  The same single launch with fixed arguments.
 * Errors: those of kivi_ragged_decode_step and kivi_paged_layout. */
kivi_status kivi_paged_decode_step(const kivi_geom *geom, const kivi_paged_cache *cache,
                                   const int32_t *state_in, int32_t *state_out,
                                   const uint16_t *k_new, const uint16_t *v_new,
                                   const uint16_t *q, float *out, float softmax_scale,
                                   void *ws, size_t ws_bytes, void *stream);

/* Static description of a status code (never NULL). */
const char *kivi_status_string(kivi_status status);

/* hipError_t of the last failed HIP call made by this thread (0 if none). */
int32_t kivi_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_H_ */
