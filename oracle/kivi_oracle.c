/*
 * kivi_oracle.c -- plain, slow CPU oracle of the KIVI hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may call it.  It shares no code, header,
 * table or helper with the HIP library: it defines its own types and writes
 * the documented byte layout with its own index formulas.
 *
 * Built with `gcc -O2 -ffp-contract=off` (no fast-math, so no FTZ/DAZ and
 * no fused multiply-add): every float operation below is one IEEE single
 * (or double) operation, rounded to nearest even.
 *
 * What it computes, and where the pages define it:
 *  - per-channel key groups and per-token value groups of G elements
 *    ("KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache",
 *    method paragraph; catalog record kivi-2bit-llama3-8b-gqa-8k,
 *    Methodology: G = 32, R = 128);
 *  - an asymmetric min-max quantiser (paper title "Asymmetric"; news article
 *    "KV cache quantization squeezes 5GB ...", asymmetry paragraph).  The
 *    pages print no formula; the one used is the plain reading: scale =
 *    range / (2^b - 1), zero = group minimum, round half to even;
 *  - a bf16 residual of the most recent tokens, flushed G at a time into a
 *    new group (catalog record, KV bytes basis);
 *  - decode attention over the dequantised history plus the residual, in
 *    double precision (exact softmax attention; a plain definition), and
 *    the same attention over an uncompressed bf16 cache, the baseline the
 *    pages compare against;
 *  - the KV-bytes-per-token arithmetic of the catalog record (KV bytes basis
 *    and notes) and of the news article (memory-math paragraph).
 *
 * Parity pins live in the test-suite (constant groups exact, error bound of
 * half a step, extreme values, constructed ties, fixed packed bytes, the
 * pages' byte figures, streaming == prefill, attention against library SDPA,
 * closed forms and brute force).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int batch, kv_heads, q_per_kv, head_dim, bits, group, residual, max_tokens;
  int meta;   /* scale/zero format: 0 = fp32 scale, fp32 zero; 1 = fp16 scale, bf16 zero */
} kivio_geom;

/* Host arrays in the documented layout (see the comments of each field). */
typedef struct {
  uint8_t *k_codes;   /* [B][H][T][D*b/8]                 */
  void *k_scale;      /* [B][H][T/G][D]        (fp32, or fp16 bits) */
  void *k_zero;       /* [B][H][T/G][D]        (fp32, or bf16 bits) */
  uint8_t *v_codes;   /* [B][H][T/G][G/8][D][b]           */
  void *v_scale;      /* [B][H][T/G][D/G][G]   (fp32, or fp16 bits) */
  void *v_zero;       /* [B][H][T/G][D/G][G]   (fp32, or bf16 bits) */
  uint16_t *k_res;    /* [B][H][R+G][D] bf16 bits         */
  uint16_t *v_res;    /* [B][H][R+G][D] bf16 bits         */
  int n_q, n_res, res_start;
} kivio_cache;

/* ---------------------------------------------------------------- bf16 */

static float bf16_to_float(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return f;
}

/* --------------------------------------------------------- quantiser --- */

/* One asymmetric min-max group of n values (x already widened to float).
 * scale = (max - min) / L, zero = min, code = rint((x - min) * (1/scale))
 * clamped to [0, L]; a group whose scale is below FLT_MIN (constant, or a
 * subnormal range) gets all-zero codes so that it dequantises to its min. */
void kivio_quantize_values(const float *x, int n, int bits, uint8_t *code,
                           float *scale, float *zero) {
  float mn = x[0], mx = x[0];
  for (int i = 1; i < n; ++i) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  const float levels = (float)((1 << bits) - 1);
  const float s = (mx - mn) / levels;
  const float inv = (s >= FLT_MIN) ? 1.0f / s : 0.0f;
  for (int i = 0; i < n; ++i) {
    float y = rintf((x[i] - mn) * inv);
    y = fminf(fmaxf(y, 0.0f), levels);
    code[i] = (uint8_t)y;
  }
  *scale = s;
  *zero = mn;
}

/* One group in the 16-bit scale/zero format (no page fixes a metadata
 * format; the record's byte basis counts none).  The zero stays the group
 * minimum, a bf16 input value, so bf16 holds it exactly.  The scale
 * (max - min) / L is rounded to fp16, to nearest even, and saturates at the
 * largest finite fp16, 65504; the codes are then computed from that rounded
 * scale with the same formula as above, so that code * scale + zero is the
 * value the cache represents.  scale / zero receive the fp16 / bf16 bits. */
static uint16_t fp16_bits_rne(float x);
static float fp16_value(uint16_t bits);

void kivio_quantize_values_h(const float *x, int n, int bits, uint8_t *code,
                             uint16_t *scale, uint16_t *zero) {
  float mn = x[0], mx = x[0];
  for (int i = 1; i < n; ++i) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  const float levels = (float)((1 << bits) - 1);
  const uint16_t sh = fp16_bits_rne((mx - mn) / levels);
  const float s = fp16_value(sh);
  const float inv = (s >= FLT_MIN) ? 1.0f / s : 0.0f;
  for (int i = 0; i < n; ++i) {
    float y = rintf((x[i] - mn) * inv);
    y = fminf(fmaxf(y, 0.0f), levels);
    code[i] = (uint8_t)y;
  }
  uint32_t w;
  memcpy(&w, &mn, sizeof w);
  *scale = sh;
  *zero = (uint16_t)(w >> 16);   /* mn is a widened bf16: the low half is zero */
}

/* IEEE binary16 of a non-negative float, round to nearest even, saturating
 * at 65504: q = 2^(e-10) is the spacing of binary16 numbers at x's binade
 * (e >= -14; below that the subnormal spacing 2^-24), x / q is exact in
 * double and rounded to an integer with ties to even. */
static uint16_t fp16_bits_rne(float x) {
  if (!(x > 0.0f)) return 0;
  if (x >= 65504.0f) return 0x7BFF;
  int e;
  frexp((double)x, &e);   /* x = m * 2^e, 0.5 <= m < 1 */
  e -= 1;                 /* x in [2^e, 2^(e+1)) */
  if (e < -14) e = -14;
  const double q = ldexp(1.0, e - 10);
  double n = nearbyint((double)x / q);   /* default rounding: to nearest even */
  if (n >= 2048.0) {      /* rounded up into the next binade */
    n /= 2.0;
    e += 1;
  }
  if (e > 15) return 0x7BFF;
  if (n < 1024.0) return (uint16_t)n;    /* subnormal (e == -14): mantissa only */
  return (uint16_t)(((e + 15) << 10) | ((int)n - 1024));
}

static float fp16_value(uint16_t bits) {
  const int e = (bits >> 10) & 0x1F, m = bits & 0x3FF;
  if (e == 0) return (float)ldexp((double)m, -24);
  return (float)ldexp((double)(1024 + m), e - 25);
}

/* --------------------------------------------------- layout indexing --- */

static size_t unit_count(const kivio_geom *g) {
  return (size_t)g->batch * (size_t)g->kv_heads;
}
static int n_groups_cap(const kivio_geom *g) { return g->max_tokens / g->group; }
static int ring_slots(const kivio_geom *g) { return g->residual + g->group; }

/* write a b-bit code into a little-endian bit stream at code position pos */
static void put_code(uint8_t *base, size_t pos, int bits, uint8_t code) {
  size_t bit = pos * (size_t)bits;
  uint8_t *byte = base + bit / 8;
  int sh = (int)(bit % 8);
  uint8_t mask = (uint8_t)(((1u << bits) - 1u) << sh);
  *byte = (uint8_t)((*byte & ~mask) | ((code << sh) & mask));
}
static uint8_t get_code(const uint8_t *base, size_t pos, int bits) {
  size_t bit = pos * (size_t)bits;
  return (uint8_t)((base[bit / 8] >> (bit % 8)) & ((1u << bits) - 1u));
}

/* K: token row t of unit u; channel c is code number c of the row. */
static uint8_t *k_row(const kivio_geom *g, const kivio_cache *c, size_t u, int t) {
  size_t row_bytes = (size_t)g->head_dim * g->bits / 8;
  return c->k_codes + (u * (size_t)g->max_tokens + (size_t)t) * row_bytes;
}
/* V: group gi, octet o, channel ch of unit u: 8 codes, token 8o+k is code k. */
static uint8_t *v_cell(const kivio_geom *g, const kivio_cache *c, size_t u, int gi,
                       int o, int ch) {
  size_t octets = (size_t)g->group / 8;
  size_t idx = ((u * (size_t)n_groups_cap(g) + (size_t)gi) * octets + (size_t)o) *
                   (size_t)g->head_dim + (size_t)ch;
  return c->v_codes + idx * (size_t)g->bits;
}
static size_t k_meta(const kivio_geom *g, size_t u, int gi, int ch) {
  return (u * (size_t)n_groups_cap(g) + (size_t)gi) * (size_t)g->head_dim + (size_t)ch;
}
static size_t v_meta(const kivio_geom *g, size_t u, int gi, int j, int i) {
  size_t cg = (size_t)g->head_dim / (size_t)g->group;
  return ((u * (size_t)n_groups_cap(g) + (size_t)gi) * cg + (size_t)j) * (size_t)g->group +
         (size_t)i;
}
static size_t ring_at(const kivio_geom *g, size_t u, int slot, int ch) {
  return (u * (size_t)ring_slots(g) + (size_t)slot) * (size_t)g->head_dim + (size_t)ch;
}

/* Quantise the n values of one group in the geometry's scale/zero format and
 * store scale and zero at index idx of the K (is_v = 0) or V arrays. */
static void store_group_meta(const kivio_geom *g, kivio_cache *c, int is_v, size_t idx,
                             const float *x, int n, int bits, uint8_t *code) {
  void *sc = is_v ? c->v_scale : c->k_scale, *zr = is_v ? c->v_zero : c->k_zero;
  if (g->meta == 1) {
    kivio_quantize_values_h(x, n, bits, code, (uint16_t *)sc + idx, (uint16_t *)zr + idx);
  } else {
    kivio_quantize_values(x, n, bits, code, (float *)sc + idx, (float *)zr + idx);
  }
}

/* scale and zero at index idx of the K (is_v = 0) or V arrays, as doubles */
static double meta_scale(const kivio_geom *g, const kivio_cache *c, int is_v, size_t idx) {
  const void *sc = is_v ? c->v_scale : c->k_scale;
  if (g->meta == 1) return (double)fp16_value(((const uint16_t *)sc)[idx]);
  return (double)((const float *)sc)[idx];
}
static double meta_zero(const kivio_geom *g, const kivio_cache *c, int is_v, size_t idx) {
  const void *zr = is_v ? c->v_zero : c->k_zero;
  if (g->meta == 1) return (double)bf16_to_float(((const uint16_t *)zr)[idx]);
  return (double)((const float *)zr)[idx];
}

/* Quantise one group of G tokens into group index gi.  src_k / src_v give
 * token i (0..G-1) of unit u as bf16 rows of D values. */
static void quantize_group(const kivio_geom *g, kivio_cache *c, size_t u, int gi,
                           const uint16_t *const *src_k, const uint16_t *const *src_v) {
  const int G = g->group, D = g->head_dim, b = g->bits;
  float x[64];
  uint8_t code[64];
  /* keys: one group per channel, along the G tokens */
  for (int ch = 0; ch < D; ++ch) {
    for (int i = 0; i < G; ++i) x[i] = bf16_to_float(src_k[i][ch]);
    store_group_meta(g, c, 0, k_meta(g, u, gi, ch), x, G, b, code);
    for (int i = 0; i < G; ++i) put_code(k_row(g, c, u, gi * G + i), (size_t)ch, b, code[i]);
  }
  /* values: one group per token and block of G channels */
  for (int i = 0; i < G; ++i) {
    for (int j = 0; j < D / G; ++j) {
      for (int e = 0; e < G; ++e) x[e] = bf16_to_float(src_v[i][j * G + e]);
      store_group_meta(g, c, 1, v_meta(g, u, gi, j, i), x, G, b, code);
      for (int e = 0; e < G; ++e) {
        int ch = j * G + e;
        put_code(v_cell(g, c, u, gi, i / 8, ch), (size_t)(i % 8), b, code[e]);
      }
    }
  }
}

/* ------------------------------------------------------------ prefill --- */

/* Tokens quantised by a prefill of S tokens: whole groups, leaving at least
 * R tokens in the residual. */
int kivio_prefill_split(int seq_len, int group, int residual) {
  if (seq_len <= residual) return 0;
  return group * ((seq_len - residual) / group);
}

/* k, v: bf16 [B][H][S][D].  Returns 0, or -1 if the history does not fit. */
int kivio_prefill(const kivio_geom *g, kivio_cache *c, const uint16_t *k,
                  const uint16_t *v, int seq_len) {
  const int G = g->group, D = g->head_dim;
  const int n_q = kivio_prefill_split(seq_len, G, g->residual);
  const int r = seq_len - n_q;
  if (n_q > g->max_tokens || r > ring_slots(g)) return -1;
  const uint16_t *rows_k[64], *rows_v[64];
  for (size_t u = 0; u < unit_count(g); ++u) {
    const uint16_t *ku = k + u * (size_t)seq_len * D;
    const uint16_t *vu = v + u * (size_t)seq_len * D;
    for (int gi = 0; gi < n_q / G; ++gi) {
      for (int i = 0; i < G; ++i) {
        rows_k[i] = ku + (size_t)(gi * G + i) * D;
        rows_v[i] = vu + (size_t)(gi * G + i) * D;
      }
      quantize_group(g, c, u, gi, rows_k, rows_v);
    }
    for (int i = 0; i < r; ++i)
      for (int ch = 0; ch < D; ++ch) {
        c->k_res[ring_at(g, u, i, ch)] = ku[(size_t)(n_q + i) * D + ch];
        c->v_res[ring_at(g, u, i, ch)] = vu[(size_t)(n_q + i) * D + ch];
      }
  }
  c->n_q = n_q;
  c->n_res = r;
  c->res_start = 0;
  return 0;
}

/* ------------------------------------------------------ append / flush --- */

/* k_new, v_new: bf16 [B][H][D].  Returns 0, or -1 if the ring is full. */
int kivio_append(const kivio_geom *g, kivio_cache *c, const uint16_t *k_new,
                 const uint16_t *v_new) {
  const int D = g->head_dim, slots = ring_slots(g);
  if (c->n_res >= slots) return -1;
  const int slot = (c->res_start + c->n_res) % slots;
  for (size_t u = 0; u < unit_count(g); ++u)
    for (int ch = 0; ch < D; ++ch) {
      c->k_res[ring_at(g, u, slot, ch)] = k_new[u * D + ch];
      c->v_res[ring_at(g, u, slot, ch)] = v_new[u * D + ch];
    }
  c->n_res += 1;
  return 0;
}

/* Quantise the G oldest residual tokens iff the ring is full.  Returns 1 if
 * it flushed, 0 if not, -1 if the history is full. */
int kivio_flush(const kivio_geom *g, kivio_cache *c) {
  const int G = g->group, slots = ring_slots(g);
  if (c->n_res != slots) return 0;
  if (c->n_q + G > g->max_tokens) return -1;
  const uint16_t *rows_k[64], *rows_v[64];
  for (size_t u = 0; u < unit_count(g); ++u) {
    for (int i = 0; i < G; ++i) {
      int slot = (c->res_start + i) % slots;
      rows_k[i] = c->k_res + ring_at(g, u, slot, 0);
      rows_v[i] = c->v_res + ring_at(g, u, slot, 0);
    }
    quantize_group(g, c, u, c->n_q / G, rows_k, rows_v);
  }
  c->n_q += G;
  c->n_res -= G;
  c->res_start = (c->res_start + G) % slots;
  return 1;
}

/* -------------------------------------------------------- dequantise --- */

/* All cached keys and values of unit u as doubles, token-major [n][D]:
 * rows 0..n_q-1 are the dequantised history (code * scale + zero), rows
 * n_q..n_q+n_res-1 the residual in logical order (oldest first). */
void kivio_dequant_unit(const kivio_geom *g, const kivio_cache *c, long unit,
                        double *k_out, double *v_out) {
  const int G = g->group, D = g->head_dim, b = g->bits, slots = ring_slots(g);
  const size_t u = (size_t)unit;
  for (int t = 0; t < c->n_q; ++t) {
    const int gi = t / G, i = t % G;
    for (int ch = 0; ch < D; ++ch) {
      uint8_t kc = get_code(k_row(g, c, u, t), (size_t)ch, b);
      k_out[(size_t)t * D + ch] = (double)kc * meta_scale(g, c, 0, k_meta(g, u, gi, ch)) +
                                  meta_zero(g, c, 0, k_meta(g, u, gi, ch));
      uint8_t vc = get_code(v_cell(g, c, u, gi, i / 8, ch), (size_t)(i % 8), b);
      const int j = ch / G;
      v_out[(size_t)t * D + ch] = (double)vc * meta_scale(g, c, 1, v_meta(g, u, gi, j, i)) +
                                  meta_zero(g, c, 1, v_meta(g, u, gi, j, i));
    }
  }
  for (int i = 0; i < c->n_res; ++i) {
    const int slot = (c->res_start + i) % slots;
    for (int ch = 0; ch < D; ++ch) {
      k_out[(size_t)(c->n_q + i) * D + ch] = bf16_to_float(c->k_res[ring_at(g, u, slot, ch)]);
      v_out[(size_t)(c->n_q + i) * D + ch] = bf16_to_float(c->v_res[ring_at(g, u, slot, ch)]);
    }
  }
}

/* ---------------------------------------------------------- attention --- */

/* Softmax attention of one query row over n cached tokens (doubles):
 * score_t = scale * sum_c q_c k_tc ; p = softmax(score) ; o = sum_t p_t v_t. */
void kivio_attend_row(const double *q, const double *k, const double *v, int n, int d,
                      double scale, double *o) {
  double *score = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  double m = -INFINITY;
  for (int t = 0; t < n; ++t) {
    double acc = 0.0;
    for (int ch = 0; ch < d; ++ch) acc += q[ch] * k[(size_t)t * d + ch];
    score[t] = scale * acc;
    if (score[t] > m) m = score[t];
  }
  double den = 0.0;
  for (int t = 0; t < n; ++t) {
    score[t] = exp(score[t] - m);
    den += score[t];
  }
  for (int ch = 0; ch < d; ++ch) o[ch] = 0.0;
  for (int t = 0; t < n; ++t)
    for (int ch = 0; ch < d; ++ch) o[ch] += score[t] * v[(size_t)t * d + ch];
  for (int ch = 0; ch < d; ++ch) o[ch] /= den;
  free(score);
}

/* Decode attention for the query heads of unit u = b*H + h:
 * q: bf16 [B][H*QPK][D] (whole tensor), out: float [B][H*QPK][D] (only the
 * QPK rows of this unit are written).  Returns 0, -1 on an empty cache. */
int kivio_attention_unit(const kivio_geom *g, const kivio_cache *c, long unit,
                         const uint16_t *q, float scale, float *out) {
  const int D = g->head_dim, QPK = g->q_per_kv;
  const int n = c->n_q + c->n_res;
  if (n <= 0) return -1;
  double *kk = (double *)malloc((size_t)n * D * sizeof(double));
  double *vv = (double *)malloc((size_t)n * D * sizeof(double));
  double qd[256], od[256];
  kivio_dequant_unit(g, c, unit, kk, vv);
  const long b = unit / g->kv_heads, h = unit % g->kv_heads;
  for (int j = 0; j < QPK; ++j) {
    const size_t row = ((size_t)b * g->kv_heads * QPK + (size_t)h * QPK + (size_t)j) * D;
    for (int ch = 0; ch < D; ++ch) qd[ch] = bf16_to_float(q[row + ch]);
    kivio_attend_row(qd, kk, vv, n, D, (double)scale, od);
    for (int ch = 0; ch < D; ++ch) out[row + ch] = (float)od[ch];
  }
  free(kk);
  free(vv);
  return 0;
}

/* All units, one after another. */
int kivio_attention(const kivio_geom *g, const kivio_cache *c, const uint16_t *q,
                    float scale, float *out) {
  for (size_t u = 0; u < unit_count(g); ++u)
    if (kivio_attention_unit(g, c, (long)u, q, scale, out) != 0) return -1;
  return 0;
}

/* Decode attention over an uncompressed bf16 cache, the baseline the pages
 * measure KIVI against (card: "compared with FP16"; catalog record,
 * Methodology: throughput gain over the FP16 cache).  k, v: bf16
 * [B][H][stride][D]; the first seq_len tokens of each unit are attended.
 * q: bf16 [B][H*QPK][D]; out: float [B][H*QPK][D], only the QPK rows of unit
 * u = b*H + h are written.  Plain softmax attention in doubles.  Returns 0,
 * -1 when seq_len is out of [1, stride]. */
int kivio_attention_dense_unit(const kivio_geom *g, const uint16_t *k, const uint16_t *v,
                               int seq_len, int stride, long unit, const uint16_t *q,
                               float scale, float *out) {
  const int D = g->head_dim, QPK = g->q_per_kv;
  if (seq_len < 1 || seq_len > stride) return -1;
  double *kk = (double *)malloc((size_t)seq_len * D * sizeof(double));
  double *vv = (double *)malloc((size_t)seq_len * D * sizeof(double));
  double qd[256], od[256];
  const size_t base = (size_t)unit * stride * D;
  for (size_t i = 0; i < (size_t)seq_len * D; ++i) {
    kk[i] = bf16_to_float(k[base + i]);
    vv[i] = bf16_to_float(v[base + i]);
  }
  const long b = unit / g->kv_heads, h = unit % g->kv_heads;
  for (int j = 0; j < QPK; ++j) {
    const size_t row = ((size_t)b * g->kv_heads * QPK + (size_t)h * QPK + (size_t)j) * D;
    for (int ch = 0; ch < D; ++ch) qd[ch] = bf16_to_float(q[row + ch]);
    kivio_attend_row(qd, kk, vv, seq_len, D, (double)scale, od);
    for (int ch = 0; ch < D; ++ch) out[row + ch] = (float)od[ch];
  }
  free(kk);
  free(vv);
  return 0;
}

/* ---------------------------------------------------- byte arithmetic --- */

/* KV-cache bytes per token of a model with `layers` layers, `kv_heads` kv
 * heads of `head_dim` channels, at context `ctx`, under four conventions:
 *  out[0] bf16 cache: layers*kv_heads*head_dim*2 (K+V)*2 bytes;
 *  out[1] catalog convention (catalog record, KV bytes basis): grouped term
 *         layers*kv_heads*head_dim*2*bits/8 counted at the full context, plus
 *         the bf16 residual of R tokens spread over the context;
 *  out[2] exact stored codes: the grouped term covers ctx-R tokens only;
 *  out[3] bytes this cache layout stores, scale and zero included (two fp32
 *         per group of G in K and in V), with the prefill split
 *         n_q = G*floor((ctx-R)/G) and n_q stored tokens + (ctx-n_q) bf16;
 *  out[4] the same with the 16-bit scale/zero format (fp16 scale, bf16
 *         zero). */
void kivio_bytes_per_token(int layers, int kv_heads, int head_dim, int bits, int group,
                           int residual, int ctx, double out[5]) {
  const double lhd = (double)layers * kv_heads * head_dim;
  const double bf16 = lhd * 2.0 * 2.0;
  const double grouped = lhd * 2.0 * bits / 8.0;
  const double resid = (double)residual * bf16 / (double)ctx;
  out[0] = bf16;
  out[1] = grouped + resid;
  out[2] = grouped * (double)(ctx - residual) / (double)ctx + resid;
  const int n_q = kivio_prefill_split(ctx, group, residual);
  const double per_q_token = lhd * (2.0 * bits / 8.0 + 2.0 * 2.0 * 4.0 / group);
  out[3] = ((double)n_q * per_q_token + (double)(ctx - n_q) * bf16) / (double)ctx;
  const double per_q_token16 = lhd * (2.0 * bits / 8.0 + 2.0 * 2.0 * 2.0 / group);
  out[4] = ((double)n_q * per_q_token16 + (double)(ctx - n_q) * bf16) / (double)ctx;
}
