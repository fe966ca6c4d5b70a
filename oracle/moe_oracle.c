/*
 * moe_oracle.c -- plain fp64 CPU oracle of the routed MoE feed-forward layer
 * (Step-5-Preview shape).  TEST INFRASTRUCTURE ONLY: loaded by the tests, the
 * smoke check and the benchmark's CPU-baseline leg, never by the product path.
 *
 * Sources of each step (pages as titled):
 *  - "Step-5-Preview" (NeMo AutoModel model coverage), section "Model
 *    Architecture": 352 routed experts per MoE layer, top-8 routing, one
 *    shared expert, intermediate size 1,536 for every expert, hidden 4,096,
 *    a learned router.  The parameter count in the paragraph after that table
 *    implies three hidden x intermediate matrices per expert (a gated FFN).
 *  - "Step-5 minimal inference" (inference README), introduction and the
 *    "Contents" table: block-scaled FP8 expert GEMM; section "Install": FP8
 *    E4M3; section "Long-output stability": partial results added in a fixed
 *    order with FP32 accumulation.
 *  - Where the pages are silent (score function, renormalisation, block
 *    sizes, activation, tie-break, layouts) the readings are: softmax over
 *    the experts then renormalised over the top-k (equivalently a softmax over
 *    the k chosen logits), SwiGLU, 128x128 weight blocks and 1x128 per-token
 *    activation groups with a multiplying fp32 scale, lowest expert index
 *    first on exact ties, slots in ascending expert id.
 *
 * Every loop below is the definition written out: sequential fp64 sums, no
 * blocking and no reordering.  OpenMP only splits independent tokens/rows.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Codecs                                                                    */
/* ------------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32: widen by appending 16 zero bits. */
double oref_bf16_decode(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* binary32 -> bf16, round to nearest, ties to even: drop the low 16 bits
 * after adding half an ulp (0x7FFF) plus the lowest kept bit.  NaN stays NaN. */
uint16_t oref_bf16_encode(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* OCP 8-bit E4M3 (FN variant): sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no
 * infinities; largest finite 448 (S.1111.110). */
static double e4m3_table[256];

__attribute__((constructor)) static void e4m3_build_table(void) {
  for (int c = 0; c < 256; ++c) {
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
      v = NAN;
    else if (e == 0)
      v = ldexp((double)m, -9);
    else
      v = ldexp(1.0 + m / 8.0, e - 7);
    e4m3_table[c] = s ? -v : v;
  }
}

static inline const double *e4m3_tab(void) { return e4m3_table; }

double oref_e4m3_decode(uint8_t c) { return e4m3_tab()[c]; }

/* OCP 4-bit E2M1 (the element type of MX FP4): sign, 2 exponent bits (bias
 * 1), 1 mantissa bit; exponent field 0 is subnormal (m * 2^-1); no NaN or
 * infinity; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Only the low nibble of c
 * is read. */
double oref_e2m1_decode(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* OCP E8M0 scale: an unsigned biased exponent, 2^(e - 127); 0xFF is NaN. */
double oref_e8m0_decode(uint8_t e) { return e == 0xFF ? NAN : ldexp(1.0, (int)e - 127); }

/* Round a binary32 value to E4M3: nearest representable value, ties to the
 * even mantissa; magnitudes beyond 448 saturate to 448.  Arithmetic in double
 * is exact here (a power-of-two rescale of a binary32). */
uint8_t oref_e4m3_encode(float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  if (isnan(v)) return (uint8_t)(sign | 0x7F);
  double a = fabs((double)v);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: value = m * 2^-9, m in 0..7; m == 8 is the smallest
     * normal (code 0x08), which the encoding below gives automatically. */
    double m = nearbyint(a * 512.0);
    return (uint8_t)(sign | (uint8_t)m);
  }
  int ex;
  frexp(a, &ex);   /* a = f * 2^ex, f in [0.5, 1) -> a = (2f) * 2^(ex-1) */
  int e = ex - 1;  /* unbiased exponent, -6..8 */
  double frac = ldexp(a, -e) - 1.0;   /* in [0, 1) */
  double m = nearbyint(frac * 8.0);   /* ties to even (default rounding mode) */
  if (m == 8.0) { m = 0.0; e += 1; }
  int code = ((e + 7) << 3) | (int)m;
  if (code > 0x7E) code = 0x7E;       /* 448 < a < 464 rounds down to 448 anyway */
  return (uint8_t)(sign | code);
}

/* 1x128 group quantisation, decisions in binary32 as the GPU takes them. */
void oref_quant_row(const float *v, int64_t n, uint8_t *q, float *s) {
  for (int64_t g = 0; g < n / 128; ++g) {
    float amax = 0.0f;
    for (int j = 0; j < 128; ++j) {
      float a = fabsf(v[g * 128 + j]);
      if (a > amax) amax = a;
    }
    volatile float sc = amax / 448.0f;   /* IEEE binary32 division */
    float scale = (amax == 0.0f) ? 1.0f : sc;
    s[g] = scale;
    for (int j = 0; j < 128; ++j) {
      volatile float r = v[g * 128 + j] / scale;
      q[g * 128 + j] = oref_e4m3_encode(r);
    }
  }
}

void oref_e4m3_encode_array(const float *v, int64_t n, uint8_t *q) {
  for (int64_t i = 0; i < n; ++i) q[i] = oref_e4m3_encode(v[i]);
}

void oref_bf16_encode_array(const double *v, int64_t n, uint16_t *b) {
  for (int64_t i = 0; i < n; ++i) b[i] = oref_bf16_encode(v[i]);
}

void oref_quant_bf16_rows(const uint16_t *x, int64_t rows, int64_t n, uint8_t *q, float *s) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t r = 0; r < rows; ++r) {
    float *v = (float *)malloc(sizeof(float) * (size_t)(n + 1));
    for (int64_t h = 0; h < n; ++h) v[h] = (float)oref_bf16_decode(x[r * n + h]);
    oref_quant_row(v, n, q + r * n, s + r * (n / 128));
    free(v);
  }
}

/* ------------------------------------------------------------------------ */
/* Routing                                                                   */
/* ------------------------------------------------------------------------ */

static void token_logits(const oref_layer *L, const uint16_t *xr, double *l) {
  const int H = L->hidden, E = L->num_experts;
  for (int e = 0; e < E; ++e) {
    const uint16_t *w = L->w_router + (int64_t)e * H;
    double acc = 0.0;
    for (int h = 0; h < H; ++h) acc += oref_bf16_decode(xr[h]) * oref_bf16_decode(w[h]);
    if (L->router_bias) acc += (double)L->router_bias[e];
    l[e] = acc;
  }
}

/* The value a logit is ranked by: a NaN logit ranks as -infinity (below every
 * number; among equal values the lower expert index comes first). */
static inline double rank_value(double v) { return isnan(v) ? -INFINITY : v; }

/* k largest of l[0..E) ordered by (value desc, index asc); then slots sorted
 * by ascending expert id.  Returns the gap l_(k) - l_(k+1) (0 when the two
 * are equal, infinities included). */
static double select_topk(const double *l, int E, int k, int32_t *ids) {
  char *taken = (char *)calloc((size_t)E, 1);
  double kth = 0.0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || rank_value(l[e]) > rank_value(l[best])) best = e;   /* strict: lower index keeps ties */
    }
    taken[best] = 1;
    ids[j] = best;
    kth = rank_value(l[best]);
  }
  double next = -INFINITY;
  int have_next = 0;
  for (int e = 0; e < E; ++e)
    if (!taken[e] && (!have_next || rank_value(l[e]) > next)) { next = rank_value(l[e]); have_next = 1; }
  free(taken);
  /* insertion sort of the k chosen ids, ascending */
  for (int a = 1; a < k; ++a) {
    int32_t v = ids[a];
    int b = a - 1;
    while (b >= 0 && ids[b] > v) { ids[b + 1] = ids[b]; --b; }
    ids[b + 1] = v;
  }
  if (!have_next) return INFINITY;
  return kth == next ? 0.0 : kth - next;   /* equal values, infinite ones too: a tie */
}

/* softmax over the chosen logits == full softmax renormalised over them.
 * Logits are taken at their rank value (NaN as -infinity); a logit equal to
 * the largest chosen one weighs exp(0) = 1, which extends the formula to
 * infinite logits: k chosen -infinity logits (a token whose logits are all
 * NaN) share the gate equally, 1/k each. */
static void softmax_chosen(const double *l, const int32_t *ids, int k, double *g) {
  double mx = -INFINITY;
  for (int j = 0; j < k; ++j) if (rank_value(l[ids[j]]) > mx) mx = rank_value(l[ids[j]]);
  double den = 0.0;
  for (int j = 0; j < k; ++j) {
    const double v = rank_value(l[ids[j]]);
    g[j] = v == mx ? 1.0 : exp(v - mx);
    den += g[j];
  }
  for (int j = 0; j < k; ++j) g[j] /= den;
}

static inline int64_t tok_of(const int64_t *list, int64_t i) { return list ? list[i] : i; }

void oref_route(const oref_layer *L, const uint16_t *x, int64_t T,
                const int64_t *token_list, int64_t n_list,
                int32_t *ids, double *gates, double *logits, double *gap) {
  const int H = L->hidden, E = L->num_experts, k = L->top_k;
  if (!token_list) n_list = T;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t i = 0; i < n_list; ++i) {
    int64_t t = tok_of(token_list, i);
    double *l = (double *)malloc(sizeof(double) * (size_t)E);
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    double *g = (double *)malloc(sizeof(double) * (size_t)k);
    token_logits(L, x + t * H, l);
    double gp = select_topk(l, E, k, sel);
    softmax_chosen(l, sel, k, g);
    for (int j = 0; j < k; ++j) {
      if (ids) ids[i * k + j] = sel[j];
      if (gates) gates[i * k + j] = g[j];
    }
    if (logits) memcpy(logits + i * E, l, sizeof(double) * (size_t)E);
    if (gap) gap[i] = gp;
    free(l); free(sel); free(g);
  }
}

void oref_gates_for_ids(const oref_layer *L, const uint16_t *x, int64_t T,
                        const int64_t *token_list, int64_t n_list,
                        const int32_t *ids, double *gates) {
  const int H = L->hidden, E = L->num_experts, k = L->top_k;
  if (!token_list) n_list = T;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t i = 0; i < n_list; ++i) {
    double *l = (double *)malloc(sizeof(double) * (size_t)E);
    token_logits(L, x + tok_of(token_list, i) * H, l);
    softmax_chosen(l, ids + i * k, k, gates + i * k);
    free(l);
  }
}

/* ------------------------------------------------------------------------ */
/* Grouping: stable counting sort                                            */
/* ------------------------------------------------------------------------ */

int64_t oref_permute(const int32_t *key, int64_t N, int32_t E,
                     int32_t *offsets, int32_t *perm_src, int32_t *perm_pos) {
  int64_t dropped = 0;
  for (int32_t e = 0; e <= E; ++e) offsets[e] = 0;
  for (int64_t i = 0; i < N; ++i) {
    if (key[i] < 0 || key[i] >= E) { ++dropped; continue; }
    offsets[key[i] + 1] += 1;
  }
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
  int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  for (int32_t e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int64_t i = 0; i < N; ++i) {
    if (key[i] < 0 || key[i] >= E) { if (perm_pos) perm_pos[i] = -1; continue; }
    int32_t p = fill[key[i]]++;
    if (perm_src) perm_src[p] = (int32_t)i;
    if (perm_pos) perm_pos[i] = p;
  }
  free(fill);
  return dropped;
}

/* ------------------------------------------------------------------------ */
/* Expert FFN                                                                */
/* ------------------------------------------------------------------------ */

/* Dequantised weight element (row n, column c) of the [R, C] matrix of one
 * expert whose weights start at element (fp8: byte) base and whose scales
 * start at scale index sbase:
 *   bf16:  the bf16 value;
 *   fp8:   code * scale[n/128][c/128];
 *   mxfp4: e2m1(nibble c of row n) * 2^(scale[n][c/32] - 127), row n being
 *          C/2 bytes with input c in the low nibble of byte c/2 when c is even. */
static inline double w_elem(int fmt, const void *w, const void *s, int64_t base,
                            int64_t sbase, int64_t C, int64_t n, int64_t c) {
  if (fmt == OREF_FP8) {
    const uint8_t *q = (const uint8_t *)w;
    const float *sf = (const float *)s;
    return e4m3_tab()[q[base + n * C + c]] * (double)sf[sbase + (n / 128) * (C / 128) + c / 128];
  }
  if (fmt == OREF_MXFP4) {
    const uint8_t *q = (const uint8_t *)w;
    const uint8_t *se = (const uint8_t *)s;
    const uint8_t byte = q[base + n * (C / 2) + c / 2];
    const uint8_t code = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    return oref_e2m1_decode(code) * oref_e8m0_decode(se[sbase + n * (C / 32) + c / 32]);
  }
  const uint16_t *b = (const uint16_t *)w;
  return oref_bf16_decode(b[base + n * C + c]);
}

/* Start of expert e's weights (elements; bytes for the byte formats) and of
 * its scales (scale entries) in an [E, R, C] weight tensor. */
static inline int64_t w_base(int fmt, int64_t e, int64_t R, int64_t C) {
  return fmt == OREF_MXFP4 ? e * R * (C / 2) : e * R * C;
}
static inline int64_t s_base(int fmt, int64_t e, int64_t R, int64_t C) {
  if (fmt == OREF_FP8) return e * (R / 128) * (C / 128);
  if (fmt == OREF_MXFP4) return e * R * (C / 32);
  return 0;
}

static inline double silu(double z) { return z / (1.0 + exp(-z)); }

/* Gated FFN on a dequantised input row a[H]:
 *   zg[n] = sum_h a[h] Wg[n,h],  zu[n] = sum_h a[h] Wu[n,h]
 *   h = silu(zg) * zu, stored as h_fp8 ? e4m3 + 1x128 scales : bf16
 *   out[c] = sum_i h[i] Wd[c,i]                                           */
static void gated_ffn(int H, int I, int w_fmt, int h_fp8,
                      const void *wgu, const void *sgu, int64_t gu_base, int64_t sgu_base,
                      const void *wd, const void *sd, int64_t d_base, int64_t sd_base,
                      const double *a, double *out, double *out_h) {
  double *hs = (double *)malloc(sizeof(double) * (size_t)I);
  float *hf = (float *)calloc((size_t)I + 1, sizeof(float));
  for (int n = 0; n < I; ++n) {
    double zg = 0.0, zu = 0.0;
    for (int h = 0; h < H; ++h) zg += a[h] * w_elem(w_fmt, wgu, sgu, gu_base, sgu_base, H, n, h);
    for (int h = 0; h < H; ++h) zu += a[h] * w_elem(w_fmt, wgu, sgu, gu_base, sgu_base, H, (int64_t)I + n, h);
    hf[n] = (float)(silu(zg) * zu);   /* the value the layer holds before storing h */
  }
  if (h_fp8) {
    uint8_t *q = (uint8_t *)malloc((size_t)I);
    float *sc = (float *)malloc(sizeof(float) * (size_t)(I / 128));
    oref_quant_row(hf, I, q, sc);
    for (int n = 0; n < I; ++n) hs[n] = e4m3_tab()[q[n]] * (double)sc[n / 128];
    free(q); free(sc);
  } else {
    for (int n = 0; n < I; ++n) hs[n] = oref_bf16_decode(oref_bf16_encode((double)hf[n]));
  }
  if (out_h) memcpy(out_h, hs, sizeof(double) * (size_t)I);
  for (int c = 0; c < H; ++c) {
    double acc = 0.0;
    for (int i = 0; i < I; ++i) acc += hs[i] * w_elem(w_fmt, wd, sd, d_base, sd_base, I, c, i);
    out[c] = acc;
  }
  free(hs); free(hf);
}

static void dequant_input(const oref_layer *L, const void *a, const float *a_scale, double *ad) {
  const int H = L->hidden;
  if (L->expert_format != OREF_BF16) {
    const uint8_t *q = (const uint8_t *)a;
    for (int h = 0; h < H; ++h) ad[h] = e4m3_tab()[q[h]] * (double)a_scale[h / 128];
  } else {
    const uint16_t *b = (const uint16_t *)a;
    for (int h = 0; h < H; ++h) ad[h] = oref_bf16_decode(b[h]);
  }
}

void oref_expert_row(const oref_layer *L, int32_t e, const void *a, const float *a_scale,
                     double *out, double *out_h) {
  const int64_t H = L->hidden, I = L->inter;
  double *ad = (double *)malloc(sizeof(double) * (size_t)H);
  dequant_input(L, a, a_scale, ad);
  const int fmt = L->expert_format;
  gated_ffn((int)H, (int)I, fmt, fmt != OREF_BF16,
            L->w_gate_up, L->s_gate_up, w_base(fmt, e, 2 * I, H), s_base(fmt, e, 2 * I, H),
            L->w_down, L->s_down, w_base(fmt, e, H, I), s_base(fmt, e, H, I),
            ad, out, out_h);
  free(ad);
}

void oref_expert_gate_up_factored(const oref_layer *L, int32_t e, const uint8_t *a,
                                  const float *a_scale, double *zg, double *zu) {
  const int64_t H = L->hidden, I = L->inter, KB = H / 128;
  const uint8_t *w = (const uint8_t *)L->w_gate_up + (int64_t)e * 2 * I * H;
  const float *s = (const float *)L->s_gate_up + (int64_t)e * (2 * I / 128) * KB;
  for (int64_t r = 0; r < 2 * I; ++r) {
    double acc = 0.0;
    for (int64_t kb = 0; kb < KB; ++kb) {
      double part = 0.0;
      for (int64_t k = kb * 128; k < kb * 128 + 128; ++k)
        part += e4m3_tab()[a[k]] * e4m3_tab()[w[r * H + k]];
      acc += (double)a_scale[kb] * (double)s[(r / 128) * KB + kb] * part;
    }
    if (r < I) zg[r] = acc; else zu[r - I] = acc;
  }
}

void oref_expert_gate_up_mx_factored(const oref_layer *L, int32_t e, const uint8_t *a,
                                     const float *a_scale, double *zg, double *zu) {
  const int64_t H = L->hidden, I = L->inter;
  const uint8_t *w = (const uint8_t *)L->w_gate_up + (int64_t)e * 2 * I * (H / 2);
  const uint8_t *s = (const uint8_t *)L->s_gate_up + (int64_t)e * 2 * I * (H / 32);
  for (int64_t r = 0; r < 2 * I; ++r) {
    double acc = 0.0;
    for (int64_t kg = 0; kg < H / 128; ++kg) {
      double group = 0.0;
      for (int64_t kb = 4 * kg; kb < 4 * kg + 4; ++kb) {
        double part = 0.0;
        for (int64_t k = 32 * kb; k < 32 * kb + 32; k += 2) {
          const uint8_t byte = w[r * (H / 2) + k / 2];
          part += e4m3_tab()[a[k]] * oref_e2m1_decode(byte & 0x0F);
          part += e4m3_tab()[a[k + 1]] * oref_e2m1_decode(byte >> 4);
        }
        group += oref_e8m0_decode(s[r * (H / 32) + kb]) * part;
      }
      acc += (double)a_scale[kg] * group;
    }
    if (r < I) zg[r] = acc; else zu[r - I] = acc;
  }
}

void oref_expert_gate_up_dequant(const oref_layer *L, int32_t e, const uint8_t *a,
                                 const float *a_scale, double *zg, double *zu) {
  const int64_t H = L->hidden, I = L->inter;
  const int fmt = L->expert_format;
  double *ad = (double *)malloc(sizeof(double) * (size_t)H);
  for (int64_t h = 0; h < H; ++h) ad[h] = e4m3_tab()[a[h]] * (double)a_scale[h / 128];
  for (int64_t r = 0; r < 2 * I; ++r) {
    double acc = 0.0;
    for (int64_t h = 0; h < H; ++h)
      acc += ad[h] * w_elem(fmt, L->w_gate_up, L->s_gate_up, w_base(fmt, e, 2 * I, H),
                            s_base(fmt, e, 2 * I, H), H, r, h);
    if (r < I) zg[r] = acc; else zu[r - I] = acc;
  }
  free(ad);
}

void oref_shared_row(const oref_layer *L, const uint16_t *x_row, double *out) {
  const int H = L->hidden, Is = L->shared_inter;
  if (Is <= 0 || !L->w_shared_gate_up) { for (int c = 0; c < H; ++c) out[c] = 0.0; return; }
  double *ad = (double *)malloc(sizeof(double) * (size_t)H);
  for (int h = 0; h < H; ++h) ad[h] = oref_bf16_decode(x_row[h]);
  gated_ffn(H, Is, 0, 0, L->w_shared_gate_up, NULL, 0, 0, L->w_shared_down, NULL, 0, 0, ad, out, NULL);
  free(ad);
}

void oref_expert_ffn(const oref_layer *L, const int32_t *offsets, const void *a_rows,
                     const float *a_scale, int64_t N, double *out) {
  const int64_t H = L->hidden, E = L->num_experts, G = H / 128;
  const int fp8 = L->expert_format != OREF_BF16;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t p = 0; p < N; ++p) {
    int32_t e = -1;
    for (int64_t j = 0; j < E; ++j)
      if (p >= offsets[j] && p < offsets[j + 1]) { e = (int32_t)j; break; }
    if (e < 0) { for (int64_t c = 0; c < H; ++c) out[p * H + c] = 0.0; continue; }
    const void *row = fp8 ? (const void *)((const uint8_t *)a_rows + p * H)
                          : (const void *)((const uint16_t *)a_rows + p * H);
    oref_expert_row(L, e, row, fp8 ? a_scale + p * G : NULL, out + p * H, NULL);
  }
}

/* ------------------------------------------------------------------------ */
/* Whole layer                                                               */
/* ------------------------------------------------------------------------ */

/* y = shared(x_t) + sum_j g_j FFN_{ids_j}(x_t) for one token. */
static void token_output(const oref_layer *L, const uint16_t *xr, const int32_t *ids,
                         const double *g, int nsel, double *y) {
  const int H = L->hidden, G = H / 128;
  double *o = (double *)malloc(sizeof(double) * (size_t)H);
  oref_shared_row(L, xr, y);
  uint8_t *q = NULL;
  float *sc = NULL;
  if (L->expert_format != OREF_BF16) {
    float *xf = (float *)malloc(sizeof(float) * (size_t)H);
    for (int h = 0; h < H; ++h) xf[h] = (float)oref_bf16_decode(xr[h]);
    q = (uint8_t *)malloc((size_t)H);
    sc = (float *)malloc(sizeof(float) * (size_t)G);
    oref_quant_row(xf, H, q, sc);
    free(xf);
  }
  for (int j = 0; j < nsel; ++j) {
    if (ids[j] < 0 || ids[j] >= L->num_experts) continue;
    oref_expert_row(L, ids[j], q ? (const void *)q : (const void *)xr, sc, o, NULL);
    for (int c = 0; c < H; ++c) y[c] += g[j] * o[c];
  }
  free(o); free(q); free(sc);
}

void oref_forward(const oref_layer *L, const uint16_t *x, int64_t T,
                  const int64_t *token_list, int64_t n_list, double *y,
                  int32_t *ids, double *gates, double *gap) {
  const int H = L->hidden, k = L->top_k;
  if (!token_list) n_list = T;
  int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_list * k + 1));
  double *g = (double *)malloc(sizeof(double) * (size_t)(n_list * k + 1));
  oref_route(L, x, T, token_list, n_list, sel, g, NULL, gap);
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t i = 0; i < n_list; ++i)
    token_output(L, x + tok_of(token_list, i) * H, sel + i * k, g + i * k, k, y + i * H);
  if (ids) memcpy(ids, sel, sizeof(int32_t) * (size_t)(n_list * k));
  if (gates) memcpy(gates, g, sizeof(double) * (size_t)(n_list * k));
  free(sel); free(g);
}

void oref_forward_with_ids(const oref_layer *L, const uint16_t *x, int64_t T,
                           const int64_t *token_list, int64_t n_list,
                           const int32_t *ids, double *y) {
  const int H = L->hidden, k = L->top_k;
  if (!token_list) n_list = T;
  double *g = (double *)malloc(sizeof(double) * (size_t)(n_list * k + 1));
  oref_gates_for_ids(L, x, T, token_list, n_list, ids, g);
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t i = 0; i < n_list; ++i)
    token_output(L, x + tok_of(token_list, i) * H, ids + i * k, g + i * k, k, y + i * H);
  free(g);
}

void oref_forward_triples(const oref_layer *L, const uint16_t *x, int64_t T,
                          const int32_t *tok, const int32_t *expert, const float *gate, int64_t N,
                          const int64_t *token_list, int64_t n_list, double *y) {
  const int H = L->hidden;
  if (!token_list) n_list = T;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t li = 0; li < n_list; ++li) {
    int64_t t = tok_of(token_list, li);
    int64_t cnt = 0;
    for (int64_t i = 0; i < N; ++i) if (tok[i] == t) ++cnt;
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cnt + 1));
    double *g = (double *)malloc(sizeof(double) * (size_t)(cnt + 1));
    int64_t c = 0;
    for (int64_t i = 0; i < N; ++i)
      if (tok[i] == t) { ids[c] = expert[i]; g[c] = (double)gate[i]; ++c; }
    token_output(L, x + t * H, ids, g, (int)cnt, y + li * H);
    free(ids); free(g);
  }
}

void oref_combine(const double *y_perm, const int32_t *perm_pos, const int32_t *tok,
                  int32_t k, const float *gate, int64_t N, const double *shared,
                  int64_t T, int64_t H, double *y) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < H; ++c) y[t * H + c] = shared ? shared[t * H + c] : 0.0;
  for (int64_t i = 0; i < N; ++i) {
    int64_t t = tok ? tok[i] : i / k;
    if (t < 0 || t >= T || perm_pos[i] < 0) continue;
    const double *o = y_perm + (int64_t)perm_pos[i] * H;
    for (int64_t c = 0; c < H; ++c) y[t * H + c] += (double)gate[i] * o[c];
  }
}

/* ------------------------------------------------------------------------ */
/* Backward (bf16 experts)                                                   */
/* ------------------------------------------------------------------------ */

/* One expert's forward and backward for one token a[H] with output gradient
 * d_o[H] (already multiplied by the gate):
 *   zg = a Wg^T, zu = a Wu^T, h = silu(zg) zu, o = h Wd^T       (returned: o)
 *   dh = d_o Wd, dzu = dh silu(zg), dzg = dh zu silu'(zg),
 *   silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)
 *   da += dzg Wg + dzu Wu;  dWd += d_o (x) h;  dWg += dzg (x) a;  dWu += dzu (x) a.
 * Weight gradients accumulate into dwgu [2I, H] and dwd [H, I] (may be NULL). */
static void expert_backward(int H, int I, const uint16_t *wgu, const uint16_t *wd, const double *a,
                            const double *d_o, double *o, double *da, double *dwgu, double *dwd) {
  double *zg = (double *)malloc(sizeof(double) * (size_t)I * 5);
  double *zu = zg + I, *hh = zu + I, *dzg = hh + I, *dzu = dzg + I;
  for (int n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < H; ++h) {
      g += a[h] * oref_bf16_decode(wgu[(int64_t)n * H + h]);
      u += a[h] * oref_bf16_decode(wgu[(int64_t)(I + n) * H + h]);
    }
    zg[n] = g; zu[n] = u; hh[n] = silu(g) * u;
  }
  if (o)
    for (int c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int n = 0; n < I; ++n) acc += hh[n] * oref_bf16_decode(wd[(int64_t)c * I + n]);
      o[c] = acc;
    }
  for (int n = 0; n < I; ++n) {
    double dh = 0.0;
    for (int c = 0; c < H; ++c) dh += d_o[c] * oref_bf16_decode(wd[(int64_t)c * I + n]);
    const double sg = 1.0 / (1.0 + exp(-zg[n]));
    dzu[n] = dh * zg[n] * sg;
    dzg[n] = dh * zu[n] * sg * (1.0 + zg[n] * (1.0 - sg));
  }
  for (int h = 0; h < H; ++h) {
    double acc = 0.0;
    for (int n = 0; n < I; ++n)
      acc += dzg[n] * oref_bf16_decode(wgu[(int64_t)n * H + h]) + dzu[n] * oref_bf16_decode(wgu[(int64_t)(I + n) * H + h]);
    da[h] += acc;
  }
  if (dwd)
    for (int c = 0; c < H; ++c)
      for (int n = 0; n < I; ++n) dwd[(int64_t)c * I + n] += d_o[c] * hh[n];
  if (dwgu)
    for (int n = 0; n < I; ++n)
      for (int h = 0; h < H; ++h) {
        dwgu[(int64_t)n * H + h] += dzg[n] * a[h];
        dwgu[(int64_t)(I + n) * H + h] += dzu[n] * a[h];
      }
  free(zg);
}

void oref_backward(const oref_layer *L, const uint16_t *x, int64_t T, const int32_t *ids,
                   const uint16_t *dy, const int64_t *token_list, int64_t n_list,
                   double *dx, double *dwgu, double *dwd, double *dwsgu, double *dwsd,
                   double *dwr, double *dbias) {
  const int H = L->hidden, I = L->inter, E = L->num_experts, k = L->top_k, Is = L->shared_inter;
  if (!token_list) n_list = T;
  if (dwgu) memset(dwgu, 0, sizeof(double) * (size_t)E * 2 * I * H);
  if (dwd) memset(dwd, 0, sizeof(double) * (size_t)E * H * I);
  if (dwsgu && Is > 0) memset(dwsgu, 0, sizeof(double) * (size_t)2 * Is * H);
  if (dwsd && Is > 0) memset(dwsd, 0, sizeof(double) * (size_t)H * Is);
  if (dwr) memset(dwr, 0, sizeof(double) * (size_t)E * H);
  if (dbias) memset(dbias, 0, sizeof(double) * (size_t)E);
  double *a = (double *)malloc(sizeof(double) * (size_t)H * 3);
  double *g_dy = a + H, *o = g_dy + H;
  double *l = (double *)malloc(sizeof(double) * (size_t)(E + 3 * k + 1));
  double *g = l + E, *dg = g + k, *dl = dg + k;
  /* tokens one after another: the weight gradients are sums over tokens */
  for (int64_t li = 0; li < n_list; ++li) {
    const int64_t t = tok_of(token_list, li);
    const uint16_t *xr = x + t * H;
    const int32_t *id = ids + t * k;
    double *dxt = dx + li * H;
    for (int h = 0; h < H; ++h) { a[h] = oref_bf16_decode(xr[h]); dxt[h] = 0.0; }
    /* gates: softmax over the chosen logits */
    token_logits(L, xr, l);
    double lmax = -INFINITY;
    for (int j = 0; j < k; ++j) if (l[id[j]] > lmax) lmax = l[id[j]];
    double den = 0.0;
    for (int j = 0; j < k; ++j) { g[j] = exp(l[id[j]] - lmax); den += g[j]; }
    for (int j = 0; j < k; ++j) g[j] /= den;
    /* routed experts: d_o = g_j dy_t; dg_j = <dy_t, o_j> */
    for (int j = 0; j < k; ++j) {
      const int e = id[j];
      for (int c = 0; c < H; ++c) g_dy[c] = g[j] * oref_bf16_decode(dy[t * H + c]);
      expert_backward(H, I, (const uint16_t *)L->w_gate_up + (int64_t)e * 2 * I * H,
                      (const uint16_t *)L->w_down + (int64_t)e * H * I, a, g_dy,
                      o, dxt, dwgu ? dwgu + (int64_t)e * 2 * I * H : NULL, dwd ? dwd + (int64_t)e * H * I : NULL);
      double acc = 0.0;
      for (int c = 0; c < H; ++c) acc += oref_bf16_decode(dy[t * H + c]) * o[c];
      dg[j] = acc;
    }
    /* softmax backward over the chosen logits, then the router */
    double sdg = 0.0;
    for (int j = 0; j < k; ++j) sdg += g[j] * dg[j];
    for (int j = 0; j < k; ++j) {
      dl[j] = g[j] * (dg[j] - sdg);
      const int e = id[j];
      const uint16_t *wr = L->w_router + (int64_t)e * H;
      for (int h = 0; h < H; ++h) dxt[h] += dl[j] * oref_bf16_decode(wr[h]);
      if (dwr) for (int h = 0; h < H; ++h) dwr[(int64_t)e * H + h] += dl[j] * a[h];
      if (dbias) dbias[e] += dl[j];
    }
    /* shared expert, unweighted */
    if (Is > 0 && L->w_shared_gate_up) {
      for (int c = 0; c < H; ++c) g_dy[c] = oref_bf16_decode(dy[t * H + c]);
      expert_backward(H, Is, L->w_shared_gate_up, L->w_shared_down, a, g_dy, NULL, dxt, dwsgu, dwsd);
    }
  }
  free(a); free(l);
}

int oref_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
