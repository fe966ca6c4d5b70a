/*
 * moe_oracle.h -- plain fp64 CPU oracle for the routed Mixture-of-Experts
 * feed-forward layer of Step-5-Preview.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path (the HIP
 * library under router_gemm_amd/) never links, loads or calls it, and the two
 * share no source: this file has its own bf16 and e4m3 codecs, its own
 * selection, permutation and FFN code.
 *
 * What the oracle computes is the plain per-token definition of the layer
 * (NeMo AutoModel "Step-5-Preview", section "Model Architecture": 352 routed
 * experts, top-8 routing, one shared expert, expert intermediate 1,536,
 * hidden 4,096; Step-5 minimal inference README, introduction: block-scaled
 * FP8 expert GEMM):
 *
 *   y[t] = Shared(x[t]) + sum_{e in TopK(t)} g[t,e] * FFN_e(x[t])
 *   FFN(a) = (silu(a W_g^T) * (a W_u^T)) W_d^T
 *
 * in fp64, with the quantisation points of the FP8 mode (1x128 per-token
 * activation groups, 128x128 weight blocks) applied where the layer stores a
 * value in a narrow format.  A third weight format, MX FP4 (E2M1 codes with
 * one power-of-two scale per 32 inputs), keeps the FP8 mode's activations.  Quantisation decisions (which fp8 code a value
 * gets) are taken in fp32, the precision the GPU takes them in.
 *
 * Parity status of each function is listed beside it; every function here is
 * pinned by the CPU tests (tests/test_oracle_*.py) against closed forms,
 * brute force, library routines or invariants.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layer description, host pointers.  Layouts (row-major, "out x in" like a
 * linear layer, y = a W^T):
 *   w_router        bf16 [E, H]
 *   router_bias     f32  [E] or NULL (added to the logits before selection)
 *   w_gate_up       [E, 2I, H]  rows 0..I-1 gate, rows I..2I-1 up
 *   s_gate_up       scales of w_gate_up (see below)
 *   w_down          [E, H, I]
 *   s_down          scales of w_down
 *   w_shared_gate_up bf16 [2Is, H], w_shared_down bf16 [H, Is]  (Is = 0: none)
 * expert_format:
 *   OREF_BF16  (0): expert weights are bf16 (uint16 bit patterns), no scales;
 *   OREF_FP8   (1): OCP E4M3FN bytes; s_gate_up f32 [E, 2I/128, H/128],
 *                   s_down f32 [E, H/128, I/128]; dequant = code * scale;
 *   OREF_MXFP4 (2): OCP MX FP4: E2M1 codes two to a byte, input 2j in the
 *                   low nibble of byte j ("TensorFold" pull-request page,
 *                   nvfp4 format notes: the same packing), so w_gate_up is
 *                   [E, 2I, H/2] and w_down [E, H, I/2] bytes; one E8M0
 *                   scale byte per 32 consecutive inputs of a row (OCP
 *                   Microscaling Formats specification v1.0): s_gate_up
 *                   uint8 [E, 2I, H/32], s_down uint8 [E, H, I/32];
 *                   dequant = e2m1(code) * 2^(scale - 127).
 * Activations and h are stored as E4M3 with 1x128 scales in both scaled
 * formats, as bf16 in bf16 mode. */
enum { OREF_BF16 = 0, OREF_FP8 = 1, OREF_MXFP4 = 2 };
typedef struct oref_layer {
  int32_t hidden, inter, num_experts, top_k, shared_inter;
  int32_t expert_format;
  const uint16_t *w_router;
  const float *router_bias;
  const void *w_gate_up;
  const void *s_gate_up;
  const void *w_down;
  const void *s_down;
  const uint16_t *w_shared_gate_up;
  const uint16_t *w_shared_down;
} oref_layer;

/* ---- codecs ------------------------------------------------------------ */
double oref_bf16_decode(uint16_t b);
uint16_t oref_bf16_encode(double v);          /* v -> binary32 -> bf16, each round to nearest even */
double oref_e4m3_decode(uint8_t c);           /* NaN for S.1111.111 */
uint8_t oref_e4m3_encode(float v);            /* RNE, saturate to +-448, NaN -> 0x7F|sign */
double oref_e2m1_decode(uint8_t c);           /* low 4 bits: S.EE.M, bias 1, max 6 */
double oref_e8m0_decode(uint8_t e);           /* 2^(e-127); NaN for 0xFF */

/* Per-token 1x128 activation quantisation of one row of n values (n % 128 == 0):
 * for each group, a = max|v|, s = a / 448 in fp32 (s = 1 when a == 0),
 * q = e4m3(v / s) with the division in fp32. */
void oref_quant_row(const float *v, int64_t n, uint8_t *q, float *s);

/* Array forms: element-wise encode; bf16 rows [rows, n] quantised per row. */
void oref_e4m3_encode_array(const float *v, int64_t n, uint8_t *q);
void oref_bf16_encode_array(const double *v, int64_t n, uint16_t *b);
void oref_quant_bf16_rows(const uint16_t *x, int64_t rows, int64_t n, uint8_t *q, float *s);

/* ---- routing ----------------------------------------------------------- */
/* logits l[t,e] = sum_h x[t,h] W_r[e,h] (+ bias[e]); choose the k largest
 * (exact ties: lower expert index first); slots in ascending expert id;
 * gates = softmax over the chosen k logits.  gap[t] = l_(k) - l_(k+1)
 * (k-th minus (k+1)-th largest logit; +inf when k == E).  Any output
 * pointer may be NULL.  token_list selects the tokens (NULL = 0..T-1). */
void oref_route(const oref_layer *L, const uint16_t *x, int64_t T,
                const int64_t *token_list, int64_t n_list,
                int32_t *ids, double *gates, double *logits, double *gap);

/* Gates for given ids: softmax over the logits of the given experts. */
void oref_gates_for_ids(const oref_layer *L, const uint16_t *x, int64_t T,
                        const int64_t *token_list, int64_t n_list,
                        const int32_t *ids, double *gates);

/* ---- grouping ---------------------------------------------------------- */
/* Stable counting sort of assignments 0..N-1 by key (expert id).  Keys
 * outside [0, E) are dropped: not counted, perm_pos = -1.
 * offsets[E+1] (exclusive scan of counts), perm_src[p] = i, perm_pos[i] = p.
 * Returns the number of dropped assignments. */
int64_t oref_permute(const int32_t *key, int64_t N, int32_t E,
                     int32_t *offsets, int32_t *perm_src, int32_t *perm_pos);

/* ---- expert FFN -------------------------------------------------------- */
/* Routed expert e applied to rows of an already-stored input:
 *   bf16 mode: a = bf16 row of length H;
 *   fp8 and mxfp4 modes: a = e4m3 codes (H bytes) with H/128 fp32 group scales.
 * h is stored as the GPU stores it (bf16, or e4m3 + 1x128 scales, each
 * decided from the fp32 value of h); out[H] in fp64.
 * out_h (optional, [I]) receives the dequantised stored h. */
void oref_expert_row(const oref_layer *L, int32_t e, const void *a, const float *a_scale,
                     double *out, double *out_h);

/* The same product written in the factored block form
 * sum_kb s_a[kb] s_w[nb,kb] sum_{k in kb} q_a[k] q_w[n,k]  (fp8 mode only),
 * for the gate/up pre-activations: zg[I], zu[I]. */
void oref_expert_gate_up_factored(const oref_layer *L, int32_t e, const uint8_t *a,
                                  const float *a_scale, double *zg, double *zu);
/* The same pre-activations for mxfp4 weights in the factored form of the
 * scaled MFMA: for each 128-input group kg of the activation and each
 * 32-input block kb inside it,
 *   sum_kg s_a[kg] sum_{kb in kg} 2^(s_w[n,kb]-127) sum_{k in kb} q_a[k] e2m1(q_w[n,k]). */
void oref_expert_gate_up_mx_factored(const oref_layer *L, int32_t e, const uint8_t *a,
                                     const float *a_scale, double *zg, double *zu);
/* Same pre-activations from dequantised operands (dequant then matmul;
 * fp8 and mxfp4 modes). */
void oref_expert_gate_up_dequant(const oref_layer *L, int32_t e, const uint8_t *a,
                                 const float *a_scale, double *zg, double *zu);

/* Shared expert on a bf16 row: h stored bf16; out[H] fp64. */
void oref_shared_row(const oref_layer *L, const uint16_t *x_row, double *out);

/* moe_expert_ffn equivalent over expert-grouped rows:
 * rows offsets[e]..offsets[e+1]-1 of a_rows go through expert e.
 * a_rows: bf16 [N,H] or (fp8, mxfp4) e4m3 [N,H] with a_scale [N,H/128].  out [N,H]. */
void oref_expert_ffn(const oref_layer *L, const int32_t *offsets, const void *a_rows,
                     const float *a_scale, int64_t N, double *out);

/* ---- whole layer ------------------------------------------------------- */
/* y[n_list, H] for the listed tokens (NULL = all T).  Routes with oref_route,
 * quantises x per token (fp8 and mxfp4 modes), sums shared + gated experts in fp64.
 * ids/gates/gap outputs optional ([n_list,k], [n_list,k], [n_list]). */
void oref_forward(const oref_layer *L, const uint16_t *x, int64_t T,
                  const int64_t *token_list, int64_t n_list, double *y,
                  int32_t *ids, double *gates, double *gap);

/* As oref_forward but with the routed experts forced to ids [n_list,k]
 * (gates recomputed from the oracle's logits of those experts). */
void oref_forward_with_ids(const oref_layer *L, const uint16_t *x, int64_t T,
                           const int64_t *token_list, int64_t n_list,
                           const int32_t *ids, double *y);

/* Pre-routed assignments (token, expert, gate), i = 0..N-1: for each listed
 * token t, y[t] = Shared(x[t]) + sum_{i: tok[i]==t, 0<=exp[i]<E} gate[i] FFN_exp[i](x[t]),
 * summed in increasing i. */
void oref_forward_triples(const oref_layer *L, const uint16_t *x, int64_t T,
                          const int32_t *tok, const int32_t *expert, const float *gate, int64_t N,
                          const int64_t *token_list, int64_t n_list, double *y);

/* Weighted combine of stored expert outputs (the moe_combine definition):
 * y[t] = shared[t] + sum_i gate[i] * y_perm[perm_pos[i]] over assignments of t
 * in increasing i (tok = NULL: token of i is i / k).  shared may be NULL. */
void oref_combine(const double *y_perm, const int32_t *perm_pos, const int32_t *tok,
                  int32_t k, const float *gate, int64_t N, const double *shared,
                  int64_t T, int64_t H, double *y);

/* ---- backward (bf16 experts) ------------------------------------------ */
/* Gradients of the layer with its routed experts fixed to ids [T, k] (the
 * forward's choice), for an output gradient dy (bf16 [T, H]), in fp64:
 *   gates g = softmax over the chosen logits; y[t] = Shared(x_t) + sum_j g_j FFN_j(x_t);
 *   dg_j = <dy_t, FFN_j(x_t)>, dl_j = g_j (dg_j - sum_m g_m dg_m);
 *   dx_t = Shared'(x_t)^T dy_t + sum_j [ FFN_j'(x_t)^T (g_j dy_t) + dl_j W_r[e_j] ];
 *   dW_gu[e], dW_d[e]: sums over the (token, slot) pairs routed to e of the
 *   FFN's weight gradients for output gradient g_j dy_t; the shared expert's
 *   likewise with gradient dy_t; dW_r[e] = sum dl_j x_t, dbias[e] = sum dl_j.
 * The gradient of the layer as a function (no storage rounding of h).
 * token_list restricts the sums to the listed tokens (NULL = all T);
 * dx [n_list, H]; weight gradients over the listed tokens only.  Any
 * gradient pointer except dx may be NULL. */
void oref_backward(const oref_layer *L, const uint16_t *x, int64_t T, const int32_t *ids,
                   const uint16_t *dy, const int64_t *token_list, int64_t n_list,
                   double *dx, double *dwgu, double *dwd, double *dwsgu, double *dwsd,
                   double *dwr, double *dbias);

int oref_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
