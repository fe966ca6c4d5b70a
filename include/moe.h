/*
 * moe.h -- C ABI of the MI355X (gfx950) routed Mixture-of-Experts layer.
 *
 * The layer is the MoE feed-forward block of Step-5-Preview
 * ("Step-5-Preview", NeMo AutoModel model coverage, section "Model
 * Architecture": hidden 4,096; 352 routed experts per MoE layer; top-8
 * routing; one shared expert; intermediate size 1,536 for every expert; a
 * learned router), with BF16 or block-scaled FP8 E4M3 expert weights
 * ("Step-5 minimal inference", introduction and "Contents": block-scaled FP8
 * expert GEMM and MoE primitives; section "Install": FP8 E4M3; expert dtype
 * chosen per layer by the checkpoint configuration, section "Checkpoints and
 * launch modes"):
 *
 *   y[t] = Shared(x[t]) + sum_{e in TopK(t)} g[t,e] * FFN_e(x[t])
 *   FFN(a) = (silu(a Wg^T) * (a Wu^T)) Wd^T
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless stated otherwise; tensors are
 *     row-major and contiguous, 16-byte aligned (the routed experts' weights
 *     may instead be in the tile16 layout: moe_weight_layout below).
 *     `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - The caller owns every buffer (inputs, outputs, workspace).  The library
 *     allocates and frees nothing and keeps no device state between calls.
 *     Calls on distinct streams with distinct workspaces may run concurrently.
 *   - Every call validates its arguments on the host before launching
 *     anything and returns a status; on error nothing is launched and no
 *     output is written.  T == 0 or N == 0 is a valid no-op.
 *   - Every call only enqueues work on `stream` and returns; none
 *     synchronises with the host.
 *   - Results are deterministic: the same inputs give the same bits on every
 *     run (no floating-point atomics; all sums in a fixed order).
 *
 * Numerics
 *   - Router: bf16 x and W_r, fp32 accumulation; bias (fp32, optional) added
 *     to the logits; the k largest logits are chosen, an exact tie going to
 *     the lower expert index; the k slots are returned in ascending expert id;
 *     gates = softmax over the k chosen logits (= softmax over all experts
 *     renormalised over the chosen ones), fp32.
 *   - FP8 mode: OCP E4M3FN codes (max 448, no infinities).  Weights carry one
 *     fp32 scale per 128x128 block of [out, in]; activations (x, and the
 *     intermediate h) carry one fp32 scale per token per 128 consecutive
 *     input columns: s = amax/448 (IEEE fp32 division; 1 when amax == 0),
 *     code = round-to-nearest-even(v / s).  Dequantised value = code * s.
 *   - MX FP4 mode (a low-bit weight format beside the two above): weights
 *     are OCP MX FP4, E2M1 codes two to a byte with input 2j in the low
 *     nibble of byte j (the packing of the NVFP4 linears described on the
 *     "TensorFold" pull-request page) and one E8M0 scale byte per 32
 *     consecutive inputs of a row (OCP Microscaling Formats specification
 *     v1.0); dequantised weight = e2m1(code) * 2^(scale - 127).  Activations
 *     and h are E4M3 with 1x128 scales exactly as in FP8 mode.
 *   - Expert GEMMs accumulate in fp32; h = silu(z_gate) * z_up in fp32, then
 *     stored as bf16 (bf16 experts) or E4M3 + 1x128 scales (fp8 and mxfp4
 *     experts).
 *   - Combine: fp32 sum in a fixed order -- shared expert first, then the
 *     token's assignments in increasing assignment index -- rounded once to
 *     the output dtype (the partial sums of the pages' deployment are likewise
 *     added in a fixed order in FP32: "Step-5 minimal inference", section
 *     "Long-output stability").
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_dtype {
  MOE_BF16 = 1,        /* bfloat16 */
  MOE_FP8_E4M3FN = 2,  /* OCP E4M3FN with fp32 block/group scales */
  MOE_F32 = 3,         /* IEEE binary32 */
  MOE_MXFP4_E2M1 = 4   /* OCP MX FP4: E2M1 codes, two per byte, E8M0 scale per 32 */
} moe_dtype;

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* NULL pointer where one is required, bad size or dimension,
                            k outside [1, min(E, 32)], misaligned pointer */
  MOE_EUNSUPPORTED = 2,  /* valid but not built: H % 128 != 0; bf16 experts with I % 64 != 0;
                            fp8 or mxfp4 experts with I % 128 != 0; a shared expert with
                            Is % 64 != 0; E > 1024; H, I or Is > 16384;
                            unsupported dtype combination */
  MOE_EWORKSPACE = 3,    /* ws_bytes smaller than the call needs */
  MOE_EHIP = 4           /* a HIP launch failed; moe_last_error() has the detail */
} moe_status;

/* Storage layout of the routed experts' w_gate_up and w_down
 * (moe_layer.weight_layout; bf16 and fp8 experts).
 *   MOE_LAYOUT_ROWS    row-major, as described under moe_layer (the default)
 *   MOE_LAYOUT_TILE16  the same bytes permuted inside each expert's matrix
 *                      (written by moe_pack_weights).  For an expert's matrix
 *                      of R rows x K bytes (R = 2I or H; K = H or I times the
 *                      element size), tile (t, c) -- rows 16t..16t+15, bytes
 *                      128c..128c+127 of each -- is 2048 contiguous bytes at
 *                      offset (c*R/16 + t)*2048 (the tiles of one 128-byte K
 *                      chunk are adjacent), and byte b of its row 16t+i sits
 *                      at 1024*((b/16)%2) + 16*(i + 16*(b/32)) + b%16.  Each
 *                      16-byte load of an MFMA operand fragment then reads one
 *                      whole contiguous kilobyte per wave.
 * MX FP4 experts and the shared expert's weights are always row-major;
 * moe_forward_train and moe_backward take MOE_LAYOUT_ROWS only. */
typedef enum moe_weight_layout {
  MOE_LAYOUT_ROWS = 0,
  MOE_LAYOUT_TILE16 = 1
} moe_weight_layout;

/* One MoE layer (host struct; the pointers in it are device pointers).
 *   hidden H, inter I (routed expert intermediate), num_experts E (experts
 *   held here: 352 for the whole layer, 44 for one of eight expert-parallel
 *   shares), top_k k (0 allowed only for calls that take pre-routed
 *   assignments), shared_inter Is (0 = no shared expert).
 *   expert_dtype: MOE_BF16, MOE_FP8_E4M3FN or MOE_MXFP4_E2M1.
 *   w_router        bf16 [E, H]            (moe_route / moe_forward only)
 *   router_bias     f32  [E] or NULL       (added to the logits)
 *   w_gate_up       [E, 2I, H]: rows 0..I-1 gate, rows I..2I-1 up  (bf16 or e4m3;
 *                   mxfp4: bytes [E, 2I, H/2], two codes per byte)
 *   s_gate_up       fp8: f32 [E, 2I/128, H/128]; mxfp4: E8M0 bytes [E, 2I, H/32];
 *                   bf16: NULL
 *   w_down          [E, H, I]              (bf16 or e4m3; mxfp4: bytes [E, H, I/2])
 *   s_down          fp8: f32 [E, H/128, I/128]; mxfp4: E8M0 bytes [E, H, I/32];
 *                   bf16: NULL
 *   w_shared_gate_up bf16 [2Is, H], w_shared_down bf16 [H, Is] (NULL if Is == 0)
 *   weight_layout   moe_weight_layout of w_gate_up and w_down (0: row-major)
 * Weights are read-only; they are the layout of a linear layer's weight
 * ([out, in]; y = a W^T). */
typedef struct moe_layer {
  int32_t hidden;
  int32_t inter;
  int32_t num_experts;
  int32_t top_k;
  int32_t shared_inter;
  int32_t expert_dtype;
  const void *w_router;
  const float *router_bias;
  const void *w_gate_up;
  const void *s_gate_up;
  const void *w_down;
  const void *s_down;
  const void *w_shared_gate_up;
  const void *w_shared_down;
  int32_t weight_layout;
} moe_layer;

/* Repack `count` row-major matrices of `rows` rows x `row_bytes` bytes each
 * (stored one after the other) into the MOE_LAYOUT_TILE16 layout (a
 * permutation of their bytes; the layout the expert GEMMs of "Step-5 minimal
 * inference" -- the block-scaled FP8 expert GEMM -- read fastest).  For a
 * layer's experts: w_gate_up with count = E, rows = 2I, row_bytes = H *
 * element size; w_down with count = E, rows = H, row_bytes = I * element
 * size (the fp8 scale tensors keep their layout).
 *   src, dst   device memory, 16-byte aligned, not overlapping; dst receives
 *              count*rows*row_bytes bytes.  Owned by the caller.
 * MOE_EINVAL: NULL or misaligned pointers, count <= 0, rows <= 0 or
 * rows % 16 != 0, row_bytes <= 0 or row_bytes % 128 != 0.  A load-time
 * step: enqueued on `stream` like every other call. */
moe_status moe_pack_weights(const void *src, void *dst, int64_t count, int64_t rows, int64_t row_bytes,
                            void *stream);

/* Workspace bytes that suffice for every call below except moe_backward on
 * this layer with up to T tokens and N assignments (N = T*k for routed
 * calls).  Host-only; 0 on invalid arguments. */
size_t moe_workspace_bytes(const moe_layer *layer, int64_t T, int64_t N);

/* Router: logits, top-k selection and gates.
 * ("Step-5-Preview", section "Model Architecture": learned router, top-8 of
 * 352 routed experts.)
 *   x           bf16 [T, H]
 *   topk_ids    int32 [T, k] out: chosen experts, ascending per token
 *   topk_gates  f32 [T, k] out: softmax over the chosen logits (same slots)
 *   logits      f32 [T, E] out, or NULL: router logits including the bias */
moe_status moe_route(const moe_layer *layer, const void *x, int64_t T,
                     int32_t *topk_ids, float *topk_gates, float *logits,
                     void *ws, size_t ws_bytes, void *stream);

/* Token-to-expert grouping: a stable counting sort of the N assignments by
 * expert (histogram, exclusive scan, ordered scatter), then a row gather of
 * x into expert order; in fp8 mode each gathered row is quantised per 1x128
 * group.  ("Step-5 minimal inference", "Contents": the MoE primitives.)
 *   x              bf16 [T, H]
 *   assign_expert  int32 [N]: expert of assignment i (e.g. topk_ids viewed as [T*k])
 *   assign_token   int32 [N] or NULL: token of assignment i (NULL: i / k)
 *   expert_offsets int32 [E+1] out: rows of expert e are offsets[e]..offsets[e+1]-1;
 *                  offsets[E] = assignments kept, so N - offsets[E] were dropped
 *   perm_src       int32 [N] out: assignment index placed at row p (rows in
 *                  expert order; inside an expert, increasing assignment index)
 *   perm_pos       int32 [N] out: row of assignment i (-1 if its expert or
 *                  token is out of range: such assignments are dropped)
 *   x_perm         [N, H] out: bf16 (bf16 experts) or e4m3 codes (fp8 and
 *                  mxfp4 experts); rows >= offsets[E] are left unwritten
 *   x_scale        f32 [N, H/128] out (fp8 and mxfp4 experts; NULL for bf16) */
moe_status moe_permute(const moe_layer *layer, const void *x, int64_t T,
                       const int32_t *assign_expert, const int32_t *assign_token, int64_t N,
                       int32_t *expert_offsets, int32_t *perm_src, int32_t *perm_pos,
                       void *x_perm, float *x_scale,
                       void *ws, size_t ws_bytes, void *stream);

/* Grouped expert FFN: for every expert e, rows offsets[e]..offsets[e+1]-1 of
 * x_perm go through gate/up (one grouped GEMM with a fused SwiGLU epilogue),
 * then down (a second grouped GEMM).  ("Step-5 minimal inference",
 * introduction: block-scaled FP8 expert GEMM; "Step-5-Preview", "Model
 * Architecture": intermediate 1,536 per expert.)
 *   expert_offsets int32 [E+1] (device; offsets[E] <= N)
 *   x_perm         [N, H] bf16 (bf16 experts) or e4m3 (fp8 and mxfp4 experts)
 *   x_scale        f32 [N, H/128] (fp8 and mxfp4 experts; NULL for bf16)
 *   y_perm         [N, H] out, y_dtype MOE_BF16 or MOE_F32; rows >= offsets[E]
 *                  are left unwritten
 * The shared expert runs through this call as a one-expert bf16 layer
 * (num_experts = 1, inter = Is, w_gate_up/w_down = the shared weights,
 * offsets {0, T}, x_perm = x). */
moe_status moe_expert_ffn(const moe_layer *layer, const int32_t *expert_offsets,
                          const void *x_perm, const float *x_scale, int64_t N,
                          void *y_perm, int32_t y_dtype,
                          void *ws, size_t ws_bytes, void *stream);

/* Weighted un-permute and combine, adding the shared-expert output:
 *   y[t] = shared[t] + sum_{i: token(i) = t} gates[i] * y_perm[perm_pos[i]]
 * in fp32, shared first, then increasing i; rounded once to out_dtype.
 * ("Step-5-Preview", "Model Architecture": the routed experts' outputs are
 * weighted by the router and the one shared expert's output is added;
 * "Step-5 minimal inference", "Long-output stability": partial results are
 * added in a fixed order with FP32 accumulation.)
 *   y_perm       [N, H] (y_dtype MOE_BF16 or MOE_F32)
 *   perm_pos     int32 [N]  (-1: assignment skipped)
 *   assign_token int32 [N] or NULL (NULL: token(i) = i / k)
 *   gates        f32 [N]
 *   shared_out   [T, H] (shared_dtype MOE_BF16 or MOE_F32) or NULL
 *   y            [T, H] out (out_dtype MOE_BF16 or MOE_F32); tokens with no
 *                assignment get the shared output (or 0). */
moe_status moe_combine(const moe_layer *layer, const void *y_perm, int32_t y_dtype,
                       const int32_t *perm_pos, const int32_t *assign_token,
                       const float *gates, int64_t N,
                       const void *shared_out, int32_t shared_dtype, int64_t T,
                       void *y, int32_t out_dtype,
                       void *ws, size_t ws_bytes, void *stream);

/* The whole layer: route -> permute -> routed expert FFN -> shared expert
 * FFN -> combine, all on `stream` ("Step-5-Preview", "Model Architecture":
 * top-8 of 352 routed experts plus one shared expert, intermediate 1,536;
 * "Step-5 minimal inference", introduction: block-scaled FP8 expert GEMMs).
 * The shared expert rides in the routed experts' launches, or runs in a
 * launch of its own when Is % 128 != 0 while I % 128 == 0.
 *   x          bf16 [T, H]
 *   y          [T, H] out (MOE_BF16 or MOE_F32)
 *   topk_ids   int32 [T, k] out or NULL;  topk_gates f32 [T, k] out or NULL */
moe_status moe_forward(const moe_layer *layer, const void *x, int64_t T,
                       void *y, int32_t out_dtype,
                       int32_t *topk_ids, float *topk_gates,
                       void *ws, size_t ws_bytes, void *stream);

/* The layer on pre-routed assignments: one expert-parallel rank's share of
 * the layer ("Step-5 minimal inference", introduction and "Contents": TP=EP=8
 * places 44 of the 352 experts on each rank), whose (token, expert, gate)
 * triples come from elsewhere.
 *   y[t] = shared(x[t]) + sum_{i: assign_token[i] = t} gates[i] * FFN_{assign_expert[i]}(x[t])
 * in fp32 (shared first, then increasing i), rounded once to out_dtype: the
 * result of moe_permute, moe_expert_ffn (routed experts, and the shared
 * expert as its one-expert layer), moe_combine, with the shared expert's
 * work inside the routed experts' launches (one gate/up and one down launch).
 *   x             bf16 [T, H]
 *   assign_expert int32 [N]: local expert of assignment i; assign_token int32 [N]:
 *                 its token; an assignment with either out of range is dropped
 *   gates         f32 [N], taken as given (no renormalisation)
 *   y             [T, H] out (MOE_BF16 or MOE_F32); a token with no assignment
 *                 gets the shared expert's output (or 0)
 * top_k and w_router are not used (top_k may be 0).  T == 0 is a no-op. */
moe_status moe_forward_routed(const moe_layer *layer, const void *x, int64_t T,
                              const int32_t *assign_expert, const int32_t *assign_token, const float *gates,
                              int64_t N, void *y, int32_t out_dtype,
                              void *ws, size_t ws_bytes, void *stream);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): its scratch memory is a device array the library owns,
 * MOE_NOALLOC_SCRATCH_BYTES on each GPU it runs on, held until the process
 * ends.  It allocates and frees nothing.  Same arguments, kernels and outputs
 * as moe_forward (bit for bit).
 *   MOE_EWORKSPACE  the call needs more scratch than the array holds (what
 *                   moe_forward would need; for the Step-5 layer: T above 359
 *                   tokens with bf16 experts, above 469 with fp8 or mxfp4
 *                   experts); checked on the host before the device is touched.
 * Other errors as moe_forward.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on the same GPU (two streams, two threads) race and must be serialised by
 * the caller.  Nothing in the array needs to be cleared between calls. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_layer *layer, const void *x, int64_t T,
                               void *y, int32_t out_dtype,
                               int32_t *topk_ids, float *topk_gates, void *stream);

/* Workspace bytes moe_backward needs for up to T tokens (moe_workspace_bytes
 * does not cover moe_backward).  Host-only; 0 on invalid arguments. */
size_t moe_backward_workspace_bytes(const moe_layer *layer, int64_t T);

/* Backward of the whole layer with bf16 experts, for training: the gradients
 * of L = sum_t <y[t], dy[t]> for the forward above with the routed experts
 * held fixed at topk_ids ("Step-5-Preview", section "Full-Depth H100
 * Benchmark": the layer is trained in BF16; section "Model Architecture":
 * learned router, top-8, one shared expert).  With g = softmax over the chosen
 * logits l_j and o_j = FFN_{e_j}(x):
 *   dg_j = <dy, o_j>;  dl_j = g_j (dg_j - sum_m g_m dg_m)    (softmax backward)
 *   each expert's SwiGLU FFN is differentiated with output gradient g_j dy
 *   (shared expert: dy); dW_router[e] += dl_j x, dbias[e] += dl_j,
 *   dx += dl_j W_router[e_j].
 * The expert pre-activations come from z_saved (moe_forward_train on the
 * same x; its ids and gates) or, with z_saved NULL, are recomputed from x
 * (then nothing is kept from the forward but topk_ids and topk_gates).
 * GEMM inputs are bf16 (x, dy, the
 * weights, g * h and the gradient of the pre-activations, rounded to bf16),
 * accumulation fp32; per-row and per-token reductions in a fixed order.
 *   x            bf16 [T, H]  (the forward's input)
 *   topk_ids     int32 [T, k] (the forward's choice; an id outside [0, E) is skipped)
 *   topk_gates   f32 [T, k]   (the forward's gates: softmax over the chosen logits)
 *   dy           bf16 [T, H]  (gradient of the layer output)
 *   z_saved      f32, layout of moe_forward_train, or NULL
 *   dx           f32 [T, H] out
 *   dw_gate_up   f32 [E, 2I, H] out;  dw_down f32 [E, H, I] out
 *   dw_shared_gate_up f32 [2Is, H] out, dw_shared_down f32 [H, Is] out (NULL if Is == 0)
 *   dw_router    f32 [E, H] out;  dbias f32 [E] out or NULL
 * Gradients are written, not accumulated; experts that receive no token get
 * zero gradients.  MOE_EUNSUPPORTED unless expert_dtype == MOE_BF16; top_k >= 1
 * and w_router are required.  T == 0 is a no-op (nothing written). */
moe_status moe_backward(const moe_layer *layer, const void *x, int64_t T,
                        const int32_t *topk_ids, const float *topk_gates, const void *dy,
                        const float *z_saved, float *dx, float *dw_gate_up, float *dw_down,
                        float *dw_shared_gate_up, float *dw_shared_down,
                        float *dw_router, float *dbias,
                        void *ws, size_t ws_bytes, void *stream);

/* Floats of the pre-activation buffer moe_forward_train fills for up to T
 * tokens: T*k*2I (routed rows) + T*2Is (shared expert).  0 on invalid
 * arguments. */
size_t moe_saved_z_floats(const moe_layer *layer, int64_t T);

/* moe_forward for training (bf16 experts only): the same launches and the
 * same outputs, and the gate/up GEMMs also write their fp32 pre-activations
 * z = [a W_g^T | a W_u^T] (2I values per row; Megatron-style activation
 * saving, so that moe_backward need not recompute them):
 *   z_saved  f32 out, moe_saved_z_floats(layer, T) floats: rows 0..T*k-1 =
 *            the routed assignments in expert order (the order of moe_permute
 *            on topk_ids; rows of dropped assignments are left unwritten),
 *            then T rows of the shared expert in token order ([T, 2Is]).
 * topk_ids and topk_gates are required (moe_backward takes them). */
moe_status moe_forward_train(const moe_layer *layer, const void *x, int64_t T,
                             void *y, int32_t out_dtype,
                             int32_t *topk_ids, float *topk_gates, float *z_saved,
                             void *ws, size_t ws_bytes, void *stream);

/* Static string naming a status. */
const char *moe_status_string(moe_status s);
/* Detail of the last failure on the calling thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
