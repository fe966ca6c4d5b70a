// moe_kernels.h -- host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// launch-site timers (timing.cpp); sites are the moe_site values of moe_timing.h
void timing_before(int site, hipStream_t st);
void timing_after(int site, hipStream_t st);
constexpr size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// ---- router (router.hip)
int router_ksplit(int64_t T, int E, int H);
hipError_t launch_router(const uint16_t *x, const uint16_t *wr, const float *bias, int64_t T, int E,
                         int H, int k, float *partial, int S, int32_t *ids, float *gates,
                         float *logits, hipStream_t st);

// ---- stable counting sort and row gather (permute.hip)
constexpr int kSortChunk = 512;
// Workspace int32 words the sort needs for N keys into nbins bins.
size_t sort_ws_words(int64_t N, int64_t nbins);
// Stable counting sort of i = 0..N-1 by keys[i] in [0, nbins); a key outside
// that range, or with aux[i] outside [0, aux_bound) when aux != NULL, is
// dropped (perm_pos = -1).  offsets [nbins+1]; perm_src [N] (rows >= offsets[nbins]
// untouched); perm_pos [N]; ws: sort_ws_words(N, nbins) int32 words.
hipError_t launch_counting_sort(const int32_t *keys, const int32_t *aux, int64_t aux_bound, int64_t N,
                                int64_t nbins, int32_t *offsets, int32_t *perm_src, int32_t *perm_pos,
                                int32_t *ws, hipStream_t st);
// x_perm[p] = x[token(perm_src[p])] for p < offsets_end[0]; token(i) = tok ? tok[i] : i / k.
// fp8: per-row 1x128 quantisation into codes + scales.
hipError_t launch_gather_rows(const uint16_t *x, int64_t H, const int32_t *perm_src, const int32_t *tok,
                              int k, int64_t N, const int32_t *offsets_end, bool fp8, void *x_perm,
                              float *x_scale, hipStream_t st);
// Per-token 1x128 quantisation of x into e4m3 codes and scales (the same
// arithmetic as the fp8 gather, without the permutation).
hipError_t launch_quantize_rows(const uint16_t *x, int64_t H, int64_t T, uint8_t *xq, float *x_scale,
                                hipStream_t st);

// ---- grouped expert GEMMs (expert_gemm.hip)
// One group = one set of experts with its own weights, rows and outputs.  A
// launch covers up to two groups (the routed experts and the shared expert),
// so the shared expert's tiles run inside the routed experts' launch.
struct FfnGroup {
  const uint8_t *x;    // [nrows, H] rows in expert order: e4m3 codes (fp8, mx) or bf16
  const float *xs;     // [nrows, H/128] (fp8)
  const uint8_t *wgu;  // [E, 2I, H]: rows 0..I-1 gate, I..2I-1 up
  const float *sgu;    // [E, 2I/128, H/128] (fp8)
  const uint8_t *wd;   // [E, H, I]
  const float *sd;     // [E, H/128, I/128] (fp8)
  const int32_t *off;  // [E+1] device offsets of each expert's rows; NULL: E == 1, rows [0, nrows)
  uint8_t *h;          // [nrows, I] intermediate: e4m3 (fp8) or bf16
  float *hs;           // [nrows, I/128] (fp8)
  void *y;             // [nrows, H] output, bf16 or f32
  // MX FP4 weights (mx = 1): wgu [E, 2I, H/2] and wd [E, H, I/2] hold two
  // E2M1 codes per byte, mgu [E, 2I, H/32] and md [E, H, I/32] one E8M0
  // scale byte per 32 inputs of a row; x and h are e4m3 as in fp8 mode.
  const uint8_t *mgu;
  const uint8_t *md;
  int32_t E, I, nrows, fp8, y_f32, mx;
  // Optional (tiled kernels only): row r of the GEMM input is row
  // xsrc[r] / xdiv of x (and xs), so the rows need not be gathered first.
  const int32_t *xsrc;
  int32_t xdiv;
  // Optional (bf16 experts): [nrows, 2I] fp32, receives the gate/up
  // pre-activations of each row (gate half, then up half) for a backward.
  float *z;
  // wgu and wd in the 16-row tile layout (bf16 and fp8 weights): in each
  // expert's [R, K] matrix the 16 x 128-byte tile (t, c) -- rows 16t..16t+15,
  // bytes 128c..128c+127 -- is 2048 contiguous bytes at (c * R/16 + t) * 2048
  // (the tiles of one K chunk are adjacent); byte b of its row i sits at
  // 1024 ((b / 16) % 2) + 16 (i + 16 (b / 32)) + b % 16, so that each of the
  // two 16-byte loads of an MFMA fragment (lane l = row + 16 k-group) reads
  // 1 KB of contiguous memory.
  int32_t tile16;
};
constexpr int kMaxGroups = 2;
// Tile list entry: group (0 or 1), expert of that group, first row (relative
// to the expert's offset).
struct TileEntry {
  int32_t ge;   // group << 24 | expert
  int32_t m0;
};
struct FfnPlan {
  int tiled;       // 1: LDS-tiled persistent kernels (128- or 256-row token tiles; MX FP4: 64 or 256), 0: streaming
  int mt;          // streaming: 16-row token subtiles per workgroup
  int gw;          // streaming: gate (and up) 16-row weight tiles per wave (2 -> 128 h columns)
  int bm;          // token rows per tile-list entry
  int max_tiles;   // capacity of the tile list
  // streaming, few tokens: K split this many ways (4 or 8) for the one-expert bf16
  // group sgroup (the shared expert), whose fp32 partial sums (spart_floats,
  // after the tile list in the same workspace) a finishing pass adds in order
  int ssplit;
  int sgroup;
  int64_t spart_floats;
};
// Tile-list workspace header (int32 words): [0] tile count, [1] tiles of
// group 0; the tile list follows.
constexpr int kTileHdrWords = 64;
FfnPlan ffn_plan(const FfnGroup *g, int ngroups, int H);
size_t ffn_tiles_bytes(const FfnPlan &p);
// LDS-tiled variant (expert_gemm_tiled.hip); tiles built with bm-row entries,
// bm = 128 (256 x 128 work items, 4 waves) or 256 (256 x 256, 8 waves).
hipError_t launch_tiled_ffn(const FfnGroup *g, int ngroups, int H, const void *tiles, int32_t *hdr, int num_cus,
                            int bm, int site, hipStream_t st);
// LDS-tiled variant for MX FP4 weights (expert_gemm_tiled_mx.hip): one group,
// tiles built with 64-row entries; needs H and I multiples of 256.
bool tiled_mx_supported(const FfnGroup &g, int H);
hipError_t launch_tiled_mx_ffn(const FfnGroup &g, int H, const void *tiles, int32_t *hdr, int num_cus, int site,
                               hipStream_t st);
// 256 x 256 items for MX FP4 weights (expert_gemm_tiled.hip): the MX group
// and optionally a bf16 group (the shared expert) in one launch, tiles built
// with 256-row entries; H and the MX group's I multiples of 256.
hipError_t launch_wide_mx_ffn(const FfnGroup *g, int ngroups, int H, const void *tiles, int32_t *hdr, int num_cus,
                              int site, hipStream_t st);
// Compute units of the current device (cached per device).
int num_compute_units();
// site: timing site of the gate/up launch (the down launch uses site + 1).
// tiles_ready: the tile list in tiles_ws was written beforehand (launch_permute_small).
hipError_t launch_expert_ffn(const FfnGroup *g, int ngroups, int H, const FfnPlan &plan, int32_t *tiles_ws,
                             int site, hipStream_t st, bool tiles_ready = false);

// Tile list of a row-segmented grouped launch: bm-row entries over g's
// experts (expert_gemm.hip).
// Repack count row-major [rows, row_bytes] matrices into the tile16 layout
// (layout.hip); rows % 16 == 0, row_bytes % 128 == 0.
hipError_t launch_pack_tile16(const uint8_t *src, uint8_t *dst, int64_t count, int64_t rows, int64_t row_bytes,
                              hipStream_t st);
hipError_t launch_build_tiles(const FfnGroup &g, int bm, int max_tiles, TileEntry *tiles, int32_t *hdr,
                              hipStream_t st);

// Tile list written by the one-launch grouping below: bm-row entries; with
// lead_group, group 0 is one expert of lead_rows rows (the shared expert) and
// the sorted experts are group 1.  tiles == NULL: no list.
struct SmallTiles {
  TileEntry *tiles;
  int32_t *hdr;
  int bm, max_tiles, lead_group, lead_rows;
};
// The sort of the N = T*k routed assignments (token i / k) into nbins
// experts, its tables, the tile list and the (fp8: quantised) row gather of
// x, in one launch, for N <= 512 and nbins <= 1024 (permute_small_ok):
// the results of launch_counting_sort + launch_gather_rows + the tile list.
bool permute_small_ok(int64_t N, int64_t nbins);
// launch_counting_sort, and where its launches allow (the chunk table with
// up to 4096 bins) the expert GEMMs' tile list from the same offsets, as
// build_tiles_kernel would write it: *tiles_done says whether it was written.
hipError_t launch_counting_sort_tiles(const int32_t *keys, const int32_t *aux, int64_t aux_bound, int64_t N,
                                      int64_t nbins, int32_t *offsets, int32_t *perm_src, int32_t *perm_pos,
                                      int32_t *ws, const SmallTiles &tl, bool *tiles_done, hipStream_t st);
hipError_t launch_permute_small(const int32_t *keys, int64_t N, int64_t nbins, int k, const uint16_t *x, int64_t H,
                                bool fp8, int32_t *offsets, int32_t *perm_src, int32_t *perm_pos, void *x_perm,
                                float *x_scale, const SmallTiles &tl, hipStream_t st);

// ---- backward of the layer, bf16 experts (backward.hip)
// One set of experts (the routed experts, or the shared expert as G = 1 with
// off = NULL) whose rows are already in expert order.
struct BwdExpert {
  int H, I, G;
  int64_t rows;              // N: rows in expert order
  int64_t T;                 // tokens (routed: for the softmax backward)
  int k;
  const uint16_t *x;         // [N, H] bf16 input rows
  const uint16_t *dy;        // [N, H] bf16 output gradient rows (ungated)
  const uint16_t *wgu;       // [G, 2I, H]
  const uint16_t *wd;        // [G, H, I]
  const int32_t *off;        // [G+1] or NULL (G == 1, rows [0, N))
  const float *gates;        // [T*k] gate of each assignment, or NULL (gate 1)
  const int32_t *perm_src;   // [N] assignment of each row (with gates)
  const int32_t *perm_pos;   // [T*k] row of each assignment (with dl)
  float *z;                  // [N, 2I] pre-activations: recomputed here, or given (z_given)
  int z_given;
  float *u;                  // [N, I] scratch: dy W_down
  uint16_t *hg;              // [N, I] scratch: gate * h, bf16
  uint16_t *dz;              // [N, 2I] scratch: gradient of z, bf16
  float *dg;                 // [N] gate gradients, or NULL
  float *dl;                 // [N] logit gradients, or NULL
  float *dx_rows;            // [N, H] out: input gradient of each row through the expert
  float *dwgu;               // [G, 2I, H] out
  float *dwd;                // [G, H, I] out
  int32_t *tiles;            // tile-list workspace: kTileHdrWords + 2 * bwd_max_tiles(N, G) words
  int max_tiles;
};
int bwd_max_tiles(int64_t rows, int G);
hipError_t launch_expert_backward(const BwdExpert &X, hipStream_t st);
// dW_r[e] = sum of dl[p] x_perm[p] over e's rows; dbias (NULL: skipped) = sum of dl[p].
hipError_t launch_router_backward(const float *dl, const uint16_t *x_perm, const int32_t *off, int E, int H,
                                  float *dwr, float *dbias, hipStream_t st);
// dx[t] = dx_shared[t] (NULL: 0) + sum_j dx_rows[perm_pos[t k + j]] + sum_j dl W_r[ids[t k + j]].
hipError_t launch_dx_backward(const float *dx_shared, const float *dx_rows, const int32_t *perm_pos,
                              const int32_t *ids, const float *dl, const uint16_t *wr, int64_t T, int k, int H,
                              float *dx, hipStream_t st);

// ---- the C ABI's forward on a given scratch buffer (moe_api.cpp)
// Workspace bytes moe_forward needs for T tokens (0 on invalid arguments).
size_t forward_ws_bytes(const moe_layer *L, int64_t T);
// moe_forward with its scratch memory at ws (ws_bytes usable).
moe_status forward_with_ws(const moe_layer *L, const void *x, int64_t T, void *y, int32_t out_dtype,
                           int32_t *topk_ids, float *topk_gates, void *ws, size_t ws_bytes, void *stream);
// Record `msg` as moe_last_error() and return s.
moe_status api_error(moe_status s, const char *msg);

// ---- combine (combine.hip)
// y[t] = shared[t] + sum over the token's assignments (fixed order) of g * y_perm[perm_pos]
// tok_off/tok_list: per-token assignment lists (NULL: assignments t*k .. t*k+k-1).
hipError_t launch_combine(const void *y_perm, bool yp_f32, const int32_t *perm_pos, const int32_t *tok_off,
                          const int32_t *tok_list, int k, const float *gates, const void *shared,
                          bool sh_f32, int64_t T, int64_t H, int64_t nrows, void *y, bool out_f32, hipStream_t st);

}  // namespace moe
