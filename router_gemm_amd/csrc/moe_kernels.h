// moe_kernels.h -- host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// Writes {0, n} into dst[0..1] (device).
hipError_t launch_fill_offsets2(int32_t *dst, int32_t n, hipStream_t st);

// ---- grouped expert GEMMs (expert_gemm.hip)
struct FfnPlan {
  int mt;          // 16-row token subtiles per workgroup
  int max_tiles;   // capacity of the tile list
};
FfnPlan ffn_plan(int64_t N, int E);
size_t ffn_tiles_bytes(const FfnPlan &p);
// h: [N, I] bf16 or e4m3 (+ hs [N, I/128]).
hipError_t launch_expert_ffn(const uint8_t *x, const float *xs, const uint8_t *w_gu, const float *s_gu,
                             const uint8_t *w_d, const float *s_d, const int32_t *offsets, int E, int H,
                             int I, int64_t N, bool fp8, const FfnPlan &plan, int32_t *tiles,
                             uint8_t *h, float *hs, void *y, bool y_f32, bool shared_site, hipStream_t st);

// ---- combine (combine.hip)
// y[t] = shared[t] + sum over the token's assignments (fixed order) of g * y_perm[perm_pos]
// tok_off/tok_list: per-token assignment lists (NULL: assignments t*k .. t*k+k-1).
hipError_t launch_combine(const void *y_perm, bool yp_f32, const int32_t *perm_pos, const int32_t *tok_off,
                          const int32_t *tok_list, int k, const float *gates, const void *shared,
                          bool sh_f32, int64_t T, int64_t H, int64_t nrows, void *y, bool out_f32, hipStream_t st);

}  // namespace moe
