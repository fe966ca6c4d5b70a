// combine.hip -- weighted un-permute of the expert outputs plus the shared
// expert:  y[t] = shared[t] + sum_{assignments i of t} g[i] * y_perm[perm_pos[i]],
// summed in fp32 in a fixed order (shared first, then increasing i) and
// rounded once.  The pages' deployment adds its partial results in a fixed
// order with FP32 accumulation ("Step-5 minimal inference", section
// "Long-output stability"); the same rule makes this sum reproducible.

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

// 8 consecutive values of an fp32 or bf16 row: the raw load and its
// conversion are separate steps, so that several loads can be in flight
// before the first conversion waits for its data.
struct Raw8 {
  i32x4 a, b;
};
template <bool F32>
__device__ __forceinline__ Raw8 raw8(const void *base, int64_t idx) {
  Raw8 r;
  if constexpr (F32) {
    const i32x4 *p = reinterpret_cast<const i32x4 *>(reinterpret_cast<const float *>(base) + idx);
    r.a = p[0];
    r.b = p[1];
  } else {
    r.a = load16(reinterpret_cast<const uint16_t *>(base) + idx);
  }
  return r;
}
template <bool F32>
__device__ __forceinline__ void cvt8(const Raw8 &r, float v[8]) {
  if constexpr (F32) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // each element goes through a scalar first: hipcc drops the index of a
      // vector element used directly as __builtin_bit_cast's operand
      const int32_t lo = r.a[q], hi = r.b[q];
      v[q] = __builtin_bit_cast(float, lo);
      v[4 + q] = __builtin_bit_cast(float, hi);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_to_f32((uint32_t)r.a[q] & 0xFFFFu);
      v[2 * q + 1] = bf16_to_f32((uint32_t)r.a[q] >> 16);
    }
  }
}
template <bool F32>
__device__ __forceinline__ void load8(const void *base, int64_t idx, float v[8]) {
  cvt8<F32>(raw8<F32>(base, idx), v);
}

// Grid: one workgroup (256 threads) per (token, 2048-column block); each
// thread owns 8 consecutive columns.
//
// Assignments t*k .. t*k+k-1 (the router's layout, 1 <= k <= 8): the rows and
// gates are the same for the whole workgroup, so they come through scalar
// loads with no staging, and the shared row and all k expert rows are loaded
// before the first add: one memory latency per workgroup after the row
// indices.  Otherwise (a token list, or k outside 1..8) the token's
// assignments are taken in batches of up to 32 staged in LDS, and every
// thread issues its row loads 8 at a time before summing them in order.
constexpr int kCombBatch = 32;

__device__ __forceinline__ void store8(void *y, bool f32, int64_t idx, const float acc[8]) {
  if (f32) {
    f32x4 *o = reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(y) + idx);
    o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    i32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = (int)(pack_bf16x2(acc[2 * q], acc[2 * q + 1]));
    store16(reinterpret_cast<uint16_t *>(y) + idx, r);
  }
}

// YF32 / SF32: y_perm / the shared rows are fp32 (else bf16).
template <bool YF32, bool SF32>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y_perm,
                                                      const int32_t *__restrict__ perm_pos,
                                                      const int32_t *__restrict__ tok_off,
                                                      const int32_t *__restrict__ tok_list, int k,
                                                      const float *__restrict__ gates,
                                                      const void *__restrict__ shared, int64_t H, int64_t nrows,
                                                      void *__restrict__ y, int out_f32) {
  __shared__ int32_t srow[kCombBatch];
  __shared__ float sgate[kCombBatch];
  const int64_t t = blockIdx.x;
  const int64_t c = (int64_t)blockIdx.y * 2048 + (int64_t)threadIdx.x * 8;
  const bool active = c < H;
  float acc[8];
  if (!tok_off && k >= 1 && k <= 8) {
    // slots past k re-read slot k-1 (in bounds, left out below), so the 16
    // loads are unconditional and go out together
    int32_t pr[8];
    float g[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = t * k + min(u, k - 1);
      pr[u] = perm_pos[i];
      g[u] = gates[i];
    }
    // both sets in registers before the row loads (which need the rows
    // anyway): keeps the compiler from sinking each gate load into its slot's
    // branch, where the loads would wait one after another
#pragma unroll
    for (int u = 0; u < 8; ++u) asm volatile("" ::"s"(pr[u]), "s"(g[u]));
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u >= k || pr[u] < 0 || pr[u] >= nrows) pr[u] = -1;   // -1: assignment skipped
    if (!active) return;
    // a skipped slot reads row 0 (none when nrows == 0) and is left out of the sum
    Raw8 rs, rv[8];
    if (shared) rs = raw8<SF32>(shared, t * H + c);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < k && nrows > 0) rv[u] = raw8<YF32>(y_perm, (int64_t)(pr[u] >= 0 ? pr[u] : 0) * H + c);
    if (shared) {
      cvt8<SF32>(rs, acc);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u >= k || pr[u] < 0) continue;
      float v[8];
      cvt8<YF32>(rv[u], v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(g[u], v[q], acc[q]);
    }
    store8(y, out_f32 != 0, t * H + c, acc);
    return;
  }
  int jbeg, jend;
  if (tok_off) {
    jbeg = tok_off[t];
    jend = tok_off[t + 1];
  } else {
    jbeg = (int)(t * k);
    jend = jbeg + k;
  }
  if (shared && active) {
    load8<SF32>(shared, t * H + c, acc);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  }
  for (int jb = jbeg; jb < jend; jb += kCombBatch) {
    const int n = min(kCombBatch, jend - jb);
    if ((int)threadIdx.x < n) {
      const int32_t i = tok_list ? tok_list[jb + threadIdx.x] : jb + (int)threadIdx.x;
      const int32_t p = perm_pos[i];
      srow[threadIdx.x] = (p < 0 || p >= nrows) ? -1 : p;   // -1: assignment skipped
      sgate[threadIdx.x] = gates[i];
    }
    __syncthreads();
    if (active && nrows > 0) {   // nrows == 0: every slot is skipped
      for (int q0 = 0; q0 < n; q0 += 8) {
        float v[8][8];
        int32_t pr[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          pr[u] = q0 + u < n ? srow[q0 + u] : -1;
          // a skipped slot reads row 0 and is left out of the sum below
          load8<YF32>(y_perm, (int64_t)(pr[u] >= 0 ? pr[u] : 0) * H + c, v[u]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (pr[u] < 0) continue;
          const float g = sgate[q0 + u];
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(g, v[u][q], acc[q]);
        }
      }
    }
    __syncthreads();
  }
  if (active) store8(y, out_f32 != 0, t * H + c, acc);
}

hipError_t launch_combine(const void *y_perm, bool yp_f32, const int32_t *perm_pos, const int32_t *tok_off,
                          const int32_t *tok_list, int k, const float *gates, const void *shared,
                          bool sh_f32, int64_t T, int64_t H, int64_t nrows, void *y, bool out_f32, hipStream_t st) {
  if (T == 0) return hipSuccess;
  timing_before(8, st);
  const dim3 grid((unsigned)T, (unsigned)cdiv(H, 2048));
  const int of = out_f32 ? 1 : 0;
#define MOE_COMBINE(Y, S) \
  combine_kernel<Y, S><<<grid, 256, 0, st>>>(y_perm, perm_pos, tok_off, tok_list, k, gates, shared, H, nrows, y, of)
  if (yp_f32) {
    if (sh_f32) MOE_COMBINE(true, true); else MOE_COMBINE(true, false);
  } else {
    if (sh_f32) MOE_COMBINE(false, true); else MOE_COMBINE(false, false);
  }
#undef MOE_COMBINE
  timing_after(8, st);
  return hipGetLastError();
}

}  // namespace moe
