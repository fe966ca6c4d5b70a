// combine.hip -- weighted un-permute of the expert outputs plus the shared
// expert:  y[t] = shared[t] + sum_{assignments i of t} g[i] * y_perm[perm_pos[i]],
// summed in fp32 in a fixed order (shared first, then increasing i) and
// rounded once.  The pages' deployment adds its partial results in a fixed
// order with FP32 accumulation ("Step-5 minimal inference", section
// "Long-output stability"); the same rule makes this sum reproducible.

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

__device__ __forceinline__ void load8(const void *base, bool f32, int64_t idx, float v[8]) {
  if (f32) {
    const f32x4 *p = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(base) + idx);
    const f32x4 a = p[0], b = p[1];
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  } else {
    const i32x4 r = load16(reinterpret_cast<const uint16_t *>(base) + idx);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_to_f32((uint32_t)r[q] & 0xFFFFu);
      v[2 * q + 1] = bf16_to_f32((uint32_t)r[q] >> 16);
    }
  }
}

// Grid: one workgroup (256 threads) per (token, 2048-column block); each
// thread owns 8 consecutive columns.  The token's assignments are taken in
// batches of up to 32: their rows and gates are staged in LDS, then every
// thread issues its row loads 8 at a time before summing them in order, so
// the memory latency is paid once per 8 rows rather than twice per row.
constexpr int kCombBatch = 32;

__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y_perm, int yp_f32,
                                                      const int32_t *__restrict__ perm_pos,
                                                      const int32_t *__restrict__ tok_off,
                                                      const int32_t *__restrict__ tok_list, int k,
                                                      const float *__restrict__ gates,
                                                      const void *__restrict__ shared, int sh_f32, int64_t H, int64_t nrows,
                                                      void *__restrict__ y, int out_f32) {
  __shared__ int32_t srow[kCombBatch];
  __shared__ float sgate[kCombBatch];
  const int64_t t = blockIdx.x;
  const int64_t c = (int64_t)blockIdx.y * 2048 + (int64_t)threadIdx.x * 8;
  const bool active = c < H;
  int jbeg, jend;
  if (tok_off) {
    jbeg = tok_off[t];
    jend = tok_off[t + 1];
  } else {
    jbeg = (int)(t * k);
    jend = jbeg + k;
  }
  float acc[8];
  if (shared && active) {
    load8(shared, sh_f32 != 0, t * H + c, acc);
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
          load8(y_perm, yp_f32 != 0, (int64_t)(pr[u] >= 0 ? pr[u] : 0) * H + c, v[u]);
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
  if (!active) return;
  if (out_f32) {
    f32x4 *o = reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(y) + t * H + c);
    o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    i32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = (int)(pack_bf16x2(acc[2 * q], acc[2 * q + 1]));
    store16(reinterpret_cast<uint16_t *>(y) + t * H + c, r);
  }
}

hipError_t launch_combine(const void *y_perm, bool yp_f32, const int32_t *perm_pos, const int32_t *tok_off,
                          const int32_t *tok_list, int k, const float *gates, const void *shared,
                          bool sh_f32, int64_t T, int64_t H, int64_t nrows, void *y, bool out_f32, hipStream_t st) {
  if (T == 0) return hipSuccess;
  timing_before(8, st);
  const dim3 grid((unsigned)T, (unsigned)cdiv(H, 2048));
  combine_kernel<<<grid, 256, 0, st>>>(y_perm, yp_f32 ? 1 : 0, perm_pos, tok_off, tok_list, k, gates,
                                              shared, sh_f32 ? 1 : 0, H, nrows, y, out_f32 ? 1 : 0);
  timing_after(8, st);
  return hipGetLastError();
}

}  // namespace moe
