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

// One workgroup (256 threads) per token; each thread owns 8 consecutive columns
// per 2048-column stride.
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y_perm, int yp_f32,
                                                      const int32_t *__restrict__ perm_pos,
                                                      const int32_t *__restrict__ tok_off,
                                                      const int32_t *__restrict__ tok_list, int k,
                                                      const float *__restrict__ gates,
                                                      const void *__restrict__ shared, int sh_f32, int64_t H, int64_t nrows,
                                                      void *__restrict__ y, int out_f32) {
  const int64_t t = blockIdx.x;
  int jbeg, jend;
  if (tok_off) {
    jbeg = tok_off[t];
    jend = tok_off[t + 1];
  } else {
    jbeg = (int)(t * k);
    jend = jbeg + k;
  }
  for (int64_t c = (int64_t)threadIdx.x * 8; c < H; c += 2048) {
    float acc[8];
    if (shared) {
      load8(shared, sh_f32 != 0, t * H + c, acc);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    }
    for (int j = jbeg; j < jend; ++j) {
      const int32_t i = tok_list ? tok_list[j] : j;
      const int32_t p = perm_pos[i];
      if (p < 0 || p >= nrows) continue;
      const float g = gates[i];
      float v[8];
      load8(y_perm, yp_f32 != 0, (int64_t)p * H + c, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(g, v[q], acc[q]);
    }
    if (out_f32) {
      f32x4 *o = reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(y) + t * H + c);
      o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
      o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      i32x4 r;
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = (int)(f32_to_bf16(acc[2 * q]) | (f32_to_bf16(acc[2 * q + 1]) << 16));
      store16(reinterpret_cast<uint16_t *>(y) + t * H + c, r);
    }
  }
}

hipError_t launch_combine(const void *y_perm, bool yp_f32, const int32_t *perm_pos, const int32_t *tok_off,
                          const int32_t *tok_list, int k, const float *gates, const void *shared,
                          bool sh_f32, int64_t T, int64_t H, int64_t nrows, void *y, bool out_f32, hipStream_t st) {
  if (T == 0) return hipSuccess;
  timing_before(8, st);
  combine_kernel<<<(unsigned)T, 256, 0, st>>>(y_perm, yp_f32 ? 1 : 0, perm_pos, tok_off, tok_list, k, gates,
                                              shared, sh_f32 ? 1 : 0, H, nrows, y, out_f32 ? 1 : 0);
  timing_after(8, st);
  return hipGetLastError();
}

}  // namespace moe
