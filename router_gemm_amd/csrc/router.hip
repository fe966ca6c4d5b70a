// router.hip -- router logits (bf16 MFMA, fp32 accumulation) and the
// wavefront top-k selection with renormalised softmax gates.
//
// Layer definition: "Step-5-Preview" (NeMo AutoModel model coverage), section
// "Model Architecture": a learned router picks the top 8 of 352 routed
// experts per token.  Gates are the softmax over the chosen logits, which is
// the softmax over all experts renormalised over the chosen ones.

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

// logits partial sums: partial[s][t][e] = sum_{h in chunk s} x[t,h] * Wr[e,h].
// Grid (ceil(E/64), ceil(T/64), S); 4 waves, wave w owns tokens
// [64*by + 16w, +16) x experts [64*bx, +64) as four 16x16 MFMA tiles.
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, float *__restrict__ partial,
    int T, int E, int H, int kchunk) {
  const int lane = lane_id(), w = wave_id();
  const int e0 = blockIdx.x * 64;
  const int t0 = blockIdx.y * 64 + 16 * w;
  const int s = blockIdx.z;
  const int kbeg = s * kchunk + 8 * (lane >> 4);
  const int trow = t0 + (lane & 15);
  const bool tvalid = trow < T;
  const uint16_t *xp = x + (int64_t)(tvalid ? trow : 0) * H + kbeg;
  const uint16_t *wp[4];
  bool ev[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int er = e0 + 16 * j + (lane & 15);
    ev[j] = er < E;
    wp[j] = wr + (int64_t)(ev[j] ? er : 0) * H + kbeg;
  }
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const i32x4 zero = {0, 0, 0, 0};
#pragma unroll 4
  for (int k = 0; k < kchunk; k += 32) {
    const i32x4 a = tvalid ? load16(xp + k) : zero;
    i32x4 b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = ev[j] ? load16(wp[j] + k) : zero;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = mfma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b[j]), acc[j]);
  }
  // lane holds D[token 4*(lane/16)+r][expert lane%16] of each tile
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + 16 * j + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 4 * (lane >> 4) + r;
      if (t < T && e < E) partial[((int64_t)s * T + t) * E + e] = acc[j][r];
    }
  }
}

// Router logits for many tokens: LDS-tiled, one pass over K (S = 1).
// Workgroup tile 64 tokens x 192 experts; per 64-wide K chunk (128 bytes of
// bf16) the 256 rows (64 token rows, 192 router-weight rows) are copied
// straight into LDS (a ring of three 32 KB stages, two in flight), so a token
// row fetched once feeds 192 experts and a weight row feeds 64 tokens.  Wave w
// owns all 64 tokens x experts [48w, 48w+48): 4 x 3 MFMA tiles of 16x16.
// Rows past T or E repeat a valid row and are not stored.
namespace {
constexpr int RT_M = 64, RT_N = 192, RT_ROWS = RT_M + RT_N;
constexpr int RT_STAGE = RT_ROWS * 128, RT_NSTAGE = 3;
}  // namespace

__global__ __launch_bounds__(256, 1) void router_logits_tiled_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, float *__restrict__ logits, int T, int E,
    int H) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = lane_id(), w = uniform(wave_id());
  const int t0 = blockIdx.y * RT_M, e0 = blockIdx.x * RT_N;
  const int64_t rowb = (int64_t)H * 2;
  const int nchunk = (int)(rowb / 128);
  // this lane's 8 copies per chunk: LDS row r = 8 * (w + 4q) + lane / 8
  uint32_t off[8];
  const uint8_t *src[2] = {reinterpret_cast<const uint8_t *>(x), reinterpret_cast<const uint8_t *>(wr)};
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = 8 * (w + 4 * q) + (lane >> 3);
    const int c = (lane & 7) ^ swz_f(r);
    const int grow = r < RT_M ? min(t0 + r, T - 1) : min(e0 + r - RT_M, E - 1);
    off[q] = (uint32_t)(grow * rowb + c * 16);
  }
  // q < 2: token rows (r < 64), q >= 2: weight rows
  auto issue = [&](int kc, uint8_t *sb) {
#pragma unroll
    for (int q = 0; q < 8; ++q) dma16(src[q < 2 ? 0 : 1] + (int64_t)kc * 128 + off[q], sb + (w + 4 * q) * 1024);
  };
  f32x4 acc[4][3];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  issue(0, lds);
  if (nchunk > 1) issue(1, lds + RT_STAGE);
  for (int kc = 0; kc < nchunk; ++kc) {
    if (kc + 2 < nchunk) issue(kc + 2, lds + ((kc + 2) % RT_NSTAGE) * RT_STAGE);
    // chunk kc landed: the copies of kc+1 and kc+2 may still be in flight
    if (kc + 2 < nchunk)
      wait_vm<16>();
    else if (kc + 1 < nchunk)
      wait_vm<8>();
    else
      wait_vm<0>();
    wg_barrier();
    const uint8_t *sb = lds + (kc % RT_NSTAGE) * RT_STAGE;
    const int ck = 2 * (lane >> 4);
    i32x4 a[4][2], b[3][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * i + (lane & 15);
      a[i][0] = *reinterpret_cast<const i32x4 *>(sb + swz(r, ck));
      a[i][1] = *reinterpret_cast<const i32x4 *>(sb + swz(r, ck + 1));
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int r = RT_M + 48 * w + 16 * j + (lane & 15);
      b[j][0] = *reinterpret_cast<const i32x4 *>(sb + swz(r, ck));
      b[j][1] = *reinterpret_cast<const i32x4 *>(sb + swz(r, ck + 1));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8, a[i][0]), __builtin_bit_cast(bf16x8, b[j][0]), acc[i][j]);
        acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8, a[i][1]), __builtin_bit_cast(bf16x8, b[j][1]), acc[i][j]);
      }
    // every wave is done reading this stage before it is refilled (kc + 3)
    wait_vm_lgkm0<63>();
    wg_barrier();
  }
  // lane holds D[token 4*(lane/16)+r][expert lane%16] of tile (i, j)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int e = e0 + 48 * w + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * i + 4 * (lane >> 4) + r;
        if (t < T && e < E) logits[(int64_t)t * E + e] = acc[i][j][r];
      }
    }
}

// One wave per token: logits = sum of the S partials (in order s = 0..S-1)
// + bias; k rounds of a wave-wide arg-max under the order (value desc, index
// asc), a NaN logit ranking as -infinity; slots sorted by expert id; gates =
// exp(l - l_max) / sum, fp32.
template <int NJ>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float *__restrict__ partial, int S, const float *__restrict__ bias, int T, int E, int k,
    int32_t *__restrict__ ids, float *__restrict__ gates, float *__restrict__ logits_out) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= T) return;
  float v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) v[j] = 0.f;
  // partial sums added in split order s = 0..S-1 (S <= 8); every split's
  // values are loaded before the first add, so the loads overlap
  float pv[8][NJ];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const float *p = partial + ((int64_t)(s < S ? s : 0) * T + t) * E;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      pv[s][j] = (s < S && e < E) ? p[e] : 0.f;
    }
  }
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (s < S) v[j] += pv[s][j];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      if (bias) v[j] += bias[e];
      if (logits_out) logits_out[(int64_t)t * E + e] = v[j];
      if (v[j] != v[j]) v[j] = -__builtin_huge_valf();   // a NaN logit ranks as -infinity
    }
  }
  uint32_t taken = 0;
  float my_v = 0.f;
  int my_e = 0;
  for (int it = 0; it < k; ++it) {
    float bv = -__builtin_huge_valf();
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !((taken >> j) & 1u) && (v[j] > bv || (v[j] == bv && e < be))) {
        bv = v[j];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oe = __shfl_xor(be, o, kWave);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (be < E && (be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == it) {
      my_v = bv;
      my_e = be;
    }
  }
  // slot of the j-th winner = number of winners with a smaller expert id
  int rank = 0;
  for (int j = 0; j < k; ++j) {
    const int ej = __shfl(my_e, j, kWave);
    rank += (ej < my_e) ? 1 : 0;
  }
  // a chosen logit equal to the largest weighs exp(0) = 1 (so k chosen
  // -infinity logits, a token whose logits are all NaN, get 1/k each)
  const float vmax = __shfl(my_v, 0, kWave);
  const float ex = lane < k ? (my_v == vmax ? 1.0f : expf(my_v - vmax)) : 0.f;
  const float den = __shfl(wave_sum(ex), 0, kWave);
  if (lane < k) {
    ids[(int64_t)t * k + rank] = my_e;
    gates[(int64_t)t * k + rank] = __fdiv_rn(ex, den);
  }
}

// Many tokens: the LDS-tiled kernel (one pass, S = 1).
// (per-lane copy offsets are 32-bit: the token rows must span < 2 GiB)
static bool router_tiled(int64_t T, int H) { return T >= 2048 && H % 64 == 0 && T * H * 2 < (int64_t(1) << 31); }

int router_ksplit(int64_t T, int E, int H) {
  if (router_tiled(T, H)) return 1;
  const int64_t tiles = cdiv(E, 64) * cdiv(T, 64);
  int S = 1;
  // split K (at most 8 ways) until there are enough workgroups, keeping chunks
  // of >= 256 that are multiples of 32
  while (S < 8 && tiles * S < 256 && H % (2 * S) == 0 && (H / (2 * S)) % 32 == 0 && H / (2 * S) >= 256) S *= 2;
  return S;
}

hipError_t launch_router(const uint16_t *x, const uint16_t *wr, const float *bias, int64_t T, int E,
                         int H, int k, float *partial, int S, int32_t *ids, float *gates,
                         float *logits, hipStream_t st) {
  if (T == 0) return hipSuccess;
  timing_before(0, st);
  if (router_tiled(T, H) && S == 1) {
    const size_t lds = (size_t)RT_NSTAGE * RT_STAGE;
    static bool attr_set[64] = {};
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev >= 0 && dev < 64 && !attr_set[dev]) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&router_logits_tiled_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr_set[dev] = true;
    }
    dim3 gt((unsigned)cdiv(E, RT_N), (unsigned)cdiv(T, RT_M));
    router_logits_tiled_kernel<<<gt, 256, lds, st>>>(x, wr, partial, (int)T, E, H);
  } else {
    dim3 g1((unsigned)cdiv(E, 64), (unsigned)cdiv(T, 64), (unsigned)S);
    router_logits_kernel<<<g1, 256, 0, st>>>(x, wr, partial, (int)T, E, H, H / S);
  }
  timing_after(0, st);
  const unsigned g2 = (unsigned)cdiv(T, 4);
  const int nj = (int)cdiv(E, 64);
  timing_before(1, st);
#define MOE_TOPK_CASE(NJ)                                                                      \
  case NJ:                                                                                     \
    router_topk_kernel<NJ><<<g2, 256, 0, st>>>(partial, S, bias, (int)T, E, k, ids, gates, logits); \
    break;
  switch (nj) {
    MOE_TOPK_CASE(1) MOE_TOPK_CASE(2) MOE_TOPK_CASE(3) MOE_TOPK_CASE(4)
    MOE_TOPK_CASE(5) MOE_TOPK_CASE(6) MOE_TOPK_CASE(7) MOE_TOPK_CASE(8)
    MOE_TOPK_CASE(9) MOE_TOPK_CASE(10) MOE_TOPK_CASE(11) MOE_TOPK_CASE(12)
    MOE_TOPK_CASE(13) MOE_TOPK_CASE(14) MOE_TOPK_CASE(15) MOE_TOPK_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MOE_TOPK_CASE
  timing_after(1, st);
  return hipGetLastError();
}

}  // namespace moe
