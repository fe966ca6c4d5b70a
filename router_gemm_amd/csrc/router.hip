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
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int er = e0 + 16 * j + (lane & 15);
    wp[j] = wr + (int64_t)(er < E ? er : 0) * H + kbeg;
  }
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // batches of 8 K-steps: all 40 loads of a batch are issued before its
  // MFMAs.  Rows past T and experts past E read a valid row (their outputs
  // are not stored), and steps past the chunk re-read its last step (their
  // MFMAs are skipped), so every load is unconditional and in bounds.
  for (int k0 = 0; k0 < kchunk; k0 += 256) {
    i32x4 a[8], b[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kk = min(k0 + 32 * u, kchunk - 32);
      a[u] = load16(xp + kk);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[u][j] = load16(wp[j] + kk);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + 32 * u < kchunk)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j] = mfma_bf16(__builtin_bit_cast(bf16x8, a[u]), __builtin_bit_cast(bf16x8, b[u][j]), acc[j]);
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

// Router logits for many tokens: LDS-tiled, K split S ways into partials.
// Workgroup tile 128 tokens x 192 experts over chunks [s*cps, s*cps + cps) of
// K; per 64-wide K chunk (128 bytes of bf16) the 320 rows (128 token rows,
// 192 router-weight rows) are copied straight into LDS (a ring of three 40 KB
// stages, two in flight), so a token row fetched once feeds 192 experts and a
// weight row feeds 128 tokens: the copies, which bound this kernel, move
// T*E*H*2*(1/192 + 1/128) bytes in all.  Eight waves, two per SIMD: wave w
// owns tokens [64*(w/4), +64) x experts [48*(w%4), +48) as 4 x 3 MFMA tiles
// of 16x16.  Rows past T or E repeat a valid row and are not stored.
namespace {
constexpr int RT_M = 128, RT_N = 192, RT_ROWS = RT_M + RT_N;
constexpr int RT_STAGE = RT_ROWS * 128, RT_NSTAGE = 3;
constexpr int RT_Q = RT_ROWS / 64;   // copies per lane per chunk (8 waves x 8 rows each)
static_assert(RT_M % 64 == 0 && RT_ROWS % 64 == 0, "copy rows come in groups of 64");
}  // namespace

__global__ __launch_bounds__(512, 1) void router_logits_tiled_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, float *__restrict__ partial, int T, int E,
    int H, int cps) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = lane_id(), w = uniform(wave_id());
  const int t0 = blockIdx.y * RT_M, e0 = blockIdx.x * RT_N, s = blockIdx.z;
  const int64_t rowb = (int64_t)H * 2;
  const int kc0 = s * cps;
  const int nchunk = max(0, min(cps, (int)(rowb / 128) - kc0));
  // this lane's RT_Q copies per chunk: LDS row r = 8 * (w + 8q) + lane / 8
  uint32_t off[RT_Q];
  const uint8_t *src[2] = {reinterpret_cast<const uint8_t *>(x), reinterpret_cast<const uint8_t *>(wr)};
#pragma unroll
  for (int q = 0; q < RT_Q; ++q) {
    const int r = 8 * (w + 8 * q) + (lane >> 3);
    const int c = (lane & 7) ^ swz_f(r);
    const int grow = r < RT_M ? min(t0 + r, T - 1) : min(e0 + r - RT_M, E - 1);
    off[q] = (uint32_t)(grow * rowb + c * 16);
  }
  // q < RT_M / 32: token rows, the rest: weight rows
  auto issue = [&](int kc, uint8_t *sb) {
#pragma unroll
    for (int q = 0; q < RT_Q; ++q)
      dma16(src[q < RT_M / 64 ? 0 : 1] + (int64_t)(kc0 + kc) * 128 + off[q], sb + (w + 8 * q) * 1024);
  };
  const int wm = w >> 2, wn = w & 3;
  f32x4 acc[4][3];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nchunk > 0) issue(0, lds);
  if (nchunk > 1) issue(1, lds + RT_STAGE);
  for (int kc = 0; kc < nchunk; ++kc) {
    if (kc + 2 < nchunk) issue(kc + 2, lds + ((kc + 2) % RT_NSTAGE) * RT_STAGE);
    // chunk kc landed: the copies of kc+1 and kc+2 may still be in flight
    if (kc + 2 < nchunk)
      wait_vm<2 * RT_Q>();
    else if (kc + 1 < nchunk)
      wait_vm<RT_Q>();
    else
      wait_vm<0>();
    wg_barrier();
    const uint8_t *sb = lds + (kc % RT_NSTAGE) * RT_STAGE;
    const int ck = 2 * (lane >> 4);
    i32x4 b[3][2];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int r = RT_M + 48 * wn + 16 * j + (lane & 15);
      b[j][0] = *reinterpret_cast<const i32x4 *>(sb + swz(r, ck));
      b[j][1] = *reinterpret_cast<const i32x4 *>(sb + swz(r, ck + 1));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 64 * wm + 16 * i + (lane & 15);
      const i32x4 a0 = *reinterpret_cast<const i32x4 *>(sb + swz(r, ck));
      const i32x4 a1 = *reinterpret_cast<const i32x4 *>(sb + swz(r, ck + 1));
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8, a0), __builtin_bit_cast(bf16x8, b[j][0]), acc[i][j]);
        acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8, a1), __builtin_bit_cast(bf16x8, b[j][1]), acc[i][j]);
      }
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
      const int e = e0 + 48 * wn + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 64 * wm + 16 * i + 4 * (lane >> 4) + r;
        if (t < T && e < E) partial[((int64_t)s * T + t) * E + e] = acc[i][j][r];
      }
    }
}

// Order-preserving map of a float (NaN excluded) to uint32: a larger float has
// a larger key, and 0 lies below every key (-infinity maps to 0x007FFFFF).
// Callers pass -0 as +0 so that the two zeros tie.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return __builtin_bit_cast(float, (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Largest key over the wave, in every lane: max over each 16-lane row with
// DPP moves (quad exchanges of 1 and 2, row rotations by 4 and 8), then over
// the four rows' results read from lanes 0, 16, 32 and 48.  All 64 lanes must
// be active.
__device__ __forceinline__ uint32_t wave_max_key(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false));   // row_ror:4
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));   // row_ror:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// One wave per token: logits = sum of the S partials (in order s = 0..S-1)
// + bias; k rounds of a wave-wide arg-max under the order (value desc, index
// asc), a NaN logit ranking as -infinity; slots sorted by expert id; gates =
// exp(l - l_max) / sum, fp32, the sum taken over the winners in the order
// they were chosen.
//
// Lane l holds experts [l*NJ, l*NJ + NJ), so among lanes holding the largest
// key the lowest lane holds the lowest expert index (and inside a lane the
// first of equal keys is kept): a round is a DPP max of the lanes' best keys,
// a ballot of the lanes that hold it and the lowest of them, with no
// cross-lane shuffles.  Every winner's id and value are wave-uniform, so the
// slot ranks and the softmax denominator are kept up to date round by round.
template <int NJ, int SB>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float *__restrict__ partial, int S, const float *__restrict__ bias, int T, int E, int k,
    int32_t *__restrict__ ids, float *__restrict__ gates, float *__restrict__ logits_out) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= T) return;
  const int e0 = lane * NJ;
  float v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) v[j] = 0.f;
  // partial sums added in split order; the loads of a batch of SB splits are
  // issued before the first add, so their latencies overlap (SB no larger
  // than the split count needs: the batch's registers set the occupancy)
  for (int s0 = 0; s0 < S; s0 += SB) {
    float pv[SB][NJ];
#pragma unroll
    for (int s = 0; s < SB; ++s) {
      const float *p = partial + ((int64_t)(s0 + s < S ? s0 + s : 0) * T + t) * E + e0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) pv[s][j] = (s0 + s < S && e0 + j < E) ? p[j] : 0.f;
    }
#pragma unroll
    for (int s = 0; s < SB; ++s)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (s0 + s < S) v[j] += pv[s][j];
  }
  uint32_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = e0 + j;
    key[j] = 0;
    if (e < E) {
      if (bias) v[j] += bias[e];
      if (logits_out) logits_out[(int64_t)t * E + e] = v[j];
      const float r = v[j] != v[j] ? -__builtin_huge_valf() : v[j] + 0.0f;   // NaN -> -infinity, -0 -> +0
      key[j] = order_key(r);
    }
  }
  float my_v = 0.f, vmax = 0.f, den = 0.f;
  int my_e = 0, my_rank = 0;
  for (int it = 0; it < k; ++it) {
    uint32_t bk = 0;
    int bj = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (key[j] > bk) {
        bk = key[j];
        bj = j;
      }
    const uint32_t m = wave_max_key(bk);
    const int wl = __builtin_ctzll(__builtin_amdgcn_ballot_w64(bk == m));
    const int ew = __builtin_amdgcn_readlane(e0 + bj, wl);
    const float vw = key_value(m);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (lane == wl && j == bj) key[j] = 0;   // taken
    // earlier winners (lanes < it) against the new one
    const int below = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < it && my_e < ew));
    if (lane < it && ew < my_e) ++my_rank;
    if (lane == it) {
      my_v = vw;
      my_e = ew;
      my_rank = below;
    }
    // a chosen logit equal to the largest weighs exp(0) = 1 (so k chosen
    // -infinity logits, a token whose logits are all NaN, get 1/k each)
    if (it == 0) vmax = vw;
    den += vw == vmax ? 1.0f : expf(vw - vmax);
  }
  if (lane < k) {
    const float ex = my_v == vmax ? 1.0f : expf(my_v - vmax);
    ids[(int64_t)t * k + my_rank] = my_e;
    gates[(int64_t)t * k + my_rank] = __fdiv_rn(ex, den);
  }
}

// Many tokens: the LDS-tiled kernel (one pass, S = 1).
// (per-lane copy offsets are 32-bit: the token rows must span < 2 GiB)
static bool router_tiled(int64_t T, int H) { return T >= 2048 && H % 64 == 0 && T * H * 2 < (int64_t(1) << 31); }

// The tiled kernel's split: enough workgroups for every CU (K chunks of 64
// kept at 8 or more per split).
static int tiled_split(int64_t T, int E, int H) {
  const int64_t tiles = cdiv(E, RT_N) * cdiv(T, RT_M);
  int S = 1;
  while (S < 16 && tiles * S < 256 && (H / 64) / (2 * S) >= 8) S *= 2;
  return S;
}

int router_ksplit(int64_t T, int E, int H) {
  if (router_tiled(T, H)) return tiled_split(T, E, H);
  const int64_t tiles = cdiv(E, 64) * cdiv(T, 64);
  int S = 1;
  // split K (at most 16 ways) until there are enough workgroups, keeping
  // chunks of >= 256 that are multiples of 32
  while (S < 16 && tiles * S < 256 && H % (2 * S) == 0 && (H / (2 * S)) % 32 == 0 && H / (2 * S) >= 256) S *= 2;
  return S;
}

hipError_t launch_router(const uint16_t *x, const uint16_t *wr, const float *bias, int64_t T, int E,
                         int H, int k, float *partial, int S, int32_t *ids, float *gates,
                         float *logits, hipStream_t st) {
  if (T == 0) return hipSuccess;
  timing_before(0, st);
  if (router_tiled(T, H) && S == tiled_split(T, E, H)) {
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
    const int cps = (int)cdiv(H / 64, S);
    dim3 gt((unsigned)cdiv(E, RT_N), (unsigned)cdiv(T, RT_M), (unsigned)S);
    router_logits_tiled_kernel<<<gt, 512, lds, st>>>(x, wr, partial, (int)T, E, H, cps);
  } else {
    dim3 g1((unsigned)cdiv(E, 64), (unsigned)cdiv(T, 64), (unsigned)S);
    router_logits_kernel<<<g1, 256, 0, st>>>(x, wr, partial, (int)T, E, H, H / S);
  }
  timing_after(0, st);
  const unsigned g2 = (unsigned)cdiv(T, 4);
  const int nj = (int)cdiv(E, 64);
  timing_before(1, st);
#define MOE_TOPK_CASE(NJ)                                                                                  \
  case NJ:                                                                                                 \
    if (S <= 2)                                                                                            \
      router_topk_kernel<NJ, 2><<<g2, 256, 0, st>>>(partial, S, bias, (int)T, E, k, ids, gates, logits);   \
    else                                                                                                   \
      router_topk_kernel<NJ, (NJ <= 8 ? 16 : 4)><<<g2, 256, 0, st>>>(partial, S, bias, (int)T, E, k, ids, \
                                                                    gates, logits);                        \
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
