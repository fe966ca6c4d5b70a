// backward.hip -- backward of the routed MoE layer with bf16 experts:
// recompute of the expert pre-activations, the SwiGLU and softmax-gate
// backward, data and weight gradients of the routed and shared experts, and
// the router gradients.  The gradients are those of the layer
//   y[t] = Shared(x[t]) + sum_j g[t,j] FFN_{e_j}(x[t]),  g = softmax over the chosen logits
// ("Step-5-Preview", "Model Architecture": learned top-8 router, one shared
// expert, SwiGLU experts; "Full-Depth H100 Benchmark": the layer is trained
// in BF16).
//
// The backward's GEMMs are grouped bf16 GEMMs C_g = A_g B_g^T over K in two
// kernels, both fed by direct-to-LDS copies (no operand passes through
// registers on its way into LDS).  rows_kernel: groups (experts) own token
// rows (the data gradients dy W_down and dz W_gate_up, and the recompute of
// the pre-activations when the forward did not keep them); the token rows are
// K-contiguous, the expert's weights are read along either axis of their
// stored [out, in] layout ("N" layout: element (r, k) at r*rs + k; "T"
// layout: at k*ks + r).  wgrad_kernel: groups own a token range (the weight
// gradients, sums over an expert's rows), both operands row-contiguous.
// Row-contiguous tiles are staged as stored and read with gfx950's
// transposing LDS read.  fp32 accumulation and output throughout.

#include <algorithm>

#include "../../include/moe_timing.h"
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

// Operand element (r, k) of group g: base + g * gstride + r * rs + k * ks (bf16).
struct GemmOp {
  const uint16_t *base;
  int64_t gstride, rs, ks;
};

struct GemmArgs {
  GemmOp a, b;
  float *c;            // fp32 output, C_g at c + g * cgstride, row pitch ldc
  int64_t ldc, cgstride;
  const int32_t *off;  // [G+1] segment offsets, or NULL: one group owning [0, rows) / [0, K)
  int G, M, N, K;      // M: rows (row-grouped: all rows); K: reduction length (K-grouped: all of it)
  int ntm, ntn;        // tiles along M (K-grouped) and N
  const TileEntry *tiles;  // row-grouped: tile list (entries of the kernel's BM rows) and its header
  const int32_t *hdr;
};

// ---------------------------------------------------------------- weight-gradient GEMM

// C_g [M, N] = sum over p in group g's token range of A[p][m] B[p][n]: both
// operands are row-contiguous in m / n ("T" layout), the K (token) range is
// short (an expert's rows).  The tiles go into LDS as stored -- [k][m] rows of
// 128 bf16 -- by direct-to-LDS copies (a three-stage ring of 32-k steps, two
// steps in flight), and the MFMA fragments (8 consecutive k of one m per
// lane) come out of them with gfx950's transposing LDS read,
// ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element i of
// the 4 x 16 block of 16-bit values whose rows the 16 lanes address (lane j
// reads 4 consecutive m of row j / 4), i.e. 4 consecutive k of one m.  Two
// such reads make one 16x16x32 operand.  128 x 128 output tiles, 4 waves of
// 64 x 64, fp32 accumulation; the output goes out through LDS in whole
// 512-byte rows, non-temporally.
namespace {
constexpr int WBK = 32;                  // K step
constexpr int WROW = 256;                // bytes of one staged k row (128 bf16)
constexpr int WTILE = WBK * WROW;        // 8 KB: one operand's tile of one step

typedef __attribute__((ext_vector_type(2))) int i32x2;

// 32-byte segment permutation of staged k row r: segment s is stored at
// s ^ wseg(r).  Over the 16 rows one transposing read touches (r = 8g + 4h +
// t, g = 0..3, t = 0..3) it takes 8 values twice each, so the 64 lanes'
// 8-byte pieces spread over all banks.
__device__ __forceinline__ int wseg(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }

// Eight transposing reads (addresses a[0..7], byte offsets in LDS), waited for
// inside the block.
__device__ __forceinline__ void lds_read_tr8(const uint32_t (&a)[8], i32x2 (&r)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
}
}  // namespace

// TB x TB output tiles (TB = 128: 4 waves, 3 stages; TB = 256: 16 waves, 4
// stages), one 64 x 64 block per wave; each operand tile of a step is TB / 128
// sub-tiles of 32 k rows x 128 columns.
template <int TB, int NSTG>
__global__ __launch_bounds__((TB / 64) * (TB / 64) * 64) void wgrad_kernel(GemmArgs a) {
  constexpr int NW = (TB / 64) * (TB / 64);
  constexpr int NT = 64 * NW;
  constexpr int WMW = TB / 64;
  constexpr int SUB = TB / 128;              // sub-tiles per operand tile
  constexpr int OPT = SUB * WTILE;           // bytes of one operand tile of a step
  constexpr int STG = 2 * OPT;
  constexpr int CI = 8 * SUB / NW;           // copy instructions per wave per operand per stage
  constexpr int PS = 2 * CI;
  constexpr int LDW = TB + 4;                // floats per staged output row
  static_assert(CI >= 1, "every wave copies");
  static_assert(64 * LDW * 4 <= NSTG * STG, "output staging fits the ring");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NSTG * STG];
  const int per = a.ntm * a.ntn;
  const int g = blockIdx.x / per;
  const int rt = blockIdx.x - g * per;
  const int m0 = (rt / a.ntn) * TB, n0 = (rt % a.ntn) * TB;
  const int kbeg = a.off ? a.off[g] : 0, kend = a.off ? a.off[g + 1] : a.K;
  const int nsteps = (int)cdiv(kend - kbeg, WBK);
  const int lane = lane_id(), w = wave_id();
  const int wm = (w % WMW) * 64, wn = (w / WMW) * 64;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)smem;

  // Copies: instruction q (= w + NW t) covers k rows 4 (q % 8) .. +3 of
  // sub-tile q / 8; lane l -> k row 4 (q % 8) + l / 16, 16-byte slot l % 16
  // of the row, which holds logical column 128 (q / 8) + 16 (slot / 2 ^
  // wseg(row)) + 8 (slot % 2) (clamped inside the operand).
  int am[CI], bn[CI], crow[CI];
#pragma unroll
  for (int t = 0; t < CI; ++t) {
    const int q = w + NW * t;
    crow[t] = 4 * (q & 7) + (lane >> 4);
    const int c = 128 * (q >> 3) + 16 * (((lane & 15) >> 1) ^ wseg(crow[t])) + 8 * (lane & 1);
    am[t] = min(m0 + c, a.M - 8);
    bn[t] = min(n0 + c, a.N - 8);
  }
  auto issue = [&](int step) {
    const int k0 = kbeg + step * WBK;
    uint8_t *st = smem + (step % NSTG) * STG;
#pragma unroll
    for (int t = 0; t < CI; ++t) {
      const int q = w + NW * t;
      const int64_t p = min(k0 + crow[t], kend - 1);
      dma16(a.a.base + p * a.a.ks + am[t], st + q * 1024);
      dma16(a.b.base + p * a.b.ks + bn[t], st + OPT + q * 1024);
    }
  };
  // Transposing reads: lane (g4 = lane / 16, j = lane % 16) reads k row
  // 8 g4 + 4 h + j / 4 (h = half of its 8 k), 4 bf16 at column mb + 4 (j % 4).
  uint32_t ra[8], rb[8];   // per-stage-relative addresses: [2 i + h], [2 j + h]
  {
    const int g4 = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * g4 + 4 * h + (jj >> 2);
      const uint32_t rowb = (uint32_t)(r * WROW + 8 * (jj & 3));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[2 * i + h] = (wm >> 7) * WTILE + rowb + 32 * ((((wm & 127) >> 4) + i) ^ wseg(r));
        rb[2 * i + h] = OPT + (wn >> 7) * WTILE + rowb + 32 * ((((wn & 127) >> 4) + i) ^ wseg(r));
      }
    }
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // NSTG - 1 steps of copies in flight: step s waits until at most the copies
  // of steps s+1 .. s+NSTG-2 are outstanding; the barrier makes every wave's
  // copies visible and frees the stage of step s - 1 for step s + NSTG - 1
#pragma unroll
  for (int q = 0; q < NSTG - 1; ++q)
    if (q < nsteps) issue(q);
  for (int s = 0; s < nsteps; ++s) {
    const int ahead = min(nsteps - 1 - s, NSTG - 2);
    if (ahead >= 2)
      wait_vm<2 * PS>();
    else if (ahead == 1)
      wait_vm<PS>();
    else
      wait_vm<0>();
    wg_barrier();
    if (s + NSTG - 1 < nsteps) issue(s + NSTG - 1);
    const uint32_t sb = lds0 + (uint32_t)((s % NSTG) * STG);
    uint32_t aa[8], ab[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      aa[q] = sb + ra[q];
      ab[q] = sb + rb[q];
    }
    i32x2 fa2[8], fb2[8];
    lds_read_tr8(aa, fa2);
    lds_read_tr8(ab, fb2);
    i32x4 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = i32x4{fa2[2 * i][0], fa2[2 * i][1], fa2[2 * i + 1][0], fa2[2 * i + 1][1]};
      fb[i] = i32x4{fb2[2 * i][0], fb2[2 * i][1], fb2[2 * i + 1][0], fb2[2 * i + 1][1]};
    }
    const int k0 = kbeg + s * WBK;
    if (k0 + WBK > kend) {
      // last step: zero the A values of k >= kend (their copies repeated row kend - 1)
      const int cnt = min(max(kend - (k0 + 8 * (lane >> 4)), 0), 8);   // valid k of this lane's 8
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t mk = (2 * q < cnt ? 0xFFFFu : 0u) | (2 * q + 1 < cnt ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i][q] = (int)((uint32_t)fa[i][q] & mk);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8, fb[j]), __builtin_bit_cast(bf16x8, fa[i]), acc[i][j]);
  }
  // lane holds C[lane % 16][4 (lane / 16) + r] of each 16 x 16 block; the
  // tile goes out 64 rows (one row of waves) at a time through LDS so that
  // every store writes whole rows of TB floats
  wg_barrier();
  float *stage = reinterpret_cast<float *>(smem);
  float *cbase = a.c + (int64_t)g * a.cgstride;
#pragma unroll
  for (int part = 0; part < WMW; ++part) {
    if (w % WMW == part) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4 *>(stage + (16 * i + (lane & 15)) * LDW + wn + 16 * j + 4 * (lane >> 4)) =
              acc[i][j];
    }
    __syncthreads();
#pragma unroll
    for (int q = threadIdx.x; q < 64 * TB / 4; q += NT) {
      const int row = q / (TB / 4), c4 = q % (TB / 4);
      const int m = m0 + 64 * part + row, n = n0 + 4 * c4;
      if (m < a.M && n < a.N)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4 *>(stage + row * LDW + 4 * c4),
                                    reinterpret_cast<f32x4 *>(cbase + (int64_t)m * a.ldc + n));
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- row-grouped GEMM, copy-staged

// C[row, n] = sum_k A(row, k) B_g(n, k) for the rows of group g (rows
// [off[g], off[g+1]), walked through a tile list of BM-row entries), with
// both tiles copied into LDS by direct-to-LDS loads
// (a three-stage ring of 32-k steps, two in flight): the token rows (K
// contiguous) as 64-byte staged rows read with ds_read_b128, the weights
// either the same way (N layout) or as [k][n] rows read with the transposing
// ds_read_b64_tr_b16 (T layout), so no operand passes through registers on
// its way into LDS.  BM x 128 tiles (BM = 256 or 128), one 64 x 64 block per
// wave.
namespace {
constexpr int RBK = 32;
constexpr int RBN256 = 256;   // columns of the 256-row tiles
constexpr int RNS256 = 4;     // their LDS stages
constexpr int RBT = 128 * RBK * 2;       // bytes of the weight tile of one step

// 16-byte unit u of staged 64-byte row r is stored at u ^ rsw(r): the 16 rows
// x 4 units of one fragment read (and of one copy) cover every bank once.
__device__ __forceinline__ int rsw(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ void lds_read4(const uint32_t (&a)[4], i32x4 (&r)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}
}  // namespace

template <int BM, int BN, int NSTG, bool BTL>
__global__ __launch_bounds__((BM / 64) * (BN / 64) * 64) void rows_kernel(GemmArgs a) {
  constexpr int NW = (BM / 64) * (BN / 64);   // waves, one 64 x 64 block each
  constexpr int WMW = BM / 64;                // waves along M
  constexpr int RAT = BM * RBK * 2;           // bytes of the token tile of one step
  constexpr int STAGE = RAT + BN * RBK * 2;
  constexpr int AI = BM / 16 / NW;            // token-tile copy instructions per wave
  constexpr int BI = BN / 16 / NW;            // weight-tile copy instructions per wave
  constexpr int PS = AI + BI;                 // copy instructions per wave per stage
  static_assert(AI >= 1 && BI >= 1, "every wave copies");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NSTG * STAGE];
  const int tile = blockIdx.x / a.ntn;
  if (tile >= a.hdr[0]) return;
  const int n0 = (blockIdx.x - tile * a.ntn) * BN;
  const TileEntry te = a.tiles[tile];
  const int g = te.ge & 0xFFFFFF;
  const int m0 = (a.off ? a.off[g] : 0) + te.m0;
  const int mend = a.off ? a.off[g + 1] : a.M;
  const int nsteps = a.K / RBK;
  const uint16_t *abase = a.a.base;
  const uint16_t *bbase = a.b.base + (int64_t)g * a.b.gstride;
  const int lane = lane_id(), w = wave_id();
  const int wm = (w % WMW) * 64, wn = (w / WMW) * 64;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)smem;

  // Token copies: instruction q (= w + NW t) covers staged rows 16q .. 16q+15;
  // lane l -> row 16q + l / 4, slot l % 4 = logical unit (l % 4) ^ rsw(row),
  // i.e. k = 8 unit.  Rows past the group's end repeat its last row (their
  // outputs are not stored).
  int64_t aoff[AI];
#pragma unroll
  for (int t = 0; t < AI; ++t) {
    const int r = 16 * (w + NW * t) + (lane >> 2);
    aoff[t] = (int64_t)min(m0 + r, mend - 1) * a.a.rs + 8 * ((lane & 3) ^ rsw(r));
  }
  // Weight copies.  N layout: like the tokens, BN rows (weight rows beyond N
  // repeat row N - 1).  T layout: BN / 128 sub-tiles of 32 k rows x 128
  // columns (256 bytes); instruction q covers k rows 4 (q % 8) .. +3 of
  // sub-tile q / 8, lane l -> k row 4 (q % 8) + l / 16, 16-byte slot l % 16
  // = logical column 128 (q / 8) + 16 ((slot / 2) ^ wseg(row)) + 8 (slot % 2)
  // (clamped inside N).
  int64_t boff[BI];
#pragma unroll
  for (int t = 0; t < BI; ++t) {
    const int q = w + NW * t;
    if constexpr (!BTL) {
      const int r = 16 * q + (lane >> 2);
      boff[t] = (int64_t)min(n0 + r, a.N - 1) * a.b.rs + 8 * ((lane & 3) ^ rsw(r));
    } else {
      const int r = 4 * (q & 7) + (lane >> 4);
      const int n = 128 * (q >> 3) + 16 * (((lane & 15) >> 1) ^ wseg(r)) + 8 * (lane & 1);
      boff[t] = (int64_t)r * a.b.ks + min(n0 + n, a.N - 8);
    }
  }
  auto issue = [&](int step) {
    const int k0 = step * RBK;
    uint8_t *st = smem + (step % NSTG) * STAGE;
#pragma unroll
    for (int t = 0; t < AI; ++t) dma16(abase + aoff[t] + k0, st + (w + NW * t) * 1024);
#pragma unroll
    for (int t = 0; t < BI; ++t)
      dma16(bbase + boff[t] + (BTL ? (int64_t)k0 * a.b.ks : (int64_t)k0), st + RAT + (w + NW * t) * 1024);
  };
  // Fragment reads (stage-relative).  Tokens: row wm + 16 i + lane % 16,
  // unit lane / 16.  Weights, N layout: row wn + 16 j + lane % 16; T layout:
  // two transposing reads of k rows 8 (lane / 16) + 4 h + (lane % 16) / 4, 4
  // values at column wn + 16 j + 4 (lane % 4).
  uint32_t ra[4], rb[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wm + 16 * i + (lane & 15);
    ra[i] = (uint32_t)(r * 64 + 16 * ((lane >> 4) ^ rsw(r)));
  }
  if constexpr (!BTL) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn + 16 * j + (lane & 15);
      rb[j] = (uint32_t)(RAT + r * 64 + 16 * ((lane >> 4) ^ rsw(r)));
    }
  } else {
    const int g4 = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * g4 + 4 * h + (jj >> 2);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        rb[2 * j + h] = (uint32_t)(RAT + (wn >> 7) * RBT + r * WROW + 8 * (jj & 3) +
                                   32 * ((((wn & 127) >> 4) + j) ^ wseg(r)));
    }
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // NSTG - 1 steps of copies in flight: step s waits until at most the copies
  // of steps s+1 .. s+NSTG-2 are outstanding
#pragma unroll
  for (int q = 0; q < NSTG - 1; ++q)
    if (q < nsteps) issue(q);
  for (int s = 0; s < nsteps; ++s) {
    const int ahead = min(nsteps - 1 - s, NSTG - 2);
    if (ahead >= 2)
      wait_vm<2 * PS>();
    else if (ahead == 1)
      wait_vm<PS>();
    else
      wait_vm<0>();
    wg_barrier();
    if (s + NSTG - 1 < nsteps) issue(s + NSTG - 1);
    const uint32_t sb = lds0 + (uint32_t)((s % NSTG) * STAGE);
    uint32_t aa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aa[i] = sb + ra[i];
    i32x4 fa[4], fb[4];
    lds_read4(aa, fa);
    if constexpr (!BTL) {
      uint32_t ab[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ab[j] = sb + rb[j];
      lds_read4(ab, fb);
    } else {
      uint32_t ab[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) ab[q] = sb + rb[q];
      i32x2 f2[8];
      lds_read_tr8(ab, f2);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = i32x4{f2[2 * j][0], f2[2 * j][1], f2[2 * j + 1][0], f2[2 * j + 1][1]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8, fb[j]), __builtin_bit_cast(bf16x8, fa[i]), acc[i][j]);
  }
  // lane holds C[lane % 16][4 (lane / 16) + r] of each 16 x 16 block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm + 16 * i + (lane & 15);
    if (m >= mend) continue;
    float *crow = a.c + (int64_t)m * a.ldc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + 16 * j + 4 * (lane >> 4);
      if (n < a.N) *reinterpret_cast<f32x4 *>(crow + n) = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------- element-wise steps

// Gate of row p: gates[perm_src[p]] (routed rows), 1 for the shared expert.
__device__ __forceinline__ float row_gate(const float *gates, const int32_t *perm_src, int64_t p) {
  return gates ? gates[perm_src[p]] : 1.0f;
}

// One wave per row p, 4 consecutive columns per lane at a time (I % 4 == 0):
//   h = silu(z_gate) z_up;  hg[p] = g h (bf16, the down layer's input as seen
//   by dW_down);  dg[p] = <u[p], h> with u = dy W_down, so that dg is the
//   gate's gradient <dy, FFN(x)> (lane partial sums, then the wave tree: a
//   fixed order);  with dh = g u, the SwiGLU backward
//   dz_up = dh silu(z_gate),  dz_gate = dh z_up sigma(z_gate) (1 + z_gate (1 - sigma(z_gate))),
//   stored bf16 as [gate half | up half], the layout of z.
__global__ __launch_bounds__(256) void bwd_swiglu_kernel(const float *__restrict__ z, const float *__restrict__ u,
                                                         const float *__restrict__ gates,
                                                         const int32_t *__restrict__ perm_src,
                                                         const int32_t *__restrict__ kept, int64_t N, int I,
                                                         uint16_t *__restrict__ hg, uint16_t *__restrict__ dz,
                                                         float *__restrict__ dg) {
  const int64_t p = (int64_t)blockIdx.x * 4 + wave_id();
  if (p >= (kept ? *kept : N)) return;
  const int lane = lane_id();
  const float g = row_gate(gates, perm_src, p);
  const float *zr = z + p * 2 * I, *ur = u + p * I;
  uint16_t *hr = hg + p * I, *dr = dz + p * 2 * I;
  float acc = 0.f;
  for (int i = 4 * lane; i < I; i += 4 * kWave) {
    const f32x4 zg = *reinterpret_cast<const f32x4 *>(zr + i);
    const f32x4 zu = *reinterpret_cast<const f32x4 *>(zr + I + i);
    const f32x4 uu = *reinterpret_cast<const f32x4 *>(ur + i);
    uint32_t h16[4], g16[4], u16[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-zg[q]));
      const float hv = zg[q] * sg * zu[q];
      const float dh = g * uu[q];
      acc = __builtin_fmaf(uu[q], hv, acc);
      h16[q] = f32_to_bf16(g * hv);
      u16[q] = f32_to_bf16(dh * zg[q] * sg);
      g16[q] = f32_to_bf16(dh * zu[q] * sg * (1.0f + zg[q] * (1.0f - sg)));
    }
    *reinterpret_cast<uint2 *>(hr + i) = make_uint2(h16[0] | (h16[1] << 16), h16[2] | (h16[3] << 16));
    *reinterpret_cast<uint2 *>(dr + i) = make_uint2(g16[0] | (g16[1] << 16), g16[2] | (g16[3] << 16));
    *reinterpret_cast<uint2 *>(dr + I + i) = make_uint2(u16[0] | (u16[1] << 16), u16[2] | (u16[3] << 16));
  }
  acc = wave_sum(acc);
  if (dg && lane == 0) dg[p] = acc;
}

// One thread per token: softmax backward over its k chosen logits,
// dl_j = g_j (dg_j - sum_m g_m dg_m), written at the slots' rows.
__global__ void bwd_dl_kernel(const float *__restrict__ dg, const float *__restrict__ gates,
                              const int32_t *__restrict__ perm_pos, int64_t T, int k, float *__restrict__ dl) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float s = 0.f;
  for (int j = 0; j < k; ++j) {
    const int32_t p = perm_pos[t * k + j];
    if (p >= 0) s = __builtin_fmaf(gates[t * k + j], dg[p], s);
  }
  for (int j = 0; j < k; ++j) {
    const int32_t p = perm_pos[t * k + j];
    if (p >= 0) dl[p] = gates[t * k + j] * (dg[p] - s);
  }
}

// Router weight gradient: dW_r[e][h] = sum over e's rows p (in order) of
// dl[p] x_perm[p][h], 8 consecutive h per thread (H % 8 == 0); dbias[e] =
// sum of dl[p].  Grid (E, ceil(H / 2048)).
__global__ __launch_bounds__(256) void bwd_router_w_kernel(const float *__restrict__ dl,
                                                           const uint16_t *__restrict__ x_perm,
                                                           const int32_t *__restrict__ off, int H,
                                                           float *__restrict__ dwr, float *__restrict__ dbias) {
  const int e = blockIdx.x;
  const int h = (blockIdx.y * 256 + threadIdx.x) * 8;
  const int p0 = off[e], p1 = off[e + 1];
  if (h < H) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int p = p0; p < p1; ++p) {
      const float d = dl[p];
      const i32x4 v = load16(x_perm + (int64_t)p * H + h);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(d, bf16_to_f32(((uint32_t)v[q >> 1] >> (16 * (q & 1))) & 0xFFFFu), acc[q]);
    }
    float *o = dwr + (int64_t)e * H + h;
    *reinterpret_cast<f32x4 *>(o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4 *>(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
  if (dbias && blockIdx.y == 0 && threadIdx.x == 0) {
    float s = 0.f;
    for (int p = p0; p < p1; ++p) s += dl[p];
    dbias[e] = s;
  }
}

// dx[t] = dx_shared[t] + sum_j dx_rows[row of (t, j)] + sum_j dl_j W_r[e_j],
// fp32, in that order (slots in increasing j); 4 consecutive h per thread
// (H % 4 == 0).  Grid (T, ceil(H / 1024)).
__global__ __launch_bounds__(256) void bwd_dx_kernel(const float *__restrict__ dx_shared,
                                                     const float *__restrict__ dx_rows,
                                                     const int32_t *__restrict__ perm_pos,
                                                     const int32_t *__restrict__ ids, const float *__restrict__ dl,
                                                     const uint16_t *__restrict__ wr, int k, int H,
                                                     float *__restrict__ dx) {
  const int64_t t = blockIdx.x;
  const int h = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (h >= H) return;
  f32x4 acc = dx_shared ? *reinterpret_cast<const f32x4 *>(dx_shared + t * H + h) : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int32_t p = perm_pos[t * k + j];
    if (p >= 0) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(dx_rows + (int64_t)p * H + h);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += v[q];
    }
  }
  for (int j = 0; j < k; ++j) {
    const int32_t p = perm_pos[t * k + j];
    if (p >= 0) {
      const float d = dl[p];
      const uint2 w = *reinterpret_cast<const uint2 *>(wr + (int64_t)ids[t * k + j] * H + h);
      acc[0] = __builtin_fmaf(d, bf16_to_f32(w.x & 0xFFFFu), acc[0]);
      acc[1] = __builtin_fmaf(d, bf16_to_f32(w.x >> 16), acc[1]);
      acc[2] = __builtin_fmaf(d, bf16_to_f32(w.y & 0xFFFFu), acc[2]);
      acc[3] = __builtin_fmaf(d, bf16_to_f32(w.y >> 16), acc[3]);
    }
  }
  *reinterpret_cast<f32x4 *>(dx + t * H + h) = acc;
}

// ---------------------------------------------------------------- host side

namespace {

bool op_t(const GemmOp &o) { return o.ks != 1; }

// Row-grouped GEMM: rows of group g are [off[g], off[g+1]) (or [0, rows)
// when off is NULL), walked through the tile list in tiles_ws (entries of bm
// rows); C[row, n] = sum_k A(row, k) B_g(n, k).  A must be N-layout and K a
// multiple of the K step.
hipError_t gemm_rows(const GemmOp &A, const GemmOp &B, float *c, int64_t ldc, const int32_t *off, int G, int64_t rows,
                     int N, int K, const int32_t *tiles_ws, int bm, int max_tiles, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (op_t(A) || K % RBK != 0 || N % 8 != 0 || (op_t(B) && B.rs != 1)) return hipErrorInvalidValue;
  const TileEntry *tiles = reinterpret_cast<const TileEntry *>(tiles_ws + kTileHdrWords);
  GemmArgs a{A, B, c, ldc, 0, off, G, (int)rows, N, K, 0, (int)cdiv(N, bm == 256 ? RBN256 : 128), tiles, tiles_ws};
  const int64_t blocks = (int64_t)max_tiles * a.ntn;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const bool bt = op_t(B);
  timing_before(MOE_SITE_BWD_DGRAD, st);
  if (bm == 256) {
    if (bt) rows_kernel<256, RBN256, RNS256, true><<<(unsigned)blocks, 4 * RBN256, 0, st>>>(a);
    else rows_kernel<256, RBN256, RNS256, false><<<(unsigned)blocks, 4 * RBN256, 0, st>>>(a);
  } else {
    if (bt) rows_kernel<128, 128, 3, true><<<(unsigned)blocks, 256, 0, st>>>(a);
    else rows_kernel<128, 128, 3, false><<<(unsigned)blocks, 256, 0, st>>>(a);
  }
  timing_after(MOE_SITE_BWD_DGRAD, st);
  return hipGetLastError();
}

// K-grouped GEMM: C_g [M, N] = sum over k in group g's range of A(m, k) B(n, k),
// for every group (a group with an empty range gets zeros).  Both operands
// T-layout.
hipError_t gemm_kseg(const GemmOp &A, const GemmOp &B, float *c, int64_t ldc, int64_t cgstride, const int32_t *off,
                     int G, int M, int N, int K, hipStream_t st) {
  if (!op_t(A) || !op_t(B)) return hipErrorInvalidValue;
  if (M % 8 != 0 || N % 8 != 0) return hipErrorInvalidValue;
  // 256 x 256 tiles when both dimensions fill them and there are enough of
  // them to keep every CU busy twice over (the shared expert, one group with a
  // long token range, has few), else 128 x 128
  const int tb = (M >= 256 && N >= 256 && (int64_t)G * cdiv(M, 256) * cdiv(N, 256) >= 2 * num_compute_units()) ? 256
                                                                                                          : 128;
  GemmArgs a{A, B, c, ldc, cgstride, off, G, M, N, K, (int)cdiv(M, tb), (int)cdiv(N, tb), nullptr, nullptr};
  const int64_t blocks = (int64_t)G * a.ntm * a.ntn;
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  timing_before(MOE_SITE_BWD_WGRAD, st);
  if (tb == 256)
    wgrad_kernel<256, 4><<<(unsigned)blocks, 1024, 0, st>>>(a);
  else
    wgrad_kernel<128, 3><<<(unsigned)blocks, 256, 0, st>>>(a);
  timing_after(MOE_SITE_BWD_WGRAD, st);
  return hipGetLastError();
}

// Row tile height for a row-grouped launch: 256-row tiles (256 columns, a
// four-stage copy ring; each group's weight column block is streamed once for
// up to 256 rows) unless the groups hold so few rows on average that half a
// 256-row tile would stay empty, then 128 x 128 tiles.
int row_tile(int64_t rows, int G) { return cdiv(rows, G) >= 128 ? 256 : 128; }
int max_tiles_for(int64_t rows, int G, int bm) { return (int)(cdiv(rows, bm) + std::min<int64_t>(rows, G) + 1); }

}  // namespace

int bwd_max_tiles(int64_t rows, int G) { return max_tiles_for(rows, G, 128); }

hipError_t launch_expert_backward(const BwdExpert &X, hipStream_t st) {
  const int H = X.H, I = X.I, G = X.G;
  const int64_t N = X.rows;
  hipError_t e;
  if (N > 0) {
    const int bm = row_tile(N, G);
    const int mt = max_tiles_for(N, G, bm);
    if (mt > X.max_tiles) return hipErrorInvalidValue;
    FfnGroup fg{};
    fg.off = X.off;
    fg.E = G;
    fg.nrows = (int32_t)N;
    e = launch_build_tiles(fg, bm, mt, reinterpret_cast<TileEntry *>(X.tiles + kTileHdrWords), X.tiles, st);
    if (e != hipSuccess) return e;
    // z = x W_gu^T: B(n = j, k = h) = W_gu[g][j][h] (unless the forward kept it)
    if (!X.z_given) {
      e = gemm_rows(GemmOp{X.x, 0, H, 1}, GemmOp{X.wgu, (int64_t)2 * I * H, H, 1}, X.z, 2 * I, X.off, G, N, 2 * I, H,
                    X.tiles, bm, mt, st);
      if (e != hipSuccess) return e;
    }
    // u = dy W_d: B(n = i, k = c) = W_d[g][c][i]
    e = gemm_rows(GemmOp{X.dy, 0, H, 1}, GemmOp{X.wd, (int64_t)H * I, 1, I}, X.u, I, X.off, G, N, I, H, X.tiles, bm,
                  mt, st);
    if (e != hipSuccess) return e;
    // rows past off[G] (assignments the sort dropped) belong to no expert
    const int32_t *kept = X.off ? X.off + G : nullptr;
    bwd_swiglu_kernel<<<(unsigned)cdiv(N, 4), 256, 0, st>>>(X.z, X.u, X.gates, X.perm_src, kept, N, I, X.hg, X.dz,
                                                            X.dg);
    if (X.dl) bwd_dl_kernel<<<(unsigned)cdiv(X.T, 256), 256, 0, st>>>(X.dg, X.gates, X.perm_pos, X.T, X.k, X.dl);
    // dx rows = dz W_gu: B(n = h, k = j) = W_gu[g][j][h]
    e = gemm_rows(GemmOp{X.dz, 0, 2 * I, 1}, GemmOp{X.wgu, (int64_t)2 * I * H, 1, H}, X.dx_rows, H, X.off, G, N, H,
                  2 * I, X.tiles, bm, mt, st);
    if (e != hipSuccess) return e;
  }
  // dW_d[g] = dy^T hg over g's rows: A(m = c, k = p) = dy[p][c], B(n = i, k = p) = hg[p][i]
  e = gemm_kseg(GemmOp{X.dy, 0, 1, H}, GemmOp{X.hg, 0, 1, I}, X.dwd, I, (int64_t)H * I, X.off, G, H, I, (int)N, st);
  if (e != hipSuccess) return e;
  // dW_gu[g] = dz^T x over g's rows: A(m = j, k = p) = dz[p][j], B(n = h, k = p) = x[p][h]
  return gemm_kseg(GemmOp{X.dz, 0, 1, 2 * I}, GemmOp{X.x, 0, 1, H}, X.dwgu, H, (int64_t)2 * I * H, X.off, G, 2 * I,
                   H, (int)N, st);
}

hipError_t launch_router_backward(const float *dl, const uint16_t *x_perm, const int32_t *off, int E, int H,
                                  float *dwr, float *dbias, hipStream_t st) {
  bwd_router_w_kernel<<<dim3((unsigned)E, (unsigned)cdiv(H, 2048)), 256, 0, st>>>(dl, x_perm, off, H, dwr, dbias);
  return hipGetLastError();
}

hipError_t launch_dx_backward(const float *dx_shared, const float *dx_rows, const int32_t *perm_pos,
                              const int32_t *ids, const float *dl, const uint16_t *wr, int64_t T, int k, int H,
                              float *dx, hipStream_t st) {
  if (T == 0) return hipSuccess;
  bwd_dx_kernel<<<dim3((unsigned)T, (unsigned)cdiv(H, 1024)), 256, 0, st>>>(dx_shared, dx_rows, perm_pos, ids, dl, wr,
                                                                          k, H, dx);
  return hipGetLastError();
}

}  // namespace moe
