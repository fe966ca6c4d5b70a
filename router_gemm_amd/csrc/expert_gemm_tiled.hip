// expert_gemm_tiled.hip -- the grouped expert GEMMs for experts with many
// rows (prefill): LDS-tiled, double-buffered, persistent and XCD-aware.  Two
// work-item shapes share the design below: 256 weight rows x 128 token rows
// on 4 waves (tiled_ffn_kernel, experts with 10..127 rows on average) and
// 256 x 256 on 8 waves (wide_ffn_kernel, 128 rows or more, 96 with fp8 weights; see "wide tiles"
// further down).  Weights come row-major or as tile16 tiles (FfnGroup::tile16),
// which are copied into LDS verbatim and read in fragment order.
//
// Same operation as the streaming kernels in expert_gemm.hip (gate/up with a
// fused SwiGLU epilogue, then down; "Step-5 minimal inference", introduction:
// block-scaled FP8 expert GEMM), organised for reuse:
//   - a workgroup tile is 256 weight rows x 128 token rows; each 128-byte K
//     chunk of both (one fp8 scale block, or 64 bf16 values) is copied straight
//     from HBM into LDS by direct-to-LDS loads (48 KB per stage, a ring of
//     three stages, two in flight while the third is consumed), so a weight
//     byte fetched once feeds 128 tokens and a token byte feeds 256 weight rows;
//   - 4 waves = 2 (weight halves of 128 rows) x 2 (token halves); a wave owns
//     8 x 4 MFMA tiles of 16x16 (128 rows x 64 tokens, 128 fp32 accumulators
//     per lane), with its token sub-tiles interleaved (16-row slices
//     wm, wm+2, wm+4, wm+6) so that a partly filled tile idles both waves
//     equally and slices beyond the last row skip their MFMAs;
//   - LDS rows are 128 bytes with the 16-byte column XOR-swizzled by row % 8,
//     so the MFMA operand reads (8 lanes = 8 consecutive rows) hit distinct banks;
//   - the grid is one workgroup per CU; work items (tile-list slot x column
//     tile) are split into 8 contiguous ranges of equal cost, one per XCD
//     (workgroup i runs on XCD i % 8); inside a range, items come in bands of
//     up to 8 token tiles of one expert, column-tile-major, so that the
//     workgroups of an XCD that run at the same time share weight and token
//     tiles in its L2.

#include <algorithm>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {
constexpr int TBN = 256;                    // weight rows per workgroup tile
constexpr int TBM = 128;                    // token rows per workgroup tile
constexpr int TW = TBN * 128;               // weight bytes per stage
constexpr int TX = TBM * 128;               // token bytes per stage
constexpr int TSX = 1024;                   // token scales per stage (4 waves x 256 B)
constexpr int TSTAGE = TW + TX + TSX;       // bytes per LDS stage
constexpr int NSTAGE = 3;
constexpr int TTHREADS = 256;

constexpr int TBAND = 8;      // token tiles of one expert whose items are interleaved

struct TiledArgs {
  FfnGroup g0, g1;
  const TileEntry *tiles;
  const int32_t *hdr;     // [0] tile count, [1] tiles of group 0
  int H;
  int nt;                 // column tiles per tile-list slot (largest over the groups)
  int c0, c1;             // K chunks of one item of group 0 / group 1 (its cost)
};

}  // namespace

// One work item: a 256 x 128 output tile (gate/up: 128 gate + the matching 128
// up rows = 128 h columns; down: 256 output columns) of one expert.
template <bool FP8, bool GATEUP, bool T16>
struct TiledItem {
  // ---- set up by the constructor
  const FfnGroup &G;
  int e, rbeg, rend, nvalid, I, K, KB, nchunk, col0, ntile, H;
  int64_t wrows;   // rows of the expert's weight matrix (2I or H)
  int64_t rowb;
  const uint8_t *wsrc, *asrc;
  const float *ascale;
  int lane, w, wn, wm;
  uint32_t woff[8], xoff[4], soff;   // per-lane byte offsets of this lane's copies

  __device__ TiledItem(const FfnGroup &g, const TileEntry &te, int nt_, int H_) : G(g), ntile(nt_), H(H_) {
    lane = threadIdx.x & 63;
    w = uniform(threadIdx.x >> 6);
    wn = w & 1;
    wm = w >> 1;
    e = te.ge & 0xFFFFFF;
    rend = min(max(group_off(G, e + 1), 0), G.nrows);
    rbeg = min(max(group_off(G, e), 0) + te.m0, rend);
    nvalid = min(rend - rbeg, TBM);
    I = G.I;
    K = GATEUP ? H : I;
    rowb = (int64_t)K * (FP8 ? 1 : 2);
    nchunk = (int)(rowb / 128);
    KB = K / 128;
    col0 = GATEUP ? ntile * 128 : ntile * TBN;
    wsrc = GATEUP ? G.wgu + (int64_t)e * 2 * I * rowb : G.wd + (int64_t)e * H * rowb;
    wrows = GATEUP ? 2 * (int64_t)I : (int64_t)H;
    const bool indirect = GATEUP && G.xsrc != nullptr;
    asrc = (GATEUP ? G.x : G.h) + (indirect ? 0 : (int64_t)rbeg * rowb);
    ascale = (GATEUP ? G.xs : G.hs) + (FP8 && !indirect ? (int64_t)rbeg * KB : 0);
    const int sub = lane >> 3;   // row within an 8-row group
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = 8 * (w + 4 * q) + sub;
      const int c = (lane & 7) ^ swz_f(r);   // logical 16-byte column landing in this lane's slot
      const int grow = GATEUP ? (r < 128 ? col0 + r : I + col0 + r - 128) : col0 + r;
      if constexpr (T16) {
        // tile16 weights: instruction j = w + 4q copies half j % 2 of the
        // item's 16-row tile j / 2 verbatim (LDS keeps the fragment-major tile)
        const int j = w + 4 * q, rt = 16 * (j >> 1);
        const int g0 = GATEUP ? (rt < 128 ? col0 + rt : I + col0 + rt - 128) : col0 + rt;
        woff[q] = (uint32_t)(((int64_t)g0 >> 4) * 2048 + 1024 * (j & 1) + 16 * lane);
      } else {
        woff[q] = (uint32_t)(grow * rowb + c * 16);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 8 * (w + 4 * q) + sub;
      const int c = (lane & 7) ^ swz_f(r);
      // rows past the end repeat a valid row; indirect rows come from x row xsrc[row] / xdiv
      const int rr = min(r, nvalid - 1);
      const int64_t src = indirect ? G.xsrc[rbeg + rr] / G.xdiv : rr;
      xoff[q] = (uint32_t)(src * rowb + c * 16);
    }
    {
      const int rr = min(32 * w + (lane & 31), nvalid - 1);
      const int64_t src = indirect ? G.xsrc[rbeg + rr] / G.xdiv : rr;
      soff = (uint32_t)(src * KB * 4);
    }
  }

  // Issue the direct-to-LDS copies of K chunk kc into stage buffer sb:
  // 8 (weights) + 4 (tokens) [+ 1 (token scales, fp8)] instructions per wave.
  __device__ __forceinline__ void issue(int kc, uint8_t *sb) const {
    const uint8_t *wb = wsrc + (int64_t)kc * (T16 ? 128 * wrows : 128);   // uniform bases, per-lane 32-bit offsets
    const uint8_t *xb = asrc + (int64_t)kc * 128;
#pragma unroll
    for (int q = 0; q < 8; ++q) dma16(wb + woff[q], sb + (w + 4 * q) * 1024);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(xb + xoff[q], sb + TW + (w + 4 * q) * 1024);
    if constexpr (FP8) dma4(reinterpret_cast<const uint8_t *>(ascale + kc) + soff, sb + TW + TX + 256 * w);
  }

  // Operands of one K chunk for this wave, read from LDS into registers.
  // A (weight) fragments: one set, refilled in place with the next chunk's
  // tile i right after tile i's MFMAs are issued.  B (token) fragments and
  // scales: two sets, the next chunk's read at the start of a step.
  struct AFrags {
    i32x4 al[8], ah[8];
  };
  template <int NJ>
  struct BFrags {
    i32x4 bl[NJ], bh[NJ];
    float sx[NJ];
    float sa, sb;
  };

  __device__ __forceinline__ int arow(int i) const {
    return (GATEUP ? (i < 4 ? 64 * wn + 16 * i : 128 + 64 * wn + 16 * (i - 4)) : 128 * wn + 16 * i) + (lane & 15);
  }

  __device__ __forceinline__ void read_a(const uint8_t *sb, int i, AFrags &A) const {
    if constexpr (T16) {   // fragment-major tile (arow(i) - lane % 16) / 16: lane l at 16 l and 1024 + 16 l
      const uint8_t *t = sb + 128 * (arow(i) - (lane & 15)) + 16 * lane;
      A.al[i] = *reinterpret_cast<const i32x4 *>(t);
      A.ah[i] = *reinterpret_cast<const i32x4 *>(t + 1024);
    } else {
      const int ck = 2 * (lane >> 4);
      A.al[i] = *reinterpret_cast<const i32x4 *>(sb + swz(arow(i), ck));
      A.ah[i] = *reinterpret_cast<const i32x4 *>(sb + swz(arow(i), ck + 1));
    }
  }

  template <int NJ>
  __device__ __forceinline__ void read_b(const uint8_t *sb, const float *wsc, int kc, BFrags<NJ> &F) const {
    const int ck = 2 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = 16 * (wm + 2 * j) + (lane & 15);
      F.bl[j] = *reinterpret_cast<const i32x4 *>(sb + TW + swz(r, ck));
      F.bh[j] = *reinterpret_cast<const i32x4 *>(sb + TW + swz(r, ck + 1));
      // token r's scale sits in wave (r / 32)'s slot, lane r % 32
      if constexpr (FP8) F.sx[j] = *reinterpret_cast<const float *>(sb + TW + TX + 256 * (r >> 5) + 4 * (r & 31));
    }
    if constexpr (FP8) {
      F.sa = GATEUP ? wsc[kc] : wsc[wn * KB + kc];
      F.sb = GATEUP ? wsc[KB + kc] : F.sa;
    }
  }

  // Chunk MFMAs from (A, F); A is refilled tile by tile from buffer `next`.
  template <int NJ>
  __device__ __forceinline__ void mma(AFrags &A, const BFrags<NJ> &F, const uint8_t *next, f32x4 (&acc)[8][4]) const {
    if constexpr (FP8) {
      // Raw block products are folded into the accumulators one weight tile
      // behind, so tile i's MFMAs are in flight while tile i-1's products are
      // scaled in by FMAs.
      float sc[2][NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        sc[0][j] = F.sa * F.sx[j];
        sc[1][j] = F.sb * F.sx[j];
      }
      constexpr int NT = 8 * NJ;
      f32x4 prev = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t <= NT; ++t) {
        f32x4 cur = {0.f, 0.f, 0.f, 0.f};
        if (t < NT) {
          const int i = t / NJ, j = t % NJ;
          const i32x8 a8 = {A.al[i][0], A.al[i][1], A.al[i][2], A.al[i][3],
                            A.ah[i][0], A.ah[i][1], A.ah[i][2], A.ah[i][3]};
          const i32x8 b8 = {F.bl[j][0], F.bl[j][1], F.bl[j][2], F.bl[j][3],
                            F.bh[j][0], F.bh[j][1], F.bh[j][2], F.bh[j][3]};
          cur = mfma_fp8(a8, b8, f32x4{0.f, 0.f, 0.f, 0.f});
          if (j == NJ - 1) read_a(next, i, A);
        }
        if (t > 0) {
          const int i = (t - 1) / NJ, j = (t - 1) % NJ;
          const float s = sc[(GATEUP && i >= 4) ? 1 : 0][j];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(prev[r], s, acc[i][j][r]);
        }
        prev = cur;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8, A.al[i]), __builtin_bit_cast(bf16x8, F.bl[j]), acc[i][j]);
          acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8, A.ah[i]), __builtin_bit_cast(bf16x8, F.bh[j]), acc[i][j]);
        }
        read_a(next, i, A);
      }
    }
  }

  // The item's weight-block scales, staged once in LDS (wsc[0][kb], wsc[1][kb]):
  // gate/up: the gate block and the up block of the tile; down: the block of
  // each weight half.  Loaded before the copy ring starts, so the only vector
  // memory operations inside the K loop are the counted direct-to-LDS copies.
  __device__ __forceinline__ void load_wscales(float *wsc) const {
    if constexpr (FP8) {
      const float *s0, *s1;
      if (GATEUP) {
        s0 = G.sgu + ((int64_t)e * (2 * I / 128) + col0 / 128) * KB;
        s1 = G.sgu + ((int64_t)e * (2 * I / 128) + (I + col0) / 128) * KB;
      } else {
        s0 = G.sd + ((int64_t)e * (H / 128) + col0 / 128) * KB;
        s1 = G.sd + ((int64_t)e * (H / 128) + (col0 + 128) / 128) * KB;
      }
      for (int i = threadIdx.x; i < 2 * KB; i += TTHREADS) wsc[i] = i < KB ? s0[i] : s1[i - KB];
    }
  }

  // One pipeline step: chunk kc's operands are already in Fcur.  Wait until
  // chunk kc+1 has landed in LDS (chunk kc+2 may still be in flight) and this
  // wave's reads of chunk kc have completed, sync the workgroup (chunk kc's
  // buffer is then free and is refilled with chunk kc+3), read chunk kc+1 into
  // Fnext, and run chunk kc's MFMAs while those reads are in flight.
  template <int NJ>
  __device__ __forceinline__ void step(int kc, uint8_t *lds, const float *wsc, AFrags &A, BFrags<NJ> &Fcur,
                                       BFrags<NJ> &Fnext, f32x4 (&acc)[8][4]) const {
    constexpr int PS = FP8 ? 13 : 12;    // vector memory instructions per wave per stage
    if (kc + 2 < nchunk)
      wait_vm_lgkm0<PS>();
    else
      wait_vm_lgkm0<0>();
    wg_barrier();
    if (kc + 3 < nchunk) issue(kc + 3, lds + ((kc + 3) % NSTAGE) * TSTAGE);
    // The last step reads its own buffer again (nothing is copied into it any
    // more), which keeps the refills unconditional.
    const int kn = kc + 1 < nchunk ? kc + 1 : kc;
    const uint8_t *next = lds + (kn % NSTAGE) * TSTAGE;
    read_b<NJ>(next, wsc, kn, Fnext);
    mma<NJ>(A, Fcur, next, acc);
  }

  template <int NJ>
  __device__ __forceinline__ void mainloop(uint8_t *lds, const float *wsc, f32x4 (&acc)[8][4]) const {
    constexpr int PS = FP8 ? 13 : 12;
    issue(0, lds);
    if (nchunk > 1) issue(1, lds + TSTAGE);
    if (nchunk > 2) issue(2, lds + 2 * TSTAGE);
    if (nchunk > 2)
      wait_vm<2 * PS>();
    else if (nchunk > 1)
      wait_vm<PS>();
    else
      wait_vm<0>();
    wg_barrier();
    AFrags A;
    BFrags<NJ> F0, F1;
#pragma unroll
    for (int i = 0; i < 8; ++i) read_a(lds, i, A);
    read_b<NJ>(lds, wsc, 0, F0);
    for (int kc = 0; kc < nchunk; kc += 2) {
      step<NJ>(kc, lds, wsc, A, F0, F1, acc);
      if (kc + 1 < nchunk) step<NJ>(kc + 1, lds, wsc, A, F1, F0, acc);
    }
  }
};

// Epilogue of a work item: lane holds rows 4*(lane/16)+r of weight tile i for
// token slice j (token row rbeg + brow[j] + lane%16).  gate/up: SwiGLU, then h
// as bf16 (and the pre-activations when asked) or as e4m3 with one scale per
// token per 128 columns (amax over the two weight-half waves through `red`,
// 2 x BM floats); down: the output rows.
template <bool FP8, bool GATEUP, int BM>
__device__ __forceinline__ void store_item(const FfnGroup &G, const f32x4 (&acc)[8][4], const int (&brow)[4],
                                           int lane, int wn, int rbeg, int nvalid, int I, int col0, int ntile,
                                           int H, float *red) {
  if constexpr (GATEUP) {
    float hv[4][4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[i][j][r] = swiglu(acc[i][j][r], acc[i + 4][j][r]);
    if constexpr (!FP8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tr = brow[j] + (lane & 15);
        if (tr >= nvalid) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = col0 + 64 * wn + 16 * i + 4 * (lane >> 4);
          const uint32_t lo = pack_bf16x2(hv[i][j][0], hv[i][j][1]);
          const uint32_t hi = pack_bf16x2(hv[i][j][2], hv[i][j][3]);
          *reinterpret_cast<uint2 *>(G.h + ((int64_t)(rbeg + tr) * I + col) * 2) = make_uint2(lo, hi);
          if (G.z) {   // pre-activations kept for a backward
            float *zr = G.z + (int64_t)(rbeg + tr) * 2 * I + col;
            *reinterpret_cast<f32x4 *>(zr) = acc[i][j];
            *reinterpret_cast<f32x4 *>(zr + I) = acc[i + 4][j];
          }
        }
      }
    } else {
      // amax over the tile's 128 h columns per token: lane (16 values), the 4
      // lanes of the token (xor 16, 32), then the two weight-half waves (LDS).
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) am = __builtin_fmaxf(am, __builtin_fabsf(hv[i][j][r]));
        am = __builtin_fmaxf(am, __shfl_xor(am, 16, kWave));
        am = __builtin_fmaxf(am, __shfl_xor(am, 32, kWave));
        if (lane < 16) red[wn * BM + brow[j] + lane] = am;
      }
      // LDS-only barrier: a __syncthreads would also wait for the next work
      // item's copies, which are in flight during this epilogue
      wait_lgkm0();
      wg_barrier();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tr = brow[j] + (lane & 15);
        const float s = group_scale(__builtin_fmaxf(red[tr], red[BM + tr]));
        if (tr >= nvalid) continue;
        const int64_t row = rbeg + tr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = col0 + 64 * wn + 16 * i + 4 * (lane >> 4);
          *reinterpret_cast<uint32_t *>(G.h + row * I + col) =
              quant4_e4m3(hv[i][j][0], hv[i][j][1], hv[i][j][2], hv[i][j][3], s);
        }
        if (wn == 0 && lane < 16) G.hs[row * (I / 128) + ntile] = s;
      }
    }
  } else if (G.y_f32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tr = brow[j] + (lane & 15);
      if (tr >= nvalid) continue;
      const int64_t row = rbeg + tr;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int col = col0 + 128 * wn + 16 * i + 4 * (lane >> 4);
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(G.y) + row * H + col) = acc[i][j];
      }
    }
  } else {
    // bf16 rows, 16 bytes per lane: lane (t, q = lane / 16) holds columns
    // 16 i + 4 q .. +3 of tiles i and i+1 (i even); lanes q and q ^ 1 swap
    // halves so that an even q ends up with columns 16 i + 4 q .. +7 of tile i
    // and an odd q with 16 (i+1) + 4 (q-1) .. +7 of tile i+1.
    const int q = lane >> 4;
    const bool even = (q & 1) == 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tr = brow[j] + (lane & 15);
      const int64_t row = rbeg + tr;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const uint32_t a0 = pack_bf16x2(acc[i][j][0], acc[i][j][1]), a1 = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        const uint32_t b0 = pack_bf16x2(acc[i + 1][j][0], acc[i + 1][j][1]),
                       b1 = pack_bf16x2(acc[i + 1][j][2], acc[i + 1][j][3]);
        // every lane takes part in the swap, stored or not
        const uint32_t r0 = (uint32_t)__shfl_xor((int)(even ? b0 : a0), 16, kWave);
        const uint32_t r1 = (uint32_t)__shfl_xor((int)(even ? b1 : a1), 16, kWave);
        if (tr < nvalid) {
          const int col = col0 + 128 * wn + (even ? 16 * i + 4 * q : 16 * (i + 1) + 4 * (q - 1));
          const i32x4 v = even ? i32x4{(int)a0, (int)a1, (int)r0, (int)r1} : i32x4{(int)r0, (int)r1, (int)b0, (int)b1};
          store16(reinterpret_cast<uint16_t *>(G.y) + row * H + col, v);
        }
      }
    }
  }
}

template <bool FP8, bool GATEUP, bool T16>
__device__ __forceinline__ void tiled_item(const FfnGroup &G, const TileEntry &te, int ntile, int H, uint8_t *lds,
                                           float *red, float *wsc) {
  TiledItem<FP8, GATEUP, T16> it(G, te, ntile, H);
  it.load_wscales(wsc);
  __syncthreads();
  const int lane = it.lane, wn = it.wn, wm = it.wm;
  // active 16-row token slices of this wave: slice j covers rows 16*(wm + 2j)
  const int nact = uniform(it.nvalid <= 16 * wm ? 0 : min(4, (it.nvalid - 16 * wm + 31) / 32));
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  switch (nact) {
    case 4: it.template mainloop<4>(lds, wsc, acc); break;
    case 3: it.template mainloop<3>(lds, wsc, acc); break;
    case 2: it.template mainloop<2>(lds, wsc, acc); break;
    case 1: it.template mainloop<1>(lds, wsc, acc); break;
    default: it.template mainloop<1>(lds, wsc, acc); break;   // keeps the barrier count equal across waves
  }
  const int rbeg = it.rbeg, nvalid = it.nvalid, I = it.I, col0 = it.col0;
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) brow[j] = 16 * (wm + 2 * j);

  store_item<FP8, GATEUP, TBM>(G, acc, brow, lane, wn, rbeg, nvalid, I, col0, ntile, H, red);
  __syncthreads();   // the next work item reuses the LDS ring and the reduction area
}

// ------------------------------------------------------------ wide tiles
//
// For experts with many rows (mean >= 128 per expert, 96 with fp8 weights, 48
// with MX FP4 in the MX variant below): a work item is 256
// weight rows x 256 token rows and a workgroup is 8 waves, two per SIMD.  A
// weight tile fetched once then feeds every row of most experts (instead of
// being fetched again for each 128-row token tile), and a K chunk moves 64 KB
// into LDS for twice the MFMAs of the 128-row item.  The LDS ring has two
// stages (65 KB each): chunk kc+1 is copied while chunk kc is consumed.  A
// wave owns 128 weight rows (wn) x 4 interleaved 16-row token slices
// 16 (wm + 4 j); it reads its chunk's token fragments once and streams the 8
// weight tiles' fragments through a double buffer, which keeps it within the
// 256 registers a wave has at two waves per SIMD.

namespace {
constexpr int WBM = 256;                    // token rows per wide tile
constexpr int WTHREADS = 512;
constexpr int WTX = WBM * 128;              // token bytes per stage
constexpr int WTSX = 4 * WBM;               // token scales per stage (4 bytes per token row)
constexpr int WSTAGE = TW + WTX + WTSX;
constexpr int WNSTAGE = 2;
}  // namespace

template <bool FP8, bool GATEUP, bool T16>
struct WideItem {
  const FfnGroup &G;
  int e, rbeg, rend, nvalid, I, K, KB, nchunk, col0, ntile, H;
  int64_t wrows;   // rows of the expert's weight matrix (2I or H)
  int64_t rowb;
  const uint8_t *wsrc, *asrc;
  const float *ascale;
  __amdgpu_buffer_rsrc_t rw, rx, rsx;   // copy sources: weights, token rows, token scales
  int lane, w, wn, wm;
  uint32_t woff[4], xoff[4], xoff2[4], soff;   // per-lane byte offsets of this lane's copies
  // LDS read offsets inside a stage: token slice 0's two 16-byte fragment
  // halves and its scale (slice j adds 8192 j / 512 j: its rows are
  // 16 (wm + 4 j) + lane % 16, whose swizzle lane % 8 does not depend on j),
  // and the weight fragment of tile 0 (tile16 copies).
  uint32_t rb_l, rb_h, rb_s, ra;

  __device__ WideItem(const FfnGroup &g, const TileEntry &te, int nt_, int H_) : G(g), ntile(nt_), H(H_) {
    lane = threadIdx.x & 63;
    w = uniform(threadIdx.x >> 6);
    wn = w & 1;
    wm = w >> 1;
    e = te.ge & 0xFFFFFF;
    rend = min(max(group_off(G, e + 1), 0), G.nrows);
    rbeg = min(max(group_off(G, e), 0) + te.m0, rend);
    nvalid = min(rend - rbeg, WBM);
    I = G.I;
    K = GATEUP ? H : I;
    rowb = (int64_t)K * (FP8 ? 1 : 2);
    nchunk = (int)(rowb / 128);
    KB = K / 128;
    col0 = GATEUP ? ntile * 128 : ntile * TBN;
    wsrc = GATEUP ? G.wgu + (int64_t)e * 2 * I * rowb : G.wd + (int64_t)e * H * rowb;
    wrows = GATEUP ? 2 * (int64_t)I : (int64_t)H;
    const bool indirect = GATEUP && G.xsrc != nullptr;
    asrc = (GATEUP ? G.x : G.h) + (indirect ? 0 : (int64_t)rbeg * rowb);
    ascale = (GATEUP ? G.xs : G.hs) + (FP8 && !indirect ? (int64_t)rbeg * KB : 0);
    const int sub = lane >> 3;   // row within an 8-row group
    // Copy instruction q = w + 8t covers rows 8q .. 8q+7 of the weight and of
    // the token tile (1 KB each); waves 0-3 issue q and q + 4 (rows 32 further
    // on: the same swizzle, weight offsets 32 rows further, token rows looked
    // up again), and the token scales of rows 64w .. 64w+63.
    if (w < 4) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 8 * (w + 8 * t) + sub;
        const int c = (lane & 7) ^ swz_f(r);   // logical 16-byte column landing in this lane's slot
        const int grow = GATEUP ? (r < 128 ? col0 + r : I + col0 + r - 128) : col0 + r;
        if constexpr (T16) {
          // tile16 weights: instruction j = w + 8t copies half j % 2 of the
          // item's 16-row tile j / 2 verbatim (LDS keeps the fragment-major tile)
          const int j = w + 8 * t, rt = 16 * (j >> 1);
          const int g0 = GATEUP ? (rt < 128 ? col0 + rt : I + col0 + rt - 128) : col0 + rt;
          woff[t] = (uint32_t)(((int64_t)g0 >> 4) * 2048 + 1024 * (j & 1) + 16 * lane);
        } else {
          woff[t] = (uint32_t)(grow * rowb + c * 16);
        }
      }
      // rows past the end repeat a valid row; indirect rows come from x row xsrc[row] / xdiv
      auto xrow = [&](int r) -> int64_t {
        const int rr = min(r, nvalid - 1);
        return indirect ? G.xsrc[rbeg + rr] / G.xdiv : rr;
      };
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 8 * (w + 8 * t) + sub, r2 = r + 32;
        xoff[t] = (uint32_t)(xrow(r) * rowb + ((lane & 7) ^ swz_f(r)) * 16);
        xoff2[t] = (uint32_t)(xrow(r2) * rowb + ((lane & 7) ^ swz_f(r2)) * 16);
      }
      soff = (uint32_t)(xrow(64 * w + lane) * KB * 4);
    }
    // buffer sizes: the expert's weight matrix, the item's token rows and
    // scales (indirect rows: any row of x, whose offsets stay below 2^31)
    {
      const uint32_t kAny = 0x7FFFFFFF;
      rw = buf_rsrc(wsrc, (uint32_t)(wrows * rowb));
      rx = buf_rsrc(asrc, indirect ? kAny : (uint32_t)(nvalid * rowb));
      rsx = buf_rsrc(ascale, indirect ? kAny : (uint32_t)(nvalid * KB * 4));
    }
    {
      const int r0 = 16 * wm + (lane & 15), ck = 2 * (lane >> 4);
      rb_l = (uint32_t)(TW + swz(r0, ck));
      rb_h = (uint32_t)(TW + swz(r0, ck + 1));
      rb_s = (uint32_t)(TW + WTX + 4 * r0);
      ra = (uint32_t)(128 * (arow(0) - (lane & 15)) + 16 * lane);
    }
  }

  // Direct-to-LDS copies of K chunk kc into stage buffer sb.  Waves 0-3 issue
  // every copy: their own (instruction q = w + 8t) and those of the wave that
  // shares their SIMD (q + 4, rows 32 further on), 8 (weights) + up to 8
  // (tokens) [+ 1 (token scales, fp8)] instructions; waves 4-7 issue none and
  // go straight to their MFMAs, so that while one wave of a SIMD waits for the
  // copy path to take its instructions the other keeps the matrix core busy.
  // A token copy whose 8 rows all lie past the item's last row is skipped: the
  // stale LDS rows it leaves only feed MFMA output columns of padding rows,
  // which are never stored (an output column depends on its own token only).
  // The waits count nothing but "all of this wave's copies".
  __device__ __forceinline__ void issue(int kc, uint8_t *sb) const {
    if (w >= 4) return;
    const uint32_t wk = (uint32_t)kc * (T16 ? 128 * (uint32_t)wrows : 128);
    const uint32_t w2 = wk + (T16 ? 4096u : 32u * (uint32_t)rowb);   // the partner's weight rows, 32 further on
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bdma16(rw, woff[t], wk, sb + (w + 8 * t) * 1024);
      bdma16(rw, woff[t], w2, sb + (w + 4 + 8 * t) * 1024);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (8 * (w + 8 * t) < nvalid) bdma16(rx, xoff[t], 128 * kc, sb + TW + (w + 8 * t) * 1024);
      if (8 * (w + 4 + 8 * t) < nvalid) bdma16(rx, xoff2[t], 128 * kc, sb + TW + (w + 4 + 8 * t) * 1024);
    }
    if constexpr (FP8) bdma4(rsx, soff, 4 * kc, sb + TW + WTX + 256 * w);
  }

  struct AFrag {
    i32x4 l, h;
  };
  template <int NJ>
  struct BFrags {
    i32x4 bl[NJ], bh[NJ];
    float sx[NJ];
    float sa, sb;
  };

  __device__ __forceinline__ int arow(int i) const {
    return (GATEUP ? (i < 4 ? 64 * wn + 16 * i : 128 + 64 * wn + 16 * (i - 4)) : 128 * wn + 16 * i) + (lane & 15);
  }

  __device__ __forceinline__ void read_a(const uint8_t *sb, int i, AFrag &A) const {
    if constexpr (T16) {   // fragment-major tile (arow(i) - lane % 16) / 16: lane l at 16 l and 1024 + 16 l
      const uint8_t *t = sb + 128 * (arow(i) - (lane & 15)) + 16 * lane;
      A.l = *reinterpret_cast<const i32x4 *>(t);
      A.h = *reinterpret_cast<const i32x4 *>(t + 1024);
    } else {
      const int ck = 2 * (lane >> 4);
      A.l = *reinterpret_cast<const i32x4 *>(sb + swz(arow(i), ck));
      A.h = *reinterpret_cast<const i32x4 *>(sb + swz(arow(i), ck + 1));
    }
  }

  template <int NJ>
  __device__ __forceinline__ void read_b(const uint8_t *sb, const float *wsc, int kc, BFrags<NJ> &F) const {
    const int ck = 2 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = 16 * (wm + 4 * j) + (lane & 15);
      F.bl[j] = *reinterpret_cast<const i32x4 *>(sb + TW + swz(r, ck));
      F.bh[j] = *reinterpret_cast<const i32x4 *>(sb + TW + swz(r, ck + 1));
      // token r's scale sits in wave (r / 32)'s slot, lane r % 32
      if constexpr (FP8) F.sx[j] = *reinterpret_cast<const float *>(sb + TW + WTX + 4 * r);
    }
    if constexpr (FP8) {
      F.sa = GATEUP ? wsc[kc] : wsc[wn * KB + kc];
      F.sb = GATEUP ? wsc[KB + kc] : F.sa;
    }
  }

  // The MFMAs of one K chunk from stage buffer sb: token fragments read once,
  // weight tile i+1's fragments read while tile i's MFMAs run.
  // Weight tile i's fragment (tile16 copies: the tile's two kilobytes at
  // 2048 (arow(i) - lane % 16) / 16 = ra + tile offset).
  __device__ __forceinline__ void read_a16(const uint8_t *sb, int i, AFrag &A) const {
    const int dt = GATEUP ? (i < 4 ? 16 * i : 128 + 16 * (i - 4)) : 16 * i;   // arow(i) - arow(0)
    const uint8_t *t = sb + ra + 128 * dt;
    A.l = *reinterpret_cast<const i32x4 *>(t);
    A.h = *reinterpret_cast<const i32x4 *>(t + 1024);
  }

  // fp8 chunk with tile16 weights.  The first MFMA's operands (weight tile 0,
  // token slice 0, their scales) are read before the other slices, so a wave
  // starts as soon as they land; each block product is folded into its
  // accumulators two MFMAs later, when it is ready (no hazard stalls).
  template <int NJ>
  __device__ __forceinline__ void chunk_fp8_t16(const uint8_t *sb, const float *wsc, int kc,
                                                f32x4 (&acc)[8][4]) const {
    i32x4 bl[NJ], bh[NJ];
    float sx[NJ];
    AFrag A[2];
    read_a16(sb, 0, A[0]);
    bl[0] = *reinterpret_cast<const i32x4 *>(sb + rb_l);
    bh[0] = *reinterpret_cast<const i32x4 *>(sb + rb_h);
    sx[0] = *reinterpret_cast<const float *>(sb + rb_s);
    const float sa = GATEUP ? wsc[kc] : wsc[wn * KB + kc];
    const float sbw = GATEUP ? wsc[KB + kc] : sa;
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NT = 8 * NJ;
    f32x4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT + 2; ++t) {
      f32x4 cur = {0.f, 0.f, 0.f, 0.f};
      if (t < NT) {
        const int i = t / NJ, j = t % NJ;
        const AFrag &a = A[i & 1];
        const i32x8 a8 = {a.l[0], a.l[1], a.l[2], a.l[3], a.h[0], a.h[1], a.h[2], a.h[3]};
        const i32x8 b8 = {bl[j][0], bl[j][1], bl[j][2], bl[j][3], bh[j][0], bh[j][1], bh[j][2], bh[j][3]};
        cur = mfma_fp8(a8, b8, f32x4{0.f, 0.f, 0.f, 0.f});
        if (t == 0) {   // the other token slices, while the first MFMA runs
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int jj = 1; jj < NJ; ++jj) {
            bl[jj] = *reinterpret_cast<const i32x4 *>(sb + rb_l + 8192 * jj);
            bh[jj] = *reinterpret_cast<const i32x4 *>(sb + rb_h + 8192 * jj);
            sx[jj] = *reinterpret_cast<const float *>(sb + rb_s + 256 * jj);
          }
        }
        if (j == 0 && i + 1 < 8) read_a16(sb, i + 1, A[(i + 1) & 1]);
      }
      if (t >= 2) {
        const int i = (t - 2) / NJ, j = (t - 2) % NJ;
        const float sc = ((GATEUP && i >= 4) ? sbw : sa) * sx[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p2[r], sc, acc[i][j][r]);
      }
      p2 = p1;
      p1 = cur;
      // keep this order: the scheduler would otherwise hoist every scale
      // product to the top and wait there for all fragment reads
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  template <int NJ>
  __device__ __forceinline__ void chunk(const uint8_t *sb, const float *wsc, int kc, f32x4 (&acc)[8][4]) const {
    if constexpr (FP8 && T16) {
      chunk_fp8_t16<NJ>(sb, wsc, kc, acc);
      return;
    }
    BFrags<NJ> F;
    read_b<NJ>(sb, wsc, kc, F);
    AFrag A[2];
    read_a(sb, 0, A[0]);
    if constexpr (FP8) {
      // raw block products are folded into the accumulators one MFMA behind
      float sc[2][NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        sc[0][j] = F.sa * F.sx[j];
        sc[1][j] = F.sb * F.sx[j];
      }
      constexpr int NT = 8 * NJ;
      f32x4 prev = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t <= NT; ++t) {
        f32x4 cur = {0.f, 0.f, 0.f, 0.f};
        if (t < NT) {
          const int i = t / NJ, j = t % NJ;
          if (j == 0 && i + 1 < 8) read_a(sb, i + 1, A[(i + 1) & 1]);
          const AFrag &a = A[i & 1];
          const i32x8 a8 = {a.l[0], a.l[1], a.l[2], a.l[3], a.h[0], a.h[1], a.h[2], a.h[3]};
          const i32x8 b8 = {F.bl[j][0], F.bl[j][1], F.bl[j][2], F.bl[j][3],
                            F.bh[j][0], F.bh[j][1], F.bh[j][2], F.bh[j][3]};
          cur = mfma_fp8(a8, b8, f32x4{0.f, 0.f, 0.f, 0.f});
        }
        if (t > 0) {
          const int i = (t - 1) / NJ, j = (t - 1) % NJ;
          const float s = sc[(GATEUP && i >= 4) ? 1 : 0][j];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(prev[r], s, acc[i][j][r]);
        }
        prev = cur;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i + 1 < 8) read_a(sb, i + 1, A[(i + 1) & 1]);
        const AFrag &a = A[i & 1];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8, a.l), __builtin_bit_cast(bf16x8, F.bl[j]), acc[i][j]);
          acc[i][j] = mfma_bf16(__builtin_bit_cast(bf16x8, a.h), __builtin_bit_cast(bf16x8, F.bh[j]), acc[i][j]);
        }
      }
    }
  }

  // The item's weight-block scales, staged in LDS before the copy ring starts.
  __device__ __forceinline__ void load_wscales(float *wsc) const {
    if constexpr (FP8) {
      const float *s0, *s1;
      if (GATEUP) {
        s0 = G.sgu + ((int64_t)e * (2 * I / 128) + col0 / 128) * KB;
        s1 = G.sgu + ((int64_t)e * (2 * I / 128) + (I + col0) / 128) * KB;
      } else {
        s0 = G.sd + ((int64_t)e * (H / 128) + col0 / 128) * KB;
        s1 = G.sd + ((int64_t)e * (H / 128) + (col0 + 128) / 128) * KB;
      }
      for (int i = threadIdx.x; i < 2 * KB; i += WTHREADS) wsc[i] = i < KB ? s0[i] : s1[i - KB];
    }
  }

  // Step kc: wait for this wave's copies of chunk kc, sync the workgroup
  // (every wave's copies have landed, and nobody reads chunk kc-1's buffer any
  // more), refill that buffer with chunk kc+1, consume chunk kc.  Chunk 0 was
  // issued into stage `par` before the call (by the previous work item, or
  // before the first); chunk kc sits in stage (par + kc) % 2.
  template <int NJ>
  __device__ __forceinline__ void mainloop(uint8_t *lds, int par, const float *wsc, f32x4 (&acc)[8][4]) const {
    for (int kc = 0; kc < nchunk; ++kc) {
      wait_vm_lgkm0<0>();
      wg_barrier();
      if (kc + 1 < nchunk) issue(kc + 1, lds + ((par + kc + 1) & 1) * WSTAGE);
      chunk<NJ>(lds + ((par + kc) & 1) * WSTAGE, wsc, kc, acc);
    }
  }
};

// A resolved work item of the wide kernel.
struct WideWork {
  TileEntry te;
  int ntile;
  int valid;
};

// Start work item w: stage its weight-block scales in wscb and issue its
// chunk 0 into stage buffer sb.
template <bool FP8, bool GATEUP, bool T16>
__device__ __forceinline__ void wide_begin_t(const FfnGroup &G, const WideWork &w, int H, uint8_t *sb, float *wscb) {
  WideItem<FP8, GATEUP, T16> it(G, w.te, w.ntile, H);
  it.load_wscales(wscb);
  it.issue(0, sb);
}
template <bool GATEUP>
__device__ __forceinline__ void wide_begin(const TiledArgs &a, const WideWork &w, uint8_t *sb, float *wscb) {
  const FfnGroup &G = (w.te.ge >> 24) ? a.g1 : a.g0;
  if (G.fp8) {
    if (G.tile16)
      wide_begin_t<true, GATEUP, true>(G, w, a.H, sb, wscb);
    else
      wide_begin_t<true, GATEUP, false>(G, w, a.H, sb, wscb);
  } else if (G.tile16) {
    wide_begin_t<false, GATEUP, true>(G, w, a.H, sb, wscb);
  } else {
    wide_begin_t<false, GATEUP, false>(G, w, a.H, sb, wscb);
  }
}

// One work item whose chunk 0 (stage par) and weight scales (wscb[0]) were
// issued beforehand.  After its last chunk's MFMAs it starts the next item
// (chunk 0 into the other stage... the stage its chunk nchunk-2 used, which
// every wave is done with; scales into wscb[1]), so that those copies are in
// flight during this item's epilogue.  Returns the next item's chunk-0 stage.
template <bool FP8, bool GATEUP, bool T16>
__device__ __forceinline__ int wide_item(const TiledArgs &a, const FfnGroup &G, const WideWork &cur,
                                         const WideWork &next, int par, uint8_t *lds, float *red, float *const wscb[2]) {
  WideItem<FP8, GATEUP, T16> it(G, cur.te, cur.ntile, a.H);
  const int lane = it.lane, wn = it.wn, wm = it.wm;
  // active 16-row token slices of this wave: slice j covers rows 16*(wm + 4j)
  const int nact = uniform(it.nvalid <= 16 * wm ? 0 : min(4, (it.nvalid - 16 * wm + 63) / 64));
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  switch (nact) {
    case 4: it.template mainloop<4>(lds, par, wscb[0], acc); break;
    case 3: it.template mainloop<3>(lds, par, wscb[0], acc); break;
    case 2: it.template mainloop<2>(lds, par, wscb[0], acc); break;
    case 1: it.template mainloop<1>(lds, par, wscb[0], acc); break;
    default: it.template mainloop<1>(lds, par, wscb[0], acc); break;   // keeps the barrier count equal across waves
  }
  const int npar = (par + it.nchunk) & 1;
  if (next.valid) wide_begin<GATEUP>(a, next, lds + npar * WSTAGE, wscb[1]);
  const int rbeg = it.rbeg, nvalid = it.nvalid, I = it.I, col0 = it.col0;
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) brow[j] = 16 * (wm + 4 * j);

  store_item<FP8, GATEUP, WBM>(G, acc, brow, lane, wn, rbeg, nvalid, I, col0, cur.ntile,
                               a.H, red);
  // the next item's first step waits for its copies and syncs the workgroup
  // before anything reads LDS; the reduction area is free once every wave is
  // past this barrier (LDS only: the copies in flight are not waited for)
  wait_lgkm0();
  wg_barrier();
  return npar;
}

// Work item L -> (tile-list slot, column tile).  The slots of one expert are
// taken in bands of up to TBAND token tiles, and the items of a band are
// ordered column-tile-major: the 32 workgroups of an XCD that start
// consecutive items share about four weight tiles and eight token tiles,
// instead of one token tile's twelve weight tiles.
template <int BM>
__device__ __forceinline__ void map_item(const TiledArgs &a, int L, int &slot, int &ntile) {
  const int s = L / a.nt;
  const TileEntry te = a.tiles[s];
  const FfnGroup &G = (te.ge >> 24) ? a.g1 : a.g0;
  const int e = te.ge & 0xFFFFFF;
  const int r0 = min(max(group_off(G, e), 0), G.nrows);
  const int r1 = min(max(group_off(G, e + 1), r0), G.nrows);
  const int t = te.m0 / BM, p = t % TBAND;
  const int band = min(TBAND, (r1 - r0 + BM - 1) / BM - (t - p));
  const int s0 = s - p, q = L - a.nt * s0;
  slot = s0 + q % max(band, 1);
  ntile = q / max(band, 1);
}

// First item of XCD range x: the ranges split the summed K-chunk cost of the
// items evenly (a bf16 item of the shared expert streams twice the bytes of
// an fp8 item), group 0's items first.
__device__ __forceinline__ int range_start(int x, int64_t n0, int count, int c0, int c1) {
  const int64_t total = n0 * c0 + (int64_t)(count - n0) * c1;
  const int64_t C = total * x / 8;
  const int64_t idx = C <= n0 * c0 ? (C + c0 - 1) / c0 : n0 + (C - n0 * c0 + c1 - 1) / c1;
  return (int)min<int64_t>(idx, count);
}

template <bool GATEUP>
__global__ __launch_bounds__(TTHREADS, 1) void tiled_ffn_kernel(TiledArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float *red = reinterpret_cast<float *>(lds + NSTAGE * TSTAGE);
  float *wsc = red + 2 * TBM;
  const int nslots = a.hdr[0];
  const int count = nslots * a.nt;
  const int64_t n0 = (int64_t)min(a.hdr[1], nslots) * a.nt;
  const int xcd = blockIdx.x & 7, per = gridDim.x >> 3, slot0 = blockIdx.x >> 3;
  const int beg = range_start(xcd, n0, count, a.c0, a.c1), end = range_start(xcd + 1, n0, count, a.c0, a.c1);
  for (int L = beg + slot0; L < end; L += per) {
    int slot, ntile;
    map_item<TBM>(a, L, slot, ntile);
    if (slot < nslots) {
      const TileEntry te = a.tiles[slot];
      const FfnGroup G = (te.ge >> 24) ? a.g1 : a.g0;
      if (!(GATEUP && ntile * 128 >= G.I)) {
        if (G.fp8) {
          if (G.tile16)
            tiled_item<true, GATEUP, true>(G, te, ntile, a.H, lds, red, wsc);
          else
            tiled_item<true, GATEUP, false>(G, te, ntile, a.H, lds, red, wsc);
        } else if (G.tile16) {
          tiled_item<false, GATEUP, true>(G, te, ntile, a.H, lds, red, wsc);
        } else {
          tiled_item<false, GATEUP, false>(G, te, ntile, a.H, lds, red, wsc);
        }
      }
    }
  }
}

// The first work item at or after L (stepping by `per`) that exists: a
// tile-list slot that is filled and, for gate/up, a column tile inside its
// group's width.  L is advanced to it (end: none).
template <bool GATEUP>
__device__ __forceinline__ WideWork wide_find(const TiledArgs &a, int &L, int end, int per, int nslots) {
  WideWork w{{0, 0}, 0, 0};
  for (; L < end; L += per) {
    int slot, ntile;
    map_item<WBM>(a, L, slot, ntile);
    if (slot >= nslots) continue;
    const TileEntry te = a.tiles[slot];
    const FfnGroup &G = (te.ge >> 24) ? a.g1 : a.g0;
    if (GATEUP && ntile * 128 >= G.I) continue;
    w.te = te;
    w.ntile = ntile;
    w.valid = 1;
    break;
  }
  return w;
}

template <bool GATEUP>
__global__ __launch_bounds__(WTHREADS, 1) void wide_ffn_kernel(TiledArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float *red = reinterpret_cast<float *>(lds + WNSTAGE * WSTAGE);
  float *wscs = red + 2 * WBM;   // two weight-scale buffers (current item, next item), 256 floats each
  const int nslots = a.hdr[0];
  const int count = nslots * a.nt;
  const int64_t n0 = (int64_t)min(a.hdr[1], nslots) * a.nt;
  const int xcd = blockIdx.x & 7, per = gridDim.x >> 3, slot0 = blockIdx.x >> 3;
  const int beg = range_start(xcd, n0, count, a.c0, a.c1), end = range_start(xcd + 1, n0, count, a.c0, a.c1);
  int L = beg + slot0;
  WideWork cur = wide_find<GATEUP>(a, L, end, per, nslots);
  if (!cur.valid) return;
  int par = 0, wb = 0;
  wide_begin<GATEUP>(a, cur, lds, wscs);
  while (cur.valid) {
    L += per;
    const WideWork next = wide_find<GATEUP>(a, L, end, per, nslots);
    float *const wscb[2] = {wscs + 256 * wb, wscs + 256 * (wb ^ 1)};
    const FfnGroup &G = (cur.te.ge >> 24) ? a.g1 : a.g0;
    if (G.fp8) {
      if (G.tile16)
        par = wide_item<true, GATEUP, true>(a, G, cur, next, par, lds, red, wscb);
      else
        par = wide_item<true, GATEUP, false>(a, G, cur, next, par, lds, red, wscb);
    } else if (G.tile16) {
      par = wide_item<false, GATEUP, true>(a, G, cur, next, par, lds, red, wscb);
    } else {
      par = wide_item<false, GATEUP, false>(a, G, cur, next, par, lds, red, wscb);
    }
    wb ^= 1;
    cur = next;
  }
}

// ------------------------------------------------------ wide tiles, MX FP4
//
// The wide item for MX FP4 weights (E2M1 codes two to a byte, one E8M0 scale
// per 32 inputs of a row; e4m3 tokens with fp32 1x128 group scales): the same
// 256 weight rows x 256 token rows, 8 waves and wave layout as the fp8/bf16
// wide item, and the same epilogue.  A K chunk of 128 inputs is 64 bytes of
// codes per weight row, so a stage is 16 KB of codes + 32 KB of token rows
// + 1 KB of token scales + 1 KB of E8M0 words (50 KB) and the ring holds
// three stages: chunks kc+1 and kc+2 are in flight while chunk kc is consumed.
//   - codes: instruction t of wave w copies the item's 16-row tile w + 8t with
//     lane l taking row l%16, bytes 16(l/16)..+15 of the chunk, so that a tile
//     lands fragment-major and each lane later reads its A operand at 16 l;
//   - token rows as in the wide item (8 rows x 128 bytes per instruction,
//     XOR-swizzled 16-byte columns); the B operand takes columns l/16 and
//     4 + l/16 of the row (the instruction's input order);
//   - one scale word per token row (waves 0-3) and per weight row (waves 4-7);
//     a lane's E8M0 byte (its row, 32-input block l/16) is the scaled MFMA's A
//     scale, the token scale multiplies the block product, which is folded into
//     the accumulators two MFMAs later.
// The next item's chunks 0 and 1 are issued right after an item's last step
// (the two stages its chunks nchunk-3 and nchunk-2 used), so the ring keeps
// running across items; the shared expert's bf16 items, when they ride in the
// launch, run the bf16 wide item on the first two 65 KB of the same LDS.

namespace {
constexpr int MXC = TBN * 64;             // code bytes per stage
constexpr int MXTOK = MXC;                // token rows (WTX bytes)
constexpr int MXTS = MXTOK + WTX;         // token scale words, 4 bytes per token row
constexpr int MXWS = MXTS + 4 * WBM;      // E8M0 words, 4 bytes per weight row
constexpr int MXSTAGE = MXWS + 4 * TBN;
constexpr int MXNSTAGE = 3;
static_assert(MXNSTAGE * MXSTAGE >= WNSTAGE * WSTAGE, "the bf16 items' ring must fit in the MX ring");
}  // namespace

template <bool GATEUP>
struct WideMxItem {
  const FfnGroup &G;
  int e, rbeg, rend, nvalid, I, K, nchunk, col0, ntile, H, nissue;
  const uint8_t *wsrc, *ssrc, *asrc;
  const float *ascale;
  __amdgpu_buffer_rsrc_t rw, rx, rsc;   // copy sources: codes, token rows, this wave's scale words
  int lane, w, wn, wm;
  uint32_t woff[2], xoff[4], soff;   // per-lane byte offsets of this lane's copies
  // LDS read offsets inside a stage: token slice 0's two fragment halves and
  // its scale word (slice j adds 8192 j / 256 j), weight tile 0's fragment and
  // its E8M0 byte (tile i adds 64 dt / 4 dt, dt = its first row - tile 0's).
  uint32_t rb_l, rb_h, rb_s, ra, rs;

  __device__ WideMxItem(const FfnGroup &g, const TileEntry &te, int nt_, int H_) : G(g), ntile(nt_), H(H_) {
    lane = threadIdx.x & 63;
    w = uniform(threadIdx.x >> 6);
    wn = w & 1;
    wm = w >> 1;
    const int g4 = lane >> 4;
    e = te.ge & 0xFFFFFF;
    rend = min(max(group_off(G, e + 1), 0), G.nrows);
    rbeg = min(max(group_off(G, e), 0) + te.m0, rend);
    nvalid = min(rend - rbeg, WBM);
    I = G.I;
    K = GATEUP ? H : I;
    nchunk = K / 128;
    col0 = GATEUP ? ntile * 128 : ntile * TBN;
    const int64_t wrows = GATEUP ? 2 * (int64_t)I : (int64_t)H;
    const int wrowb = K / 2, srowb = K / 32;
    wsrc = (GATEUP ? G.wgu : G.wd) + (int64_t)e * wrows * wrowb;
    ssrc = (GATEUP ? G.mgu : G.md) + (int64_t)e * wrows * srowb;
    const bool indirect = GATEUP && G.xsrc != nullptr;
    asrc = (GATEUP ? G.x : G.h) + (indirect ? 0 : (int64_t)rbeg * K);
    ascale = (GATEUP ? G.xs : G.hs) + (indirect ? 0 : (int64_t)rbeg * nchunk);
    auto wrow = [&](int r) { return GATEUP ? (r < 128 ? col0 + r : I + col0 + r - 128) : col0 + r; };
    // rows past the end repeat a valid row; indirect rows come from x row xsrc[row] / xdiv
    auto xrow = [&](int r) -> int64_t {
      const int rr = min(r, nvalid - 1);
      return indirect ? G.xsrc[rbeg + rr] / G.xdiv : rr;
    };
#pragma unroll
    for (int t = 0; t < 2; ++t) woff[t] = (uint32_t)(wrow(16 * (w + 8 * t) + (lane & 15)) * wrowb + 16 * g4);
    nissue = 3;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 8 * (w + 8 * t) + (lane >> 3);
      const int c = (lane & 7) ^ swz_f(r);
      xoff[t] = (uint32_t)(xrow(r) * K + c * 16);
      if (8 * (w + 8 * t) < nvalid) ++nissue;
    }
    soff = w < 4 ? (uint32_t)(xrow(64 * w + lane) * nchunk * 4) : (uint32_t)(wrow(64 * (w - 4) + lane) * srowb);
    // buffer sizes: the expert's code and scale matrices, the item's token rows
    // (indirect rows: any row of x, whose offsets the caller keeps below 2^31)
    const uint32_t kAny = 0x7FFFFFFF;
    rw = buf_rsrc(wsrc, (uint32_t)(wrows * wrowb));
    rx = buf_rsrc(asrc, indirect ? kAny : (uint32_t)(nvalid * K));
    rsc = w < 4 ? buf_rsrc(ascale, indirect ? kAny : (uint32_t)(nvalid * nchunk * 4))
                : buf_rsrc(ssrc, (uint32_t)(wrows * srowb));
    const int r0 = 16 * wm + (lane & 15);
    rb_l = (uint32_t)(MXTOK + swz(r0, g4));
    rb_h = (uint32_t)(MXTOK + swz(r0, 4 + g4));
    rb_s = (uint32_t)(MXTS + 4 * r0);
    const int a0 = GATEUP ? 64 * wn : 128 * wn;   // first weight row of tile 0
    ra = (uint32_t)(64 * a0 + 16 * lane);
    rs = (uint32_t)(MXWS + 4 * (a0 + (lane & 15)) + g4);
  }

  // Direct-to-LDS copies of K chunk kc into stage buffer sb: 2 (codes) + up to
  // 4 (tokens) + 1 (scale words) instructions per wave, nissue in all; copy q
  // of the seven.  A token copy whose 8 rows all lie past the item's last row
  // is skipped (those LDS rows only feed output columns of padding rows, which
  // are never stored).
  static constexpr int NCOPY = 7;
  __device__ __forceinline__ void issue_one(int q, int kc, uint8_t *sb) const {
    if (q < 2) {
      bdma16(rw, woff[q], 64 * kc, sb + (w + 8 * q) * 1024);
    } else if (q < 6) {
      const int t = q - 2;
      if (8 * (w + 8 * t) < nvalid) bdma16(rx, xoff[t], 128 * kc, sb + MXTOK + (w + 8 * t) * 1024);
    } else {
      bdma4(rsc, soff, 4 * kc, sb + (w < 4 ? MXTS + 256 * w : MXWS + 256 * (w - 4)));
    }
  }
  __device__ __forceinline__ void issue(int kc, uint8_t *sb) const {
#pragma unroll
    for (int q = 0; q < NCOPY; ++q) issue_one(q, kc, sb);
  }

  // Wait until this wave's copies of the chunk about to be consumed have
  // landed (those of the chunk after it may still be in flight).
  __device__ __forceinline__ void wait_one_behind() const {
    switch (nissue) {
      case 7: wait_vm_lgkm0<7>(); break;
      case 6: wait_vm_lgkm0<6>(); break;
      case 5: wait_vm_lgkm0<5>(); break;
      case 4: wait_vm_lgkm0<4>(); break;
      default: wait_vm_lgkm0<3>(); break;
    }
  }

  __device__ __forceinline__ static int tile_dt(int i) { return GATEUP ? (i < 4 ? 16 * i : 128 + 16 * (i - 4)) : 16 * i; }

  // The MFMAs of one K chunk: token fragments read once (slice 0 first, the
  // others while the first MFMA runs), weight tile i+1's fragment and scale
  // byte read while tile i's MFMAs run.
  template <int NJ>
  __device__ __forceinline__ void chunk(const uint8_t *sb, f32x4 (&acc)[8][4]) const {
    i32x4 bl[NJ], bh[NJ];
    float sx[NJ];
    i32x4 A[2];
    int sa[2];
    A[0] = *reinterpret_cast<const i32x4 *>(sb + ra);
    sa[0] = sb[rs];
    bl[0] = *reinterpret_cast<const i32x4 *>(sb + rb_l);
    bh[0] = *reinterpret_cast<const i32x4 *>(sb + rb_h);
    sx[0] = *reinterpret_cast<const float *>(sb + rb_s);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NT = 8 * NJ;
    f32x4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT + 2; ++t) {
      f32x4 cur = {0.f, 0.f, 0.f, 0.f};
      if (t < NT) {
        const int i = t / NJ, j = t % NJ;
        cur = mfma_mx(A[i & 1], bl[j], bh[j], sa[i & 1]);
        if (t == 0) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int jj = 1; jj < NJ; ++jj) {
            bl[jj] = *reinterpret_cast<const i32x4 *>(sb + rb_l + 8192 * jj);
            bh[jj] = *reinterpret_cast<const i32x4 *>(sb + rb_h + 8192 * jj);
            sx[jj] = *reinterpret_cast<const float *>(sb + rb_s + 256 * jj);
          }
        }
        if (j == 0 && i + 1 < 8) {
          A[(i + 1) & 1] = *reinterpret_cast<const i32x4 *>(sb + ra + 64 * tile_dt(i + 1));
          sa[(i + 1) & 1] = sb[rs + 4 * tile_dt(i + 1)];
        }
      }

      if (t >= 2) {
        const int i = (t - 2) / NJ, j = (t - 2) % NJ;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p2[r], sx[j], acc[i][j][r]);
      }
      p2 = p1;
      p1 = cur;
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Step kc: wait for this wave's copies of chunk kc, sync the workgroup
  // (every wave's copies have landed, and nobody reads chunk kc-1's buffer any
  // more), consume chunk kc and refill that buffer with chunk kc+2: waves 0-3
  // issue their copies before their MFMAs, waves 4-7 (the other wave on each
  // SIMD) after them, so that while one wave of a SIMD waits for the copy path
  // to take its instructions the other keeps the matrix core busy.  Chunks 0
  // and 1 were issued into stages par and par+1 (mod 3) before the call; chunk
  // kc sits in stage (par + kc) % 3.  The first step also waits for chunk 1
  // (and for the previous item's output stores, issued after it).
  template <int NJ>
  __device__ __forceinline__ void mainloop(uint8_t *lds, int par, f32x4 (&acc)[8][4]) const {
    int sc = par, sn = par == 0 ? 2 : par - 1;   // stages of chunk kc and of chunk kc+2
    const bool late = w >= 4;
    for (int kc = 0; kc < nchunk; ++kc) {
      // waves 4-7: chunk kc+1 into the stage chunk kc-2 used (free since the
      // last barrier), after their MFMAs of chunk kc-1
      if (late && kc >= 1 && kc + 1 < nchunk) issue(kc + 1, lds + (sn == 0 ? 2 : sn - 1) * MXSTAGE);
      if (kc == 0 || kc + 1 == nchunk)
        wait_vm_lgkm0<0>();
      else
        wait_one_behind();
      wg_barrier();
      // waves 0-3: chunk kc+2 into the stage chunk kc-1 used, before their MFMAs
      if (!late && kc + 2 < nchunk) issue(kc + 2, lds + sn * MXSTAGE);
      chunk<NJ>(lds + sc * MXSTAGE, acc);
      sc = sc == 2 ? 0 : sc + 1;
      sn = sn == 2 ? 0 : sn + 1;
    }
  }
};

// Issue work item w's chunks 0 and 1 into stages par and par+1 (mod 3).
template <bool GATEUP>
__device__ __forceinline__ void wide_mx_begin(const TiledArgs &a, const WideWork &w, uint8_t *lds, int par) {
  const FfnGroup &G = (w.te.ge >> 24) ? a.g1 : a.g0;
  WideMxItem<GATEUP> it(G, w.te, w.ntile, a.H);
  it.issue(0, lds + par * MXSTAGE);
  if (it.nchunk > 1) it.issue(1, lds + (par == 2 ? 0 : par + 1) * MXSTAGE);
}

// One MX work item whose chunks 0 and 1 were issued beforehand.  After its
// last step it starts the next item (if `next` is an MX item) in the two
// stages after its last chunk's, so that those copies are in flight during
// this item's epilogue.  Returns the next item's first stage.
template <bool GATEUP>
__device__ __forceinline__ int wide_mx_item(const TiledArgs &a, const FfnGroup &G, const WideWork &cur,
                                            const WideWork &next, int par, uint8_t *lds, float *red) {
  WideMxItem<GATEUP> it(G, cur.te, cur.ntile, a.H);
  const int lane = it.lane, wn = it.wn, wm = it.wm;
  // active 16-row token slices of this wave: slice j covers rows 16*(wm + 4j)
  const int nact = uniform(it.nvalid <= 16 * wm ? 0 : min(4, (it.nvalid - 16 * wm + 63) / 64));
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  switch (nact) {
    case 4: it.template mainloop<4>(lds, par, acc); break;
    case 3: it.template mainloop<3>(lds, par, acc); break;
    case 2: it.template mainloop<2>(lds, par, acc); break;
    case 1: it.template mainloop<1>(lds, par, acc); break;
    default: it.template mainloop<1>(lds, par, acc); break;   // keeps the barrier count equal across waves
  }
  const int npar = (par + it.nchunk) % MXNSTAGE;
  if (next.valid) wide_mx_begin<GATEUP>(a, next, lds, npar);
  const int rbeg = it.rbeg, nvalid = it.nvalid, I = it.I, col0 = it.col0;
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) brow[j] = 16 * (wm + 4 * j);
  store_item<true, GATEUP, WBM>(G, acc, brow, lane, wn, rbeg, nvalid, I, col0, cur.ntile, a.H, red);
  // the next item's first step waits for its copies and syncs the workgroup
  // before anything reads LDS; the reduction area is free once every wave is
  // past this barrier
  wait_lgkm0();
  wg_barrier();
  return npar;
}

// A bf16 item of the shared expert inside the MX launch (the bf16 wide item;
// bf16 items stage no weight scales).
template <bool GATEUP>
__device__ __forceinline__ int wide_bf16_item(const TiledArgs &a, const FfnGroup &G, const WideWork &cur,
                                              const WideWork &next, int par, uint8_t *lds, float *red) {
  float *const wscb[2] = {red, red};
  return G.tile16 ? wide_item<false, GATEUP, true>(a, G, cur, next, par, lds, red, wscb)
                  : wide_item<false, GATEUP, false>(a, G, cur, next, par, lds, red, wscb);
}

// MX routed experts (and a bf16 shared expert) with 256-row token tiles.  Each
// workgroup's items of one kind follow each other with their copies
// overlapped; where the kind changes the ring starts over at stage 0.
template <bool GATEUP>
__global__ __launch_bounds__(WTHREADS, 1) void wide_mx_kernel(TiledArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float *red = reinterpret_cast<float *>(lds + MXNSTAGE * MXSTAGE);
  const int nslots = a.hdr[0];
  const int count = nslots * a.nt;
  const int64_t n0 = (int64_t)min(a.hdr[1], nslots) * a.nt;
  const int xcd = blockIdx.x & 7, per = gridDim.x >> 3, slot0 = blockIdx.x >> 3;
  const int beg = range_start(xcd, n0, count, a.c0, a.c1), end = range_start(xcd + 1, n0, count, a.c0, a.c1);
  int L = beg + slot0;
  WideWork cur = wide_find<GATEUP>(a, L, end, per, nslots);
  bool begun = false;
  int par = 0;
  while (cur.valid) {
    L += per;
    const WideWork next = wide_find<GATEUP>(a, L, end, per, nslots);
    const FfnGroup &G = (cur.te.ge >> 24) ? a.g1 : a.g0;
    const bool mx = G.mx != 0;
    const bool same = next.valid && (((next.te.ge >> 24) ? a.g1 : a.g0).mx != 0) == mx;
    const WideWork nx = same ? next : WideWork{{0, 0}, 0, 0};
    if (!begun) {
      par = 0;
      if (mx)
        wide_mx_begin<GATEUP>(a, cur, lds, 0);
      else
        wide_begin<GATEUP>(a, cur, lds, red);
    }
    par = mx ? wide_mx_item<GATEUP>(a, G, cur, nx, par, lds, red) : wide_bf16_item<GATEUP>(a, G, cur, nx, par, lds, red);
    begun = same;
    cur = next;
  }
}

// LDS: the copy ring, the h-scale reduction area, the weight-scale staging (H, I <= 16384;
// the wide kernel keeps two buffers, the current item's and the next one's)
size_t tiled_lds_bytes() { return NSTAGE * TSTAGE + 2 * TBM * sizeof(float) + 2 * 128 * sizeof(float); }
size_t wide_lds_bytes() { return WNSTAGE * WSTAGE + 2 * WBM * sizeof(float) + 2 * 2 * 128 * sizeof(float); }
size_t wide_mx_lds_bytes() { return MXNSTAGE * MXSTAGE + 2 * WBM * sizeof(float); }

int num_compute_units() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

hipError_t launch_tiled_ffn(const FfnGroup *g, int ngroups, int H, const void *tiles, int32_t *hdr, int num_cus,
                            int bm, int site, hipStream_t st) {
  if (bm != 128 && bm != WBM) return hipErrorInvalidValue;
  const bool wide = bm == WBM;
  TiledArgs a{g[0], ngroups > 1 ? g[1] : g[0], static_cast<const TileEntry *>(tiles), hdr, H, 0, 0, 0};
  auto chunks = [](const FfnGroup &G, int K) { return std::max(1, K * (G.fp8 ? 1 : 2) / 128); };
  int maxI = 0;
  for (int i = 0; i < ngroups; ++i) maxI = std::max(maxI, (int)g[i].I);
  const unsigned grid = (unsigned)(std::max(num_cus, 8) / 8 * 8);
  const size_t lds = wide ? wide_lds_bytes() : tiled_lds_bytes();
  static bool attr_set[64] = {};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    const void *fns[4] = {reinterpret_cast<const void *>(&tiled_ffn_kernel<true>),
                          reinterpret_cast<const void *>(&tiled_ffn_kernel<false>),
                          reinterpret_cast<const void *>(&wide_ffn_kernel<true>),
                          reinterpret_cast<const void *>(&wide_ffn_kernel<false>)};
    const size_t need[4] = {tiled_lds_bytes(), tiled_lds_bytes(), wide_lds_bytes(), wide_lds_bytes()};
    for (int i = 0; i < 4; ++i) {
      const hipError_t e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)need[i]);
      if (e != hipSuccess) return e;
    }
    attr_set[dev] = true;
  }
  a.nt = maxI / 128;
  a.c0 = chunks(a.g0, H);
  a.c1 = chunks(a.g1, H);
  timing_before(site, st);
  if (wide)
    wide_ffn_kernel<true><<<grid, WTHREADS, lds, st>>>(a);
  else
    tiled_ffn_kernel<true><<<grid, TTHREADS, lds, st>>>(a);
  timing_after(site, st);
  a.nt = H / TBN;
  a.c0 = chunks(a.g0, a.g0.I);
  a.c1 = chunks(a.g1, a.g1.I);
  timing_before(site + 1, st);
  if (wide)
    wide_ffn_kernel<false><<<grid, WTHREADS, lds, st>>>(a);
  else
    tiled_ffn_kernel<false><<<grid, TTHREADS, lds, st>>>(a);
  timing_after(site + 1, st);
  return hipGetLastError();
}


hipError_t launch_wide_mx_ffn(const FfnGroup *g, int ngroups, int H, const void *tiles, int32_t *hdr, int num_cus,
                              int site, hipStream_t st) {
  if (ngroups < 1 || ngroups > 2) return hipErrorInvalidValue;
  for (int i = 0; i < ngroups; ++i) {
    if (g[i].mx ? !tiled_mx_supported(g[i], H) : (g[i].fp8 || g[i].I % 128 != 0)) return hipErrorInvalidValue;
  }
  if (H % 256 != 0) return hipErrorInvalidValue;
  TiledArgs a{g[0], ngroups > 1 ? g[1] : g[0], static_cast<const TileEntry *>(tiles), hdr, H, 0, 0, 0};
  // relative cost of one item for the XCD split: K chunks x the chunk's cost
  // (an MX stage is 50 KB of copies, a bf16 stage 65 KB with more LDS reads)
  auto cost = [](const FfnGroup &G, int K) { return G.mx ? 3 * std::max(1, K / 128) : 4 * std::max(1, K * 2 / 128); };
  int maxI = 0;
  for (int i = 0; i < ngroups; ++i) maxI = std::max(maxI, (int)g[i].I);
  const unsigned grid = (unsigned)(std::max(num_cus, 8) / 8 * 8);
  const size_t lds = wide_mx_lds_bytes();
  static bool attr_set[64] = {};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    const void *fns[2] = {reinterpret_cast<const void *>(&wide_mx_kernel<true>),
                          reinterpret_cast<const void *>(&wide_mx_kernel<false>)};
    for (int i = 0; i < 2; ++i) {
      const hipError_t e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    attr_set[dev] = true;
  }
  a.nt = maxI / 128;
  a.c0 = cost(a.g0, H);
  a.c1 = cost(a.g1, H);
  timing_before(site, st);
  wide_mx_kernel<true><<<grid, WTHREADS, lds, st>>>(a);
  timing_after(site, st);
  a.nt = H / TBN;
  a.c0 = cost(a.g0, a.g0.I);
  a.c1 = cost(a.g1, a.g1.I);
  timing_before(site + 1, st);
  wide_mx_kernel<false><<<grid, WTHREADS, lds, st>>>(a);
  timing_after(site + 1, st);
  return hipGetLastError();
}

}  // namespace moe
