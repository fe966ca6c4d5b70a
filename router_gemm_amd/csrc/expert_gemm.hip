// expert_gemm.hip -- grouped expert GEMMs on gfx950 MFMA:
//   gate/up:  z = a W_gu[e]^T (one grouped GEMM over [gate; up] rows), fused
//             SwiGLU epilogue h = silu(z_gate) * z_up, h stored as bf16 or as
//             E4M3 with one fp32 scale per token per 128 columns;
//   down:     o = h W_d[e]^T.
// ("Step-5 minimal inference", introduction: block-scaled FP8 expert GEMM;
// "Step-5-Preview", "Model Architecture": each expert is 4,096 -> 1,536 -> 4,096
// and the parameter count gives three such matrices, a gated FFN.)
//
// Operand roles.  Weights are the MFMA A operand (rows n of [out, in]) and
// token rows the B operand, so each lane's four accumulators are four
// consecutive output columns of one token.  Both operands are K-contiguous in
// memory: a lane reads 32 contiguous bytes of its row per 128-byte K chunk
// (128 e4m3 codes or 64 bf16 values), so no transposes are needed.
//
// Tile16 weights (FfnGroup::tile16, written by moe_pack_weights): each 16-row
// x 128-byte tile is stored in the order the two fragment loads of a wave
// consume it, so a load instruction reads one contiguous kilobyte; those loads
// use the non-temporal policy (every weight line is read exactly once).
// Row-major weights make each load touch 16 half lines and held the stream at
// about 5.8 TB/s where tile16 reaches about 6.6.
//
// FP8 block scales.  A K chunk of 128 codes is exactly one weight block column
// and one activation group, so one 16x16x128 MFMA yields the raw block
// product, and acc += P * (s_w * s_a[token]) applies both scales in fp32.
//
// MX FP4 weights.  The scaled MFMA takes an E2M1 A operand (16 bytes per lane:
// lane group g = lane/16 holds inputs 32g..32g+31 of the 128-input chunk,
// even input in the low nibble, exactly the stored packing) with one E8M0
// scale byte per lane (its row, its 32-input block), so the weight scales
// are applied inside the instruction; the E4M3 B operand is read in the
// instruction's own K order (lane group g: inputs 16g..16g+15 and
// 64+16g..64+16g+15), and the token's fp32 group scale multiplies the chunk
// product afterwards as in fp8 mode.  Such a fragment is only 64 bytes of a
// row per load instruction (half a 128-byte line), so for 16- and 32-row
// token tiles the codes are staged through LDS by direct-to-LDS copies that
// move 8 rows x a whole line per instruction (see the gate/up body).
//
// Work decomposition.  A device-built list holds one entry per (expert,
// 16*MT-row tile of that expert's rows); blockIdx.y indexes it (entries past
// the device-side count exit at once), blockIdx.x the output-column tile.
// The host never reads the per-expert counts.

#include <algorithm>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

__device__ __forceinline__ FfnGroup pick_group(const FfnGroup &g0, const FfnGroup &g1, int g) {
  return g ? g1 : g0;
}

// One workgroup (1024 threads, E <= 1024 per group): for each group in turn,
// tiles of bm rows per expert, in expert order.
__global__ __launch_bounds__(1024) void build_tiles_kernel(FfnGroup g0, FfnGroup g1, int ngroups, int bm,
                                                           int max_tiles, TileEntry *__restrict__ tiles,
                                                           int32_t *__restrict__ hdr) {
  __shared__ int32_t buf[1024];
  const int tid = threadIdx.x;
  int base0 = 0;
  for (int g = 0; g < ngroups; ++g) {
    const FfnGroup G = pick_group(g0, g1, g);
    int n = 0;
    if (tid < G.E) {
      const int b = min(max(group_off(G, tid), 0), G.nrows);
      const int e = min(max(group_off(G, tid + 1), b), G.nrows);
      n = e - b;
    }
    const int cnt = (n + bm - 1) / bm;
    __syncthreads();
    buf[tid] = cnt;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int32_t add = tid >= o ? buf[tid - o] : 0;
      __syncthreads();
      buf[tid] += add;
      __syncthreads();
    }
    const int base = base0 + buf[tid] - cnt;
    for (int j = 0; j < cnt; ++j)
      if (base + j < max_tiles) tiles[base + j] = TileEntry{(g << 24) | tid, j * bm};
    base0 += buf[1023];
    if (g == 0 && tid == 0) hdr[1] = min(base0, max_tiles);
  }
  if (tid == 0) hdr[0] = min(base0, max_tiles);
}

hipError_t launch_build_tiles(const FfnGroup &g, int bm, int max_tiles, TileEntry *tiles, int32_t *hdr,
                              hipStream_t st) {
  build_tiles_kernel<<<1, 1024, 0, st>>>(g, g, 1, bm, max_tiles, tiles, hdr);
  return hipGetLastError();
}

// Operand fragment of one lane for one 128-byte K chunk: 32 bytes.
struct Frag {
  i32x4 lo, hi;
};

__device__ __forceinline__ Frag load_frag(const uint8_t *p) { return Frag{load16(p), load16(p + 16)}; }
// The fragment of a tile16 weight tile: two 1 KB loads of the wave (lane l at
// 16 l and 1024 + 16 l), non-temporal: every weight line is read once.
__device__ __forceinline__ Frag load_frag_t16(const uint8_t *p) {
  return Frag{__builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(p)),
              __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(p + 1024))};
}

__device__ __forceinline__ i32x8 frag_fp8(const Frag &f) {
  return i32x8{f.lo[0], f.lo[1], f.lo[2], f.lo[3], f.hi[0], f.hi[1], f.hi[2], f.hi[3]};
}

// acc += A(16 rows x chunk) * B(chunk x 16 tokens); fp8 chunks are one
// 128-wide scale block, so the block product is scaled once.
template <bool FP8>
__device__ __forceinline__ f32x4 chunk_mma(const Frag &a, const Frag &b, f32x4 acc, float scale) {
  if constexpr (FP8) {
    const f32x4 p = mfma_fp8(frag_fp8(a), frag_fp8(b), f32x4{0.f, 0.f, 0.f, 0.f});
    acc[0] += p[0] * scale;
    acc[1] += p[1] * scale;
    acc[2] += p[2] * scale;
    acc[3] += p[3] * scale;
    return acc;
  } else {
    acc = mfma_bf16(__builtin_bit_cast(bf16x8, a.lo), __builtin_bit_cast(bf16x8, b.lo), acc);
    return mfma_bf16(__builtin_bit_cast(bf16x8, a.hi), __builtin_bit_cast(bf16x8, b.hi), acc);
  }
}

// acc += (E2M1 A with per-lane E8M0 scale sa) * (E4M3 B) * sx for one chunk.
__device__ __forceinline__ f32x4 chunk_mma_mx(const i32x4 &a, const Frag &b, int sa, f32x4 acc, float sx) {
  const i32x8 a8 = i32x8{a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, frag_fp8(b), f32x4{0.f, 0.f, 0.f, 0.f},
                                                                   4, 0, 0, sa, 0, 127);
  acc[0] += p[0] * sx;
  acc[1] += p[1] * sx;
  acc[2] += p[2] * sx;
  acc[3] += p[3] * sx;
  return acc;
}

// E4M3 B fragment of one chunk in the scaled MFMA's K order: inputs
// 16g..16g+15 and 64+16g..64+16g+15 of the chunk for lane group g
// (p points at the chunk start + 16g).
__device__ __forceinline__ Frag load_frag_k64(const uint8_t *p) { return Frag{load16(p), load16(p + 64)}; }

// LDS reads of staged MX weight fragments, written as one asm block that
// waits for its own results.  The compiler cannot tell these buffers apart
// from the ones the direct-to-LDS copies are still filling, so LDS reads it
// can see make it wait for every copy in flight; the callers instead wait
// with vmcnt for exactly the copies into the buffer they read.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}
// r[4j + t] = 16 bytes at a_j + 2048 t (t = 0..3, j = 0..1).
__device__ __forceinline__ void lds_read_2x4(uint32_t a0, uint32_t a1, i32x4 (&r)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:2048\n\t"
      "ds_read_b128 %2, %8 offset:4096\n\t"
      "ds_read_b128 %3, %8 offset:6144\n\t"
      "ds_read_b128 %4, %9\n\t"
      "ds_read_b128 %5, %9 offset:2048\n\t"
      "ds_read_b128 %6, %9 offset:4096\n\t"
      "ds_read_b128 %7, %9 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a0), "v"(a1));
}
// r[2j + t] = 16 bytes at a_j + 2048 t (t = 0..1, j = 0..1).
__device__ __forceinline__ void lds_read_2x2(uint32_t a0, uint32_t a1, i32x4 (&r)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:2048\n\t"
      "ds_read_b128 %2, %5\n\t"
      "ds_read_b128 %3, %5 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a0), "v"(a1));
}

struct StreamArgs {
  FfnGroup g0, g1;
  const TileEntry *tiles;
  const int32_t *ntiles;
  int H;
  int ssplit;      // > 1: group sgroup's gate/up K split this many ways (blockIdx.z), partial sums to spart
  int sgroup;
  float *spart;    // [ssplit][16][2 I] fp32 (I of group sgroup); needs nchunk >= ssplit (the plan asks H >= 1024)
};

// Rows [rbeg, rend) of the tile, clamped to the group's row count.
__device__ __forceinline__ void tile_rows(const FfnGroup &G, const TileEntry &te, int &rbeg, int &rend) {
  const int e = te.ge & 0xFFFFFF;
  rend = min(max(group_off(G, e + 1), 0), G.nrows);
  rbeg = min(max(group_off(G, e), 0) + te.m0, rend);
}

// ---------------------------------------------------------------- gate/up (streaming)
// Workgroup: 4 waves x (GW gate + GW up 16-row weight tiles) = 64*GW h
// columns x 16*MT token rows.  Each wave streams its own weight rows straight
// from HBM into MFMA operand registers (no reuse across waves, so no LDS).
// SPLIT (bf16, one 16-row tile, row-major weights): chunks
// [nchunk z / S, nchunk (z+1) / S) only, and the raw gate and up sums go to
// spart[z][row][2I] instead of through the epilogue.
template <bool FP8, bool MX, int MT, int GW, bool T16 = false, bool SPLIT = false>
__device__ __forceinline__ void gate_up_body(const FfnGroup &G, const TileEntry &te, int H, int z = 0, int S = 1,
                                             float *spart = nullptr) {
  static_assert(!SPLIT || (!FP8 && MT == 1), "the K split is for bf16 groups with 16-row tiles");
  static_assert(FP8 || !MX, "MX weights take e4m3 activations");
  static_assert(!(MX && T16), "MX weights are row-major");
  constexpr int ESZ = FP8 ? 1 : 2;
  const int lane = lane_id(), w = wave_id();
  int rbeg, rend;
  tile_rows(G, te, rbeg, rend);
  const int e = te.ge & 0xFFFFFF;
  const int I = G.I;
  const int64_t xrowb = (int64_t)H * ESZ;             // activation row bytes
  const int64_t wrowb = MX ? (int64_t)H / 2 : xrowb;  // weight row bytes
  const int hc0 = blockIdx.x * (64 * GW) + w * (16 * GW);
  const int g4 = lane >> 4;
  const int koff = MX ? 16 * g4 : 32 * g4;

  const uint8_t *wbase = G.wgu + (int64_t)e * 2 * I * wrowb;
  const uint8_t *wg[GW], *wu[GW];
  const uint8_t *mg[GW], *mu[GW];   // MX: the lane's row of E8M0 scale bytes
#pragma unroll
  for (int i = 0; i < GW; ++i) {
    const int64_t rg = hc0 + 16 * i + (lane & 15), ru = I + rg;
    if constexpr (T16) {   // lane l reads 16 l (and 1024 + 16 l) of each tile
      wg[i] = wbase + ((int64_t)(hc0 + 16 * i) >> 4) * 2048 + 16 * lane;
      wu[i] = wbase + ((int64_t)(I + hc0 + 16 * i) >> 4) * 2048 + 16 * lane;
    } else {
      wg[i] = wbase + rg * wrowb + koff;
      wu[i] = wbase + ru * wrowb + koff;
    }
    if constexpr (MX) {
      mg[i] = G.mgu + ((int64_t)e * 2 * I + rg) * (H / 32);
      mu[i] = G.mgu + ((int64_t)e * 2 * I + ru) * (H / 32);
    }
  }
  const uint8_t *xr[MT];
  bool xv[MT];
  int xrow[MT], xsrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    xrow[m] = rbeg + 16 * m + (lane & 15);
    xv[m] = xrow[m] < rend;
    xsrow[m] = xv[m] ? xrow[m] : (rbeg < rend ? rbeg : 0);   // a row that exists
    xr[m] = G.x + (int64_t)xsrow[m] * xrowb + koff;
  }
  f32x4 ag[GW][MT], au[GW][MT];
#pragma unroll
  for (int i = 0; i < GW; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) ag[i][m] = au[i][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunk = (int)(xrowb / 128);
  const int KB = H / 128;
  const float *sg = (FP8 && !MX) ? G.sgu + ((int64_t)e * (2 * I / 128) + hc0 / 128) * KB : nullptr;
  const float *su = (FP8 && !MX) ? G.sgu + ((int64_t)e * (2 * I / 128) + (I + hc0) / 128) * KB : nullptr;
  const Frag zf = Frag{i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};

  if constexpr (MX) {
    // Fallback for shapes the staged loop below does not take (64-row token
    // tiles, an odd chunk count): two-chunk steps with fragments loaded
    // straight into registers, every load of a step issued before its first
    // MFMA.
    auto plain_steps = [&]() {
      for (int c = 0; c < nchunk; c += 2) {
        const int nv = min(2, nchunk - c);
        i32x4 fg[2][GW], fu[2][GW];
        uint32_t sgw[2][GW], suw[2][GW];
        Frag fx[2][MT];
        float sx[2][MT];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int cj = j < nv ? c + j : c;   // a lone last chunk is loaded twice, counted once
#pragma unroll
          for (int i = 0; i < GW; ++i) {
            fg[j][i] = load16(wg[i] + (int64_t)cj * 64);
            fu[j][i] = load16(wu[i] + (int64_t)cj * 64);
            sgw[j][i] = *reinterpret_cast<const uint32_t *>(mg[i] + 4 * cj);
            suw[j][i] = *reinterpret_cast<const uint32_t *>(mu[i] + 4 * cj);
          }
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            // branch-free: rows past the tile read a valid row and are zeroed after
            const Frag f = load_frag_k64(xr[m] + (int64_t)cj * 128);
            const float sv = G.xs[(int64_t)xsrow[m] * KB + cj];
            fx[j][m] = xv[m] ? f : zf;
            sx[j][m] = xv[m] ? sv : 0.f;
          }
        }
        // keep every load of the step ahead of the first MFMA (the scheduler
        // otherwise interleaves load, wait, MFMA and loses the overlap)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (j >= nv) break;
#pragma unroll
          for (int i = 0; i < GW; ++i) {
            const int sag = (int)((sgw[j][i] >> (8 * g4)) & 0xFFu);
            const int sau = (int)((suw[j][i] >> (8 * g4)) & 0xFFu);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              ag[i][m] = chunk_mma_mx(fg[j][i], fx[j][m], sag, ag[i][m], sx[j][m]);
              au[i][m] = chunk_mma_mx(fu[j][i], fx[j][m], sau, au[i][m], sx[j][m]);
            }
          }
        }
      }
    };
    if (MT <= 2 && (nchunk & 1) == 0) {
      // Weight codes go through LDS.  A 16x16x128 fp4 fragment gives a row
      // only 64 bytes per load instruction (half a 128-byte line, so every L1
      // miss moves half a line); a direct-to-LDS copy instead moves 8 rows x
      // one whole line (two chunks) per instruction.  Each wave owns two 8 KB
      // buffers (its 2*GW tiles x 16 rows x 128 bytes), 16-byte columns
      // XOR-swizzled by row % 8; no other wave touches them, so no barriers.
      // Every code line is read once, so the copies are non-temporal: cached
      // normally they evicted the rows' scale words between steps (16% more
      // bytes fetched, 8% slower).
      // (two separate arrays, so that alias analysis sees that reading one
      // buffer never waits for the copies into the other)
      __shared__ __attribute__((aligned(16))) uint8_t wlds0[4][2 * GW][2048];
      __shared__ __attribute__((aligned(16))) uint8_t wlds1[4][2 * GW][2048];
      const uint8_t *tb[2 * GW];
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        tb[i] = wbase + (int64_t)(hc0 + 16 * i) * wrowb;
        tb[GW + i] = wbase + (int64_t)(I + hc0 + 16 * i) * wrowb;
      }
      const int sr = lane >> 3;
      const uint32_t coff0 = (uint32_t)(sr * wrowb + 16 * ((lane & 7) ^ sr));
      const uint32_t coff1 = coff0 + (uint32_t)(8 * wrowb);
      auto copy = [&](uint8_t *buf, int c) {
#pragma unroll
        for (int t = 0; t < 2 * GW; ++t) {
          const uint8_t *src = tb[t] + (int64_t)c * 64;
          dma16_stream(src + coff0, buf + t * 2048);
          dma16_stream(src + coff1, buf + t * 2048 + 1024);
        }
      };
      struct XB {
        uint2 sg[GW], su[GW];
        Frag x[2][MT];
        float sx[2][MT];
      };
      auto loadx = [&](XB &b, int c) {
#pragma unroll
        for (int i = 0; i < GW; ++i) {
          b.sg[i] = *reinterpret_cast<const uint2 *>(mg[i] + 4 * c);
          b.su[i] = *reinterpret_cast<const uint2 *>(mu[i] + 4 * c);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            b.x[j][m] = load_frag_k64(xr[m] + (int64_t)(c + j) * 128);
            b.sx[j][m] = G.xs[(int64_t)xsrow[m] * KB + c + j];
          }
      };
      const int rho = lane & 15;
      static_assert(GW == 2, "the staged MX gate/up path reads 2 x 4 tiles");
      auto compute = [&](const uint8_t *buf, const XB &b) {
        i32x4 fr[8];
        lds_read_2x4(lds_addr(buf + rho * 128 + 16 * ((0 + g4) ^ (rho & 7))),
                     lds_addr(buf + rho * 128 + 16 * ((4 + g4) ^ (rho & 7))), fr);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < GW; ++i) {
            const i32x4 fgv = fr[4 * j + i];
            const i32x4 fuv = fr[4 * j + GW + i];
            const int sag = (int)(((j ? b.sg[i].y : b.sg[i].x) >> (8 * g4)) & 0xFFu);
            const int sau = (int)(((j ? b.su[i].y : b.su[i].x) >> (8 * g4)) & 0xFFu);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              const float sxm = xv[m] ? b.sx[j][m] : 0.f;
              ag[i][m] = chunk_mma_mx(fgv, b.x[j][m], sag, ag[i][m], sxm);
              au[i][m] = chunk_mma_mx(fuv, b.x[j][m], sau, au[i][m], sxm);
            }
          }
      };
      // Each step issues its token loads first and its 4*GW copies last, so
      // "all but the last 4*GW vector-memory instructions done" means the
      // previous step's copies have landed.
      uint8_t *const B0 = &wlds0[w][0][0];
      uint8_t *const B1 = &wlds1[w][0][0];
      constexpr int COPIES = 4 * GW;
      XB X0, X1;
      loadx(X0, 0);
      copy(B0, 0);
      // the token loads of the first step done before the loop, as they are
      // on the way round it (a loop-carried load still in flight on one path
      // makes the compiler wait for everything at the top of the loop)
      wait_vm<COPIES>();
      int c = 0;
      for (; c + 4 < nchunk; c += 4) {
        loadx(X1, c + 2);
        copy(B1, c + 2);
        wait_vm<COPIES>();
        __builtin_amdgcn_sched_barrier(0);
        compute(B0, X0);
        __builtin_amdgcn_sched_barrier(0);
        loadx(X0, c + 4);
        copy(B0, c + 4);
        wait_vm<COPIES>();
        __builtin_amdgcn_sched_barrier(0);
        compute(B1, X1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c + 2 < nchunk) {
        loadx(X1, c + 2);
        copy(B1, c + 2);
        wait_vm<COPIES>();
        __builtin_amdgcn_sched_barrier(0);
        compute(B0, X0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<0>();
        __builtin_amdgcn_sched_barrier(0);
        compute(B1, X1);
      } else {
        wait_vm<0>();
        __builtin_amdgcn_sched_barrier(0);
        compute(B0, X0);
      }
    } else {
      plain_steps();
    }
  } else if constexpr (MT == 1) {
    // Two chunks in flight per wave (16-row token tiles, the decode shapes):
    // chunk c+1's loads are issued before chunk c's MFMAs, so a wave waits
    // one memory latency per chunk pair instead of per chunk (gate/up 1.7%
    // faster at T = 64; the wider tiles keep one chunk in flight, as their
    // registers would double).  The MFMAs keep the chunk order.
    struct Step {
      Frag fg[GW], fu[GW], fx[MT];
      float sx[MT], swg, swu;
    };
    auto load_step = [&](Step &s, int c) {
      const int64_t kb = (int64_t)c * 128;
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        if constexpr (T16) {   // chunk c of all 2I rows: c * 2I * 128 bytes in
          s.fg[i] = load_frag_t16(wg[i] + (int64_t)c * 2 * I * 128);
          s.fu[i] = load_frag_t16(wu[i] + (int64_t)c * 2 * I * 128);
        } else {
          s.fg[i] = load_frag(wg[i] + kb);
          s.fu[i] = load_frag(wu[i] + kb);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        s.fx[m] = xv[m] ? load_frag(xr[m] + kb) : zf;
        s.sx[m] = (FP8 && xv[m]) ? G.xs[(int64_t)xrow[m] * KB + c] : 0.f;
      }
      s.swg = FP8 ? sg[c] : 0.f;
      s.swu = FP8 ? su[c] : 0.f;
    };
    auto mma_step = [&](const Step &s) {
#pragma unroll
      for (int i = 0; i < GW; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          ag[i][m] = chunk_mma<FP8>(s.fg[i], s.fx[m], ag[i][m], s.swg * s.sx[m]);
          au[i][m] = chunk_mma<FP8>(s.fu[i], s.fx[m], au[i][m], s.swu * s.sx[m]);
        }
    };
    const int c_lo = SPLIT ? (int)((int64_t)nchunk * z / S) : 0;         // non-empty: nchunk >= S
    const int c_hi = SPLIT ? (int)((int64_t)nchunk * (z + 1) / S) : nchunk;
    Step s0, s1;
    load_step(s0, c_lo);
    int c = c_lo;
    for (; c + 2 < c_hi; c += 2) {
      load_step(s1, c + 1);
      mma_step(s0);
      load_step(s0, c + 2);
      mma_step(s1);
    }
    if (c + 1 < c_hi) {
      load_step(s1, c + 1);
      mma_step(s0);
      mma_step(s1);
    } else {
      mma_step(s0);
    }
  } else {
    for (int c = 0; c < nchunk; ++c) {
      const int64_t kb = (int64_t)c * 128;
      Frag fg[GW], fu[GW], fx[MT];
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        if constexpr (T16) {   // chunk c of all 2I rows: c * 2I * 128 bytes in
          fg[i] = load_frag_t16(wg[i] + (int64_t)c * 2 * I * 128);
          fu[i] = load_frag_t16(wu[i] + (int64_t)c * 2 * I * 128);
        } else {
          fg[i] = load_frag(wg[i] + kb);
          fu[i] = load_frag(wu[i] + kb);
        }
      }
      float sx[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        fx[m] = xv[m] ? load_frag(xr[m] + kb) : zf;
        sx[m] = (FP8 && xv[m]) ? G.xs[(int64_t)xrow[m] * KB + c] : 0.f;
      }
      const float swg = FP8 ? sg[c] : 0.f;
      const float swu = FP8 ? su[c] : 0.f;
#pragma unroll
      for (int i = 0; i < GW; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          ag[i][m] = chunk_mma<FP8>(fg[i], fx[m], ag[i][m], swg * sx[m]);
          au[i][m] = chunk_mma<FP8>(fu[i], fx[m], au[i][m], swu * sx[m]);
        }
    }
  }

  if constexpr (SPLIT) {   // raw sums of this K range; rows of the one tile
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int col = hc0 + 16 * i + 4 * (lane >> 4);
      if (!xv[0]) continue;
      float *p = spart + ((int64_t)z * 16 + (xrow[0] - rbeg)) * 2 * I + col;
      *reinterpret_cast<f32x4 *>(p) = ag[i][0];
      *reinterpret_cast<f32x4 *>(p + I) = au[i][0];
    }
    return;
  }
  // Epilogue: lane holds columns hc0 + 16i + 4*(lane/16) + r of token row xrow[m].
  float hv[GW][MT][4];
#pragma unroll
  for (int i = 0; i < GW; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[i][m][r] = swiglu(ag[i][m][r], au[i][m][r]);

  if constexpr (!FP8) {
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int col = hc0 + 16 * i + 4 * (lane >> 4);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (!xv[m]) continue;
        const uint32_t lo = pack_bf16x2(hv[i][m][0], hv[i][m][1]);
        const uint32_t hi = pack_bf16x2(hv[i][m][2], hv[i][m][3]);
        *reinterpret_cast<uint2 *>(G.h + ((int64_t)xrow[m] * I + col) * 2) = make_uint2(lo, hi);
        if (G.z) {   // pre-activations kept for a backward
          float *zr = G.z + (int64_t)xrow[m] * 2 * I + col;
          *reinterpret_cast<f32x4 *>(zr) = ag[i][m];
          *reinterpret_cast<f32x4 *>(zr + I) = au[i][m];
        }
      }
    }
  } else {
    // 1x128 group of h = the workgroup's 128 columns (GW == 2): amax over the
    // lane's 8 values, the 4 lanes sharing the token, then the 4 waves.
    __shared__ float red[4][16 * MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < GW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) am = __builtin_fmaxf(am, __builtin_fabsf(hv[i][m][r]));
      am = __builtin_fmaxf(am, __shfl_xor(am, 16, kWave));
      am = __builtin_fmaxf(am, __shfl_xor(am, 32, kWave));
      if (lane < 16) red[w][16 * m + lane] = am;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int tl = 16 * m + (lane & 15);
      const float am = __builtin_fmaxf(__builtin_fmaxf(red[0][tl], red[1][tl]),
                                       __builtin_fmaxf(red[2][tl], red[3][tl]));
      const float s = group_scale(am);
      if (!xv[m]) continue;
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        const int col = hc0 + 16 * i + 4 * (lane >> 4);
        const uint32_t q = quant4_e4m3(hv[i][m][0], hv[i][m][1], hv[i][m][2], hv[i][m][3], s);
        *reinterpret_cast<uint32_t *>(G.h + (int64_t)xrow[m] * I + col) = q;
      }
      if (w == 0 && lane < 16) G.hs[(int64_t)xrow[m] * (I / 128) + blockIdx.x] = s;
    }
  }
}

// MXK: the launch's e4m3 group carries MX FP4 weights.  The MX bodies are
// instantiated only there, so the bf16/fp8 kernels keep their register budget.
template <int MT, int GW, bool MXK>
__global__ __launch_bounds__(256) void gate_up_stream_kernel(StreamArgs a) {
  if ((int)blockIdx.y >= a.ntiles[0]) return;
  const TileEntry te = a.tiles[blockIdx.y];
  const FfnGroup G = pick_group(a.g0, a.g1, te.ge >> 24);
  if ((int)blockIdx.x * 64 * GW >= G.I) return;     // group narrower than the grid
  if constexpr (MT == 1 && GW == 2) {
    if (a.ssplit > 1 && (te.ge >> 24) == a.sgroup) {   // the split group's one tile: a K range per blockIdx.z
      gate_up_body<false, false, 1, 2, false, true>(G, te, a.H, (int)blockIdx.z, a.ssplit, a.spart);
      return;
    }
  }
  if (blockIdx.z > 0) return;                       // the other tiles run once
  if (G.fp8) {
    if constexpr (GW == 2) {
      if constexpr (!MXK) {
        if (G.tile16) {
          gate_up_body<true, false, MT, GW, true>(G, te, a.H);
          return;
        }
      }
      gate_up_body<true, MXK, MT, GW>(G, te, a.H);
    }
  } else if (G.tile16) {
    gate_up_body<false, false, MT, GW, true>(G, te, a.H);
  } else {
    gate_up_body<false, false, MT, GW>(G, te, a.H);
  }
}

// ---------------------------------------------------------------- down (streaming)
// Workgroup: 4 waves x NW 16-column output tiles = 64*NW columns, 16*MT rows.
template <bool FP8, bool MX, int MT, int NW, bool T16 = false>
__device__ __forceinline__ void down_body(const FfnGroup &G, const TileEntry &te, int H) {
  static_assert(FP8 || !MX, "MX weights take e4m3 activations");
  static_assert(!(MX && T16), "MX weights are row-major");
  constexpr int ESZ = FP8 ? 1 : 2;
  const int lane = lane_id(), w = wave_id();
  int rbeg, rend;
  tile_rows(G, te, rbeg, rend);
  const int e = te.ge & 0xFFFFFF;
  const int I = G.I;
  const int64_t hrowb = (int64_t)I * ESZ;             // h row bytes
  const int64_t wrowb = MX ? (int64_t)I / 2 : hrowb;  // weight row bytes
  const int c0 = blockIdx.x * (64 * NW) + w * (16 * NW);
  const int g4 = lane >> 4;
  const int koff = MX ? 16 * g4 : 32 * g4;
  const uint8_t *wbase = G.wd + (int64_t)e * H * wrowb;
  const uint8_t *wr[NW];
  const uint8_t *mr[NW];   // MX: the lane's row of E8M0 scale bytes
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int64_t r = c0 + 16 * i + (lane & 15);
    if constexpr (T16)
      wr[i] = wbase + ((int64_t)(c0 + 16 * i) >> 4) * 2048 + 16 * lane;
    else
      wr[i] = wbase + r * wrowb + koff;
    if constexpr (MX) mr[i] = G.md + ((int64_t)e * H + r) * (I / 32);
  }
  const uint8_t *hr[MT];
  bool hv[MT];
  int hrow[MT], hsrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    hrow[m] = rbeg + 16 * m + (lane & 15);
    hv[m] = hrow[m] < rend;
    hsrow[m] = hv[m] ? hrow[m] : (rbeg < rend ? rbeg : 0);   // a row that exists
    hr[m] = G.h + (int64_t)hsrow[m] * hrowb + koff;
  }
  f32x4 acc[NW][MT];
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[i][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nchunk = (int)(hrowb / 128);
  const int KB = I / 128;
  const Frag zf = Frag{i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};
  if constexpr (MX) {
    // Fallback for shapes the staged loop below does not take (see gate/up).
    auto plain_steps = [&]() {
      for (int c = 0; c < nchunk; c += 2) {
        const int nv = min(2, nchunk - c);
        i32x4 fw[2][NW];
        uint32_t sww[2][NW];
        Frag fh[2][MT];
        float sh[2][MT];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int cj = j < nv ? c + j : c;   // a lone last chunk is loaded twice, counted once
#pragma unroll
          for (int i = 0; i < NW; ++i) {
            fw[j][i] = load16(wr[i] + (int64_t)cj * 64);
            sww[j][i] = *reinterpret_cast<const uint32_t *>(mr[i] + 4 * cj);
          }
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            // branch-free: rows past the tile read a valid row and are zeroed after
            const Frag f = load_frag_k64(hr[m] + (int64_t)cj * 128);
            const float sv = G.hs[(int64_t)hsrow[m] * KB + cj];
            fh[j][m] = hv[m] ? f : zf;
            sh[j][m] = hv[m] ? sv : 0.f;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (j >= nv) break;
#pragma unroll
          for (int i = 0; i < NW; ++i) {
            const int sa = (int)((sww[j][i] >> (8 * g4)) & 0xFFu);
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[i][m] = chunk_mma_mx(fw[j][i], fh[j][m], sa, acc[i][m], sh[j][m]);
          }
        }
      }
    };
    if (MT <= 2 && (nchunk & 1) == 0) {
      // Weight codes through LDS, as in the gate/up kernel: each copy
      // instruction moves 8 rows x one whole 128-byte line; two 4 KB buffers
      // per wave, private to it.
      __shared__ __attribute__((aligned(16))) uint8_t wlds0[4][NW][2048];
      __shared__ __attribute__((aligned(16))) uint8_t wlds1[4][NW][2048];
      const uint8_t *tb[NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) tb[i] = wbase + (int64_t)(c0 + 16 * i) * wrowb;
      const int sr = lane >> 3;
      const uint32_t coff0 = (uint32_t)(sr * wrowb + 16 * ((lane & 7) ^ sr));
      const uint32_t coff1 = coff0 + (uint32_t)(8 * wrowb);
      auto copy = [&](uint8_t *buf, int c) {
#pragma unroll
        for (int t = 0; t < NW; ++t) {
          const uint8_t *src = tb[t] + (int64_t)c * 64;
          dma16_stream(src + coff0, buf + t * 2048);
          dma16_stream(src + coff1, buf + t * 2048 + 1024);
        }
      };
      struct XB {
        uint2 s[NW];
        Frag h[2][MT];
        float sh[2][MT];
      };
      auto loadx = [&](XB &b, int c) {
#pragma unroll
        for (int i = 0; i < NW; ++i) b.s[i] = *reinterpret_cast<const uint2 *>(mr[i] + 4 * c);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            b.h[j][m] = load_frag_k64(hr[m] + (int64_t)(c + j) * 128);
            b.sh[j][m] = G.hs[(int64_t)hsrow[m] * KB + c + j];
          }
      };
      const int rho = lane & 15;
      static_assert(NW == 2, "the staged MX down path reads 2 x 2 tiles");
      auto compute = [&](const uint8_t *buf, const XB &b) {
        i32x4 fr[4];
        lds_read_2x2(lds_addr(buf + rho * 128 + 16 * ((0 + g4) ^ (rho & 7))),
                     lds_addr(buf + rho * 128 + 16 * ((4 + g4) ^ (rho & 7))), fr);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < NW; ++i) {
            const i32x4 fw = fr[2 * j + i];
            const int sa = (int)(((j ? b.s[i].y : b.s[i].x) >> (8 * g4)) & 0xFFu);
#pragma unroll
            for (int m = 0; m < MT; ++m)
              acc[i][m] = chunk_mma_mx(fw, b.h[j][m], sa, acc[i][m], hv[m] ? b.sh[j][m] : 0.f);
          }
      };
      uint8_t *const B0 = &wlds0[w][0][0];
      uint8_t *const B1 = &wlds1[w][0][0];
      constexpr int COPIES = 2 * NW;
      XB X0, X1;
      loadx(X0, 0);
      copy(B0, 0);
      // the token loads of the first step done before the loop, as they are
      // on the way round it (a loop-carried load still in flight on one path
      // makes the compiler wait for everything at the top of the loop)
      wait_vm<COPIES>();
      int c = 0;
      for (; c + 4 < nchunk; c += 4) {
        loadx(X1, c + 2);
        copy(B1, c + 2);
        wait_vm<COPIES>();
        __builtin_amdgcn_sched_barrier(0);
        compute(B0, X0);
        __builtin_amdgcn_sched_barrier(0);
        loadx(X0, c + 4);
        copy(B0, c + 4);
        wait_vm<COPIES>();
        __builtin_amdgcn_sched_barrier(0);
        compute(B1, X1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c + 2 < nchunk) {
        loadx(X1, c + 2);
        copy(B1, c + 2);
        wait_vm<COPIES>();
        __builtin_amdgcn_sched_barrier(0);
        compute(B0, X0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<0>();
        __builtin_amdgcn_sched_barrier(0);
        compute(B1, X1);
      } else {
        wait_vm<0>();
        __builtin_amdgcn_sched_barrier(0);
        compute(B0, X0);
      }
    } else {
      plain_steps();
    }
  } else if constexpr (MT == 1) {
    // two chunks in flight per wave, as in the gate/up body (16-row tiles)
    struct Step {
      Frag fw[NW], fh[MT];
      float sw[NW], sh[MT];
    };
    auto load_step = [&](Step &s, int c) {
      const int64_t kb = (int64_t)c * 128;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        s.fw[i] = T16 ? load_frag_t16(wr[i] + (int64_t)c * H * 128) : load_frag(wr[i] + kb);   // H rows per chunk
        s.sw[i] = FP8 ? G.sd[((int64_t)e * (H / 128) + (c0 + 16 * i) / 128) * KB + c] : 0.f;
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        s.fh[m] = hv[m] ? load_frag(hr[m] + kb) : zf;
        s.sh[m] = (FP8 && hv[m]) ? G.hs[(int64_t)hrow[m] * KB + c] : 0.f;
      }
    };
    auto mma_step = [&](const Step &s) {
#pragma unroll
      for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[i][m] = chunk_mma<FP8>(s.fw[i], s.fh[m], acc[i][m], s.sw[i] * s.sh[m]);
    };
    Step s0, s1;
    load_step(s0, 0);
    int c = 0;
    for (; c + 2 < nchunk; c += 2) {
      load_step(s1, c + 1);
      mma_step(s0);
      load_step(s0, c + 2);
      mma_step(s1);
    }
    if (c + 1 < nchunk) {
      load_step(s1, c + 1);
      mma_step(s0);
      mma_step(s1);
    } else {
      mma_step(s0);
    }
  } else {
    for (int c = 0; c < nchunk; ++c) {
      const int64_t kb = (int64_t)c * 128;
      Frag fw[NW], fh[MT];
      float sw[NW], sh[MT];
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        fw[i] = T16 ? load_frag_t16(wr[i] + (int64_t)c * H * 128) : load_frag(wr[i] + kb);   // H rows per chunk
        sw[i] = FP8 ? G.sd[((int64_t)e * (H / 128) + (c0 + 16 * i) / 128) * KB + c] : 0.f;
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        fh[m] = hv[m] ? load_frag(hr[m] + kb) : zf;
        sh[m] = (FP8 && hv[m]) ? G.hs[(int64_t)hrow[m] * KB + c] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[i][m] = chunk_mma<FP8>(fw[i], fh[m], acc[i][m], sw[i] * sh[m]);
    }
  }
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int col = c0 + 16 * i + 4 * (lane >> 4);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (!hv[m]) continue;
      const int64_t o = (int64_t)hrow[m] * H + col;
      if (G.y_f32) {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(G.y) + o) = acc[i][m];
      } else {
        const uint32_t lo = pack_bf16x2(acc[i][m][0], acc[i][m][1]);
        const uint32_t hi = pack_bf16x2(acc[i][m][2], acc[i][m][3]);
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(G.y) + o) = make_uint2(lo, hi);
      }
    }
  }
}

template <int MT, int NW, bool MXK>
__global__ __launch_bounds__(256) void down_stream_kernel(StreamArgs a) {
  if ((int)blockIdx.y >= a.ntiles[0]) return;
  const TileEntry te = a.tiles[blockIdx.y];
  const FfnGroup G = pick_group(a.g0, a.g1, te.ge >> 24);
  if (G.fp8) {
    if constexpr (!MXK) {
      if (G.tile16) {
        down_body<true, false, MT, NW, true>(G, te, a.H);
        return;
      }
    }
    down_body<true, MXK, MT, NW>(G, te, a.H);
  } else if (G.tile16) {
    down_body<false, false, MT, NW, true>(G, te, a.H);
  } else {
    down_body<false, false, MT, NW>(G, te, a.H);
  }
}

// ---------------------------------------------------------------- host side

FfnPlan ffn_plan(const FfnGroup *g, int ngroups, int H) {
  FfnPlan p;
  int64_t rows = 0, experts = 0;
  bool all128 = true;
  for (int i = 0; i < ngroups; ++i) {
    rows += g[i].nrows;
    experts += g[i].E;
    all128 = all128 && (g[i].I % 128 == 0);
  }
  // token-tile height from the mean rows per expert of the group with the most
  // experts (the routed experts when the shared expert rides along)
  int big = 0;
  for (int i = 1; i < ngroups; ++i)
    if (g[i].E > g[big].E) big = i;
  const double avg = g[big].E > 0 ? (double)g[big].nrows / g[big].E : 0.0;
  p.mt = avg <= 16 ? 1 : (avg <= 32 ? 2 : 4);
  p.gw = all128 ? 2 : 1;
  // many rows per expert: the LDS-tiled kernels (weights reused across 128 tokens)
  // MX weights: their own tiled kernels (64-row token tiles, H and I multiples of 256)
  bool any_mx = false, mx_ok = true;
  for (int i = 0; i < ngroups; ++i)
    if (g[i].mx) {
      any_mx = true;
      mx_ok = mx_ok && tiled_mx_supported(g[i], H);
    }
  // (measured crossover on the Step-5 layer, one MI355X: with 10 or more
  // rows per expert on average the tiled kernels are faster, by 8% at 11.6
  // rows and 30% at 46.5 for fp8 and bf16 experts; MX FP4 from 12 rows, where
  // the two tie; below that the streaming kernels win, by up to 12% at 8.7)
  const double tiled_min = any_mx ? 12.0 : 10.0;
  p.tiled = (all128 && H % 256 == 0 && mx_ok && g[0].nrows > 0 && avg >= tiled_min) ? 1 : 0;
  // 256-row token tiles (a weight tile then feeds all of an expert's rows
  // from a single fetch) from 128 rows per expert with bf16 weights, from 96
  // with fp8 and from 48 with MX FP4, whose 64-row tiles below that fetch
  // each weight tile once per 64 rows (measured on the Step-5 layer: at 70
  // rows per expert the wide MX kernel is 25% faster, at 116 the wide fp8
  // one 9%; wide bf16 items lose below 128); below, 128-row tiles (MX: 64)
  const double wide_min = any_mx ? 48.0 : (g[big].fp8 ? 96.0 : 128.0);
  p.bm = p.tiled ? (avg >= wide_min ? 256 : (any_mx ? 64 : 128)) : 16 * p.mt;
  int64_t cap = 1;
  for (int i = 0; i < ngroups; ++i) cap += cdiv(g[i].nrows, p.bm) + std::min<int64_t>(g[i].nrows, g[i].E);
  p.max_tiles = (int)cap;
  // A few tokens: the shared expert's gate/up (one bf16 expert, one 16-row
  // tile) would leave each of its workgroups 512 H bytes of weights to stream
  // alone (2 MB at H = 4096; measured: without it the Step-5 layer at T = 1
  // takes 62 instead of 107 us), so its K is split four ways.  Measured on the
  // Step-5 layer: with fp8 experts 17, 13 and 12% faster at T = 1, 2, 4 (4%
  // slower at 8), with MX FP4 21, 21, 22 and 6% at T = 1, 2, 4, 8; with bf16
  // experts no gain (their own 2 MB workgroups set the launch), so no split.
  // Eight ways for one or two tokens, four above.
  p.ssplit = 1;
  p.sgroup = 0;
  p.spart_floats = 0;
  if (!p.tiled && p.mt == 1 && p.gw == 2 && ngroups == 2 && H >= 1024) {
    for (int i = 0; i < 2; ++i) {
      const FfnGroup &s = g[i];
      const FfnGroup &r = g[1 - i];
      const int rows_max = r.mx ? 8 : (r.fp8 ? 4 : 0);
      if (s.E == 1 && !s.fp8 && !s.mx && !s.tile16 && s.z == nullptr && s.nrows > 0 && s.nrows <= rows_max &&
          r.E > 1) {
        p.ssplit = s.nrows <= 2 ? 8 : 4;   // 8: 5-7% faster than 4 at T = 1, 2; 2-3% slower at 4, 8
        p.sgroup = i;
        p.spart_floats = (int64_t)p.ssplit * 16 * 2 * s.I;
        break;
      }
    }
  }
  (void)rows;
  (void)experts;
  return p;
}

size_t ffn_tiles_bytes(const FfnPlan &p) {
  return align_up(sizeof(TileEntry) * (size_t)p.max_tiles + kTileHdrWords * sizeof(int32_t), 256) +
         align_up(sizeof(float) * (size_t)p.spart_floats, 256);
}

// The split partial sums sit after the tile list in the same workspace.
static float *split_partials(int32_t *tiles_ws, const FfnPlan &p) {
  if (p.ssplit <= 1) return nullptr;
  return reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(tiles_ws) +
                                   align_up(sizeof(TileEntry) * (size_t)p.max_tiles + kTileHdrWords * sizeof(int32_t), 256));
}

// The split group's h: the ssplit partial sums of each pre-activation added
// in split order (z = 0 first), SwiGLU, rounded to bf16 as in the epilogue.
__global__ __launch_bounds__(256) void split_finish_kernel(FfnGroup G, const float *__restrict__ spart, int S) {
  const int I = G.I;
  const int64_t total = (int64_t)G.nrows * I;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int r = (int)(i / I), c = (int)(i % I);
    float g = 0.f, u = 0.f;
    for (int z = 0; z < S; ++z) {
      const float *p = spart + ((int64_t)z * 16 + r) * 2 * I;
      g += p[c];
      u += p[I + c];
    }
    reinterpret_cast<uint16_t *>(G.h)[(int64_t)r * I + c] = (uint16_t)f32_to_bf16(swiglu(g, u));
  }
}

template <int MT, bool MXK>
static void run_stream(const StreamArgs &a, const FfnPlan &plan, int maxI, int site, hipStream_t st) {
  timing_before(site, st);
  if (plan.gw == 2) {
    dim3 g1((unsigned)cdiv(maxI, 128), (unsigned)plan.max_tiles, (unsigned)(MT == 1 ? a.ssplit : 1));
    gate_up_stream_kernel<MT, 2, MXK><<<g1, 256, 0, st>>>(a);
    if (MT == 1 && a.ssplit > 1) {
      const FfnGroup &gs = a.sgroup ? a.g1 : a.g0;
      split_finish_kernel<<<(unsigned)cdiv((int64_t)gs.nrows * gs.I, 256), 256, 0, st>>>(gs, a.spart, a.ssplit);
    }
  } else {
    dim3 g1((unsigned)cdiv(maxI, 64), (unsigned)plan.max_tiles);
    gate_up_stream_kernel<MT, 1, false><<<g1, 256, 0, st>>>(a);
  }
  timing_after(site, st);
  dim3 g2((unsigned)(a.H / 128), (unsigned)plan.max_tiles);
  timing_before(site + 1, st);
  down_stream_kernel<MT, 2, MXK><<<g2, 256, 0, st>>>(a);
  timing_after(site + 1, st);
}

hipError_t launch_expert_ffn(const FfnGroup *g, int ngroups, int H, const FfnPlan &plan, int32_t *tiles_ws,
                             int site, hipStream_t st, bool tiles_ready) {
  if (ngroups < 1 || ngroups > kMaxGroups) return hipErrorInvalidValue;
  int64_t rows = 0;
  int maxI = 0;
  bool mx = false, fp8_plain = false;
  for (int i = 0; i < ngroups; ++i) {
    rows += g[i].nrows;
    maxI = std::max(maxI, (int)g[i].I);
    if (g[i].fp8 && plan.gw != 2) return hipErrorInvalidValue;
    if (g[i].mx && !g[i].fp8) return hipErrorInvalidValue;
    mx = mx || g[i].mx;
    fp8_plain = fp8_plain || (g[i].fp8 && !g[i].mx);
  }
  // one launch holds either MX or block-scaled fp8 weights (plus bf16 groups)
  if (mx && fp8_plain) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  int32_t *hdr = tiles_ws;
  TileEntry *tiles = reinterpret_cast<TileEntry *>(tiles_ws + kTileHdrWords);
  StreamArgs a{g[0], ngroups > 1 ? g[1] : g[0], tiles, hdr, H, plan.ssplit, plan.sgroup, split_partials(tiles_ws, plan)};
  if (plan.tiled && mx && plan.bm == 256) {
    // MX and bf16 groups together, 256-row tiles
    if (!tiles_ready) build_tiles_kernel<<<1, 1024, 0, st>>>(a.g0, a.g1, ngroups, plan.bm, plan.max_tiles, tiles, hdr);
    return launch_wide_mx_ffn(g, ngroups, H, tiles, hdr, num_compute_units(), site, st);
  }
  if (plan.tiled && mx) {
    // MX tiles are 64 token rows, the other groups' 128: each group gets its
    // own tile list and launches, one after the other on the stream.
    for (int i = 0; i < ngroups; ++i) {
      if (g[i].nrows == 0) continue;
      build_tiles_kernel<<<1, 1024, 0, st>>>(g[i], g[i], 1, g[i].mx ? 64 : 128, plan.max_tiles, tiles, hdr);
      const hipError_t e = g[i].mx ? launch_tiled_mx_ffn(g[i], H, tiles, hdr, num_compute_units(), site, st)
                                   : launch_tiled_ffn(&g[i], 1, H, tiles, hdr, num_compute_units(), 128, site, st);
      if (e != hipSuccess) return e;
    }
    return hipGetLastError();
  }
  if (!tiles_ready) build_tiles_kernel<<<1, 1024, 0, st>>>(a.g0, a.g1, ngroups, plan.bm, plan.max_tiles, tiles, hdr);
  if (plan.tiled) {
    if (H % 256 != 0) return hipErrorInvalidValue;
    return launch_tiled_ffn(g, ngroups, H, tiles, hdr, num_compute_units(), plan.bm, site, st);
  }
  switch (plan.mt * 2 + (mx ? 1 : 0)) {
    case 2: run_stream<1, false>(a, plan, maxI, site, st); break;
    case 4: run_stream<2, false>(a, plan, maxI, site, st); break;
    case 8: run_stream<4, false>(a, plan, maxI, site, st); break;
    case 3: run_stream<1, true>(a, plan, maxI, site, st); break;
    case 5: run_stream<2, true>(a, plan, maxI, site, st); break;
    case 9: run_stream<4, true>(a, plan, maxI, site, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
