// expert_gemm_tiled_mx.hip -- LDS-tiled grouped expert GEMMs for MX FP4
// weights (E2M1 codes, one E8M0 scale per 32 inputs of a row) at large token
// counts: gate/up with the fused SwiGLU epilogue and e4m3 h, then down.
//
// The same organisation as the fp8/bf16 tiled kernels (expert_gemm_tiled.hip),
// re-cut for 4-bit weights:
//   - a stage covers 256 inputs (two 128-input chunks), so a weight row's
//     stage is one whole 128-byte line of codes; a workgroup tile is 256
//     weight rows x 64 token rows, which keeps the bytes per MFMA of the fp8
//     tile (32 KB of codes + 16 KB of e4m3 token rows per stage, 32 scaled
//     MFMAs per wave) and halves the padding of an expert's last token tile;
//   - each stage also brings the rows' E8M0 bytes (8 per row) and the token
//     rows' two fp32 group scales; the E8M0 byte of a lane's row and 32-input
//     block goes to the scaled MFMA as its A scale, the token scale multiplies
//     the chunk product (1x128 groups, as in fp8 mode);
//   - 4 waves = 2 (weight halves of 128 rows) x 2 (token halves, interleaved
//     16-row slices wm and wm+2); a wave owns 8 x 2 MFMA tiles of 16x16;
//   - three-stage ring of direct-to-LDS copies (8 rows x 128 bytes, or 4 rows x
//     256 bytes, per instruction), 16-byte columns XOR-swizzled by row % 8;
//   - persistent, one workgroup per CU, items split over the 8 XCDs by cost
//     and taken in bands of up to 8 token tiles of one expert.
// Fragment K order: the fp4 A operand gives lane group g inputs 32g..32g+31
// of the chunk (the stored packing); the e4m3 B operand is read in the
// instruction's order, inputs 16g..16g+15 and 64+16g..64+16g+15.

#include <algorithm>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {
constexpr int XBN = 256;                   // weight rows per work item
constexpr int XBM = 64;                    // token rows per work item
constexpr int XW = XBN * 128;              // weight codes per stage (256 inputs per row)
constexpr int XT = XBM * 256;              // token codes per stage
constexpr int XTS = XBM * 16;              // token scales per stage: per row (chunk 0, chunk 1) twice
constexpr int XWS = XBN * 8;               // weight E8M0 bytes per stage: 8 per row
constexpr int XSTAGE = XW + XT + XTS + XWS;
constexpr int XNSTAGE = 3;
constexpr int XTHREADS = 256;
constexpr int XBAND = 8;
constexpr int XPS = 15;                    // vector memory instructions per wave per stage

struct MxTiledArgs {
  FfnGroup g;
  const TileEntry *tiles;
  const int32_t *hdr;     // [0] tile count
  int H;
  int nt;                 // column tiles per tile-list slot
};
}  // namespace

template <bool GATEUP>
struct MxItem {
  const FfnGroup &G;
  int e, rbeg, rend, nvalid, I, K, nstage, col0, ntile, H, KB;
  int64_t wrowb, xrowb, srowb;
  const uint8_t *wsrc, *ssrc, *asrc;
  const float *ascale;
  int lane, w, wn, wm, g4;
  uint32_t woff[8], xoff[4], soff, wsoff[2];

  __device__ MxItem(const FfnGroup &g, const TileEntry &te, int nt_, int H_) : G(g), ntile(nt_), H(H_) {
    lane = threadIdx.x & 63;
    w = uniform(threadIdx.x >> 6);
    wn = w & 1;
    wm = w >> 1;
    g4 = lane >> 4;
    e = te.ge & 0xFFFFFF;
    rend = min(max(group_off(G, e + 1), 0), G.nrows);
    rbeg = min(max(group_off(G, e), 0) + te.m0, rend);
    nvalid = min(rend - rbeg, XBM);
    I = G.I;
    K = GATEUP ? H : I;
    wrowb = K / 2;
    xrowb = K;
    srowb = K / 32;
    nstage = K / 256;
    KB = K / 128;
    col0 = GATEUP ? ntile * 128 : ntile * XBN;
    const int64_t wrows = GATEUP ? 2 * (int64_t)I : (int64_t)H;
    wsrc = (GATEUP ? G.wgu : G.wd) + (int64_t)e * wrows * wrowb;
    ssrc = (GATEUP ? G.mgu : G.md) + (int64_t)e * wrows * srowb;
    const bool indirect = GATEUP && G.xsrc != nullptr;
    asrc = (GATEUP ? G.x : G.h) + (indirect ? 0 : (int64_t)rbeg * xrowb);
    ascale = (GATEUP ? G.xs : G.hs) + (indirect ? 0 : (int64_t)rbeg * KB);
    auto wrow = [&](int r) { return GATEUP ? (r < 128 ? col0 + r : I + col0 + r - 128) : col0 + r; };
    auto xrow = [&](int r) -> int64_t {   // rows past the end repeat a valid row
      const int rr = min(r, nvalid - 1);
      return indirect ? G.xsrc[rbeg + rr] / G.xdiv : rr;
    };
    // weight codes: instruction q of wave w copies rows 8(w+4q)..+7, lane = (row, 16-byte slot)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = 8 * (w + 4 * q) + (lane >> 3);
      const int c = (lane & 7) ^ swz_f(r);
      woff[q] = (uint32_t)(wrow(r) * wrowb + c * 16);
    }
    // token codes: instruction q of wave w copies rows 4(w+4q)..+3 of 256 bytes
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 4 * (w + 4 * q) + (lane >> 4);
      const int c = (lane & 15) ^ swz_f(r);
      xoff[q] = (uint32_t)(xrow(r) * xrowb + c * 16);
    }
    // token scales: wave w copies rows 16w..16w+15, 4 words per row (chunk 0, 1, 0, 1)
    soff = (uint32_t)(xrow(16 * w + (lane >> 2)) * KB * 4 + (lane & 1) * 4);
    // weight E8M0 bytes: instruction q of wave w copies rows 32(2w+q)..+31, 2 words per row
#pragma unroll
    for (int q = 0; q < 2; ++q) wsoff[q] = (uint32_t)(wrow(32 * (2 * w + q) + (lane >> 1)) * srowb + (lane & 1) * 4);
  }

  // Direct-to-LDS copies of stage s (inputs 256s..256s+255) into buffer sb.
  __device__ __forceinline__ void issue(int s, uint8_t *sb) const {
    const uint8_t *wb = wsrc + (int64_t)s * 128;
    const uint8_t *xb = asrc + (int64_t)s * 256;
    const uint8_t *sxb = reinterpret_cast<const uint8_t *>(ascale + 2 * s);
    const uint8_t *swb = ssrc + (int64_t)s * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) dma16(wb + woff[q], sb + (w + 4 * q) * 1024);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(xb + xoff[q], sb + XW + (w + 4 * q) * 1024);
    dma4(sxb + soff, sb + XW + XT + 256 * w);
#pragma unroll
    for (int q = 0; q < 2; ++q) dma4(swb + wsoff[q], sb + XW + XT + XTS + 256 * (2 * w + q));
  }

  struct AFrags {
    i32x4 a0[8], a1[8];   // chunk 0 and chunk 1 codes of tile i
    uint2 ws[8];          // the row's 8 E8M0 bytes of the stage
  };
  template <int NJ>
  struct BFrags {
    i32x4 lo[2][NJ], hi[2][NJ];   // [chunk][slice]
    f32x2 sx[NJ];                 // token group scales of chunk 0 and chunk 1
  };

  __device__ __forceinline__ int arow(int i) const {
    return (GATEUP ? (i < 4 ? 64 * wn + 16 * i : 128 + 64 * wn + 16 * (i - 4)) : 128 * wn + 16 * i) + (lane & 15);
  }

  __device__ __forceinline__ void read_a(const uint8_t *sb, int i, AFrags &A) const {
    const int r = arow(i);
    A.a0[i] = *reinterpret_cast<const i32x4 *>(sb + r * 128 + 16 * (g4 ^ swz_f(r)));
    A.a1[i] = *reinterpret_cast<const i32x4 *>(sb + r * 128 + 16 * ((4 + g4) ^ swz_f(r)));
    A.ws[i] = *reinterpret_cast<const uint2 *>(sb + XW + XT + XTS + r * 8);
  }

  template <int NJ>
  __device__ __forceinline__ void read_b(const uint8_t *sb, BFrags<NJ> &F) const {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = 16 * (wm + 2 * j) + (lane & 15);
      const uint8_t *row = sb + XW + r * 256;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        F.lo[c][j] = *reinterpret_cast<const i32x4 *>(row + 16 * ((8 * c + g4) ^ swz_f(r)));
        F.hi[c][j] = *reinterpret_cast<const i32x4 *>(row + 16 * ((8 * c + 4 + g4) ^ swz_f(r)));
      }
      F.sx[j] = *reinterpret_cast<const f32x2 *>(sb + XW + XT + r * 16);
    }
  }

  // The stage's MFMAs; raw chunk products are folded into the accumulators
  // one MFMA behind, and tile i's A fragments are refilled from `next` right
  // after its last MFMA.
  template <int NJ>
  __device__ __forceinline__ void mma(AFrags &A, const BFrags<NJ> &F, const uint8_t *next,
                                      f32x4 (&acc)[8][2]) const {
    constexpr int NT = 8 * NJ * 2;
    f32x4 prev = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t <= NT; ++t) {
      f32x4 cur = {0.f, 0.f, 0.f, 0.f};
      if (t < NT) {
        const int i = t / (2 * NJ), j = (t / 2) % NJ, c = t % 2;
        const uint32_t word = c ? A.ws[i].y : A.ws[i].x;
        const int sa = (int)((word >> (8 * g4)) & 0xFFu);
        cur = mfma_mx(c ? A.a1[i] : A.a0[i], F.lo[c][j], F.hi[c][j], sa);
        if (j == NJ - 1 && c == 1) read_a(next, i, A);
      }
      if (t > 0) {
        const int i = (t - 1) / (2 * NJ), j = ((t - 1) / 2) % NJ, c = (t - 1) % 2;
        const float s = c ? F.sx[j][1] : F.sx[j][0];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(prev[r], s, acc[i][j][r]);
      }
      prev = cur;
    }
  }

  // One pipeline step: stage s's operands are in (A, Fcur).  Wait until
  // stage s+1 has landed (stage s+2 may still be in flight) and this wave's
  // reads of stage s are done, sync the workgroup (stage s's buffer is then
  // refilled with stage s+3), read stage s+1 into Fnext and run stage s.
  template <int NJ>
  __device__ __forceinline__ void step(int s, uint8_t *lds, AFrags &A, BFrags<NJ> &Fcur, BFrags<NJ> &Fnext,
                                       f32x4 (&acc)[8][2]) const {
    if (s + 2 < nstage)
      wait_vm_lgkm0<XPS>();
    else
      wait_vm_lgkm0<0>();
    wg_barrier();
    if (s + 3 < nstage) issue(s + 3, lds + ((s + 3) % XNSTAGE) * XSTAGE);
    // the last step reads its own buffer again (nothing is copied into it any more)
    const int sn = s + 1 < nstage ? s + 1 : s;
    const uint8_t *next = lds + (sn % XNSTAGE) * XSTAGE;
    read_b<NJ>(next, Fnext);
    mma<NJ>(A, Fcur, next, acc);
  }

  template <int NJ>
  __device__ __forceinline__ void mainloop(uint8_t *lds, f32x4 (&acc)[8][2]) const {
    issue(0, lds);
    if (nstage > 1) issue(1, lds + XSTAGE);
    if (nstage > 2) issue(2, lds + 2 * XSTAGE);
    if (nstage > 2)
      wait_vm<2 * XPS>();
    else if (nstage > 1)
      wait_vm<XPS>();
    else
      wait_vm<0>();
    wg_barrier();
    AFrags A;
    BFrags<NJ> F0, F1;
#pragma unroll
    for (int i = 0; i < 8; ++i) read_a(lds, i, A);
    read_b<NJ>(lds, F0);
    for (int s = 0; s < nstage; s += 2) {
      step<NJ>(s, lds, A, F0, F1, acc);
      if (s + 1 < nstage) step<NJ>(s + 1, lds, A, F1, F0, acc);
    }
  }
};

template <bool GATEUP>
__device__ __forceinline__ void mx_item(const FfnGroup &G, const TileEntry &te, int ntile, int H, uint8_t *lds,
                                        float *red) {
  MxItem<GATEUP> it(G, te, ntile, H);
  const int lane = it.lane, wn = it.wn, wm = it.wm;
  // active 16-row token slices of this wave: slice j covers rows 16*(wm + 2j)
  const int nact = uniform(it.nvalid <= 16 * wm ? 0 : min(2, (it.nvalid - 16 * wm + 31) / 32));
  f32x4 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nact == 2)
    it.template mainloop<2>(lds, acc);
  else
    it.template mainloop<1>(lds, acc);   // also for a wave with no rows: keeps the barrier count equal
  const int rbeg = it.rbeg, nvalid = it.nvalid, I = it.I, col0 = it.col0;
  int brow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) brow[j] = 16 * (wm + 2 * j);

  // ---- epilogue.  Lane holds rows 4*(lane/16)+r of weight tile i for token
  // slice j, token row = rbeg + brow[j] + lane%16.
  if constexpr (GATEUP) {
    float hv[4][2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[i][j][r] = swiglu(acc[i][j][r], acc[i + 4][j][r]);
    // amax over the tile's 128 h columns per token: lane (16 values), the 4
    // lanes of the token (xor 16, 32), then the two weight-half waves (LDS).
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) am = __builtin_fmaxf(am, __builtin_fabsf(hv[i][j][r]));
      am = __builtin_fmaxf(am, __shfl_xor(am, 16, kWave));
      am = __builtin_fmaxf(am, __shfl_xor(am, 32, kWave));
      if (lane < 16) red[wn * XBM + brow[j] + lane] = am;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tr = brow[j] + (lane & 15);
      const float s = group_scale(__builtin_fmaxf(red[tr], red[XBM + tr]));
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
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tr = brow[j] + (lane & 15);
      if (tr >= nvalid) continue;
      const int64_t row = rbeg + tr;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int col = col0 + 128 * wn + 16 * i + 4 * (lane >> 4);
        const int64_t o = row * H + col;
        if (G.y_f32) {
          *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(G.y) + o) = acc[i][j];
        } else {
          const uint32_t lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          const uint32_t hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
          *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(G.y) + o) = make_uint2(lo, hi);
        }
      }
    }
  }
  __syncthreads();   // the next work item reuses the LDS ring and the reduction area
}

// Work item L -> (tile-list slot, column tile): the slots of one expert in
// bands of up to XBAND token tiles, the items of a band column-tile-major.
__device__ __forceinline__ void mx_map_item(const MxTiledArgs &a, int L, int &slot, int &ntile) {
  const int s = L / a.nt;
  const TileEntry te = a.tiles[s];
  const int e = te.ge & 0xFFFFFF;
  const int r0 = min(max(group_off(a.g, e), 0), a.g.nrows);
  const int r1 = min(max(group_off(a.g, e + 1), r0), a.g.nrows);
  const int t = te.m0 / XBM, p = t % XBAND;
  const int band = min(XBAND, (r1 - r0 + XBM - 1) / XBM - (t - p));
  const int s0 = s - p, q = L - a.nt * s0;
  slot = s0 + q % max(band, 1);
  ntile = q / max(band, 1);
}

template <bool GATEUP>
__global__ __launch_bounds__(XTHREADS, 1) void tiled_mx_kernel(MxTiledArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float *red = reinterpret_cast<float *>(lds + XNSTAGE * XSTAGE);
  const int nslots = a.hdr[0];
  const int count = nslots * a.nt;
  // equal contiguous ranges per XCD (every item of this launch costs the same)
  const int xcd = blockIdx.x & 7, per = gridDim.x >> 3, slot0 = blockIdx.x >> 3;
  const int beg = (int)((int64_t)count * xcd / 8), end = (int)((int64_t)count * (xcd + 1) / 8);
  for (int L = beg + slot0; L < end; L += per) {
    int slot, ntile;
    mx_map_item(a, L, slot, ntile);
    if (slot < nslots) mx_item<GATEUP>(a.g, a.tiles[slot], ntile, a.H, lds, red);
  }
}

size_t tiled_mx_lds_bytes() { return XNSTAGE * XSTAGE + 2 * XBM * sizeof(float); }

bool tiled_mx_supported(const FfnGroup &g, int H) { return g.mx && H % 256 == 0 && g.I % 256 == 0; }

hipError_t launch_tiled_mx_ffn(const FfnGroup &g, int H, const void *tiles, int32_t *hdr, int num_cus, int site,
                               hipStream_t st) {
  if (!tiled_mx_supported(g, H)) return hipErrorInvalidValue;
  MxTiledArgs a{g, static_cast<const TileEntry *>(tiles), hdr, H, 0};
  const unsigned grid = (unsigned)(std::max(num_cus, 8) / 8 * 8);
  const size_t lds = tiled_mx_lds_bytes();
  static bool attr_set[64] = {};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    hipError_t e1 = hipFuncSetAttribute(reinterpret_cast<const void *>(&tiled_mx_kernel<true>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void *>(&tiled_mx_kernel<false>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e1 != hipSuccess) return e1;
    if (e2 != hipSuccess) return e2;
    attr_set[dev] = true;
  }
  a.nt = g.I / 128;
  timing_before(site, st);
  tiled_mx_kernel<true><<<grid, XTHREADS, lds, st>>>(a);
  timing_after(site, st);
  a.nt = H / XBN;
  timing_before(site + 1, st);
  tiled_mx_kernel<false><<<grid, XTHREADS, lds, st>>>(a);
  timing_after(site + 1, st);
  return hipGetLastError();
}

}  // namespace moe
