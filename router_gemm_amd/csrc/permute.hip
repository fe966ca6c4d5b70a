// permute.hip -- token-to-expert grouping: a deterministic stable counting
// sort (per-chunk histogram, exclusive scan, ordered scatter) and the row
// gather of x into expert order, with the per-token 1x128 FP8 quantisation
// fused into the gather.
//
// The grouping is one of the MoE primitives of "Step-5 minimal inference"
// (introduction; "Contents", kernel.py).  The order inside an expert segment
// is increasing assignment index, so the permutation is unique.
//
// Sort design: the N keys are cut into chunks of 512.  Kernel 1 sorts each
// chunk in LDS by (key, index) -- a bitonic network, total order, so the
// result does not depend on scheduling -- and writes per chunk the count of
// every bin plus each element's rank among equal keys of its chunk.  Kernel 2
// turns the [chunk][bin] counts into global bases (scan over chunks, then over
// bins).  Kernel 3 places every element at base[chunk][key] + rank.  Counts
// use no atomics, so every output is bit-for-bit reproducible.

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {
constexpr int CH = kSortChunk;   // elements per chunk
constexpr int SORT_THREADS = 256;
}

constexpr int SCAN_BLOCK = 256;         // bins per workgroup of the multi-workgroup scan
constexpr int64_t SINGLE_SCAN_BINS = 4096;

size_t sort_ws_words(int64_t N, int64_t nbins) {
  const int64_t nchunk = cdiv(N, CH);
  // chunk counts [nchunk][nbins+1], sorted keys/indices/ranks [nchunk*CH] x 3,
  // per-block totals of the multi-workgroup scan
  return (size_t)(nchunk * (nbins + 1) + 3 * nchunk * CH + cdiv(nbins, SCAN_BLOCK) + 1);
}

// Sort chunk `chunk` of the keys in LDS: sk[j] = (bin << 32 | i) ascending
// (bin nbins = dropped), start[j] = first position of sk[j]'s bin in the chunk.
__device__ __forceinline__ void sort_chunk_lds(const int32_t *__restrict__ keys, const int32_t *__restrict__ aux,
                                               int64_t aux_bound, int64_t N, int nbins, int64_t chunk,
                                               uint64_t *sk, int32_t *start) {
  const int tid = threadIdx.x;
  const int64_t base = chunk * CH;
  for (int j = tid; j < CH; j += SORT_THREADS) {
    const int64_t i = base + j;
    uint64_t v = ~0ull;  // padding sorts last
    if (i < N) {
      const int32_t key = keys[i];
      bool valid = key >= 0 && key < nbins;
      if (aux) {
        const int32_t a = aux[i];
        valid = valid && a >= 0 && a < aux_bound;
      }
      const uint32_t kk = valid ? (uint32_t)key : (uint32_t)nbins;  // bin nbins = dropped
      v = ((uint64_t)kk << 32) | (uint32_t)i;
    }
    sk[j] = v;
  }
  __syncthreads();
  // bitonic sort, ascending
  for (int size = 2; size <= CH; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = tid; p < CH / 2; p += SORT_THREADS) {
        const int lo = 2 * stride * (p / stride) + (p % stride);
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = sk[lo], b = sk[hi];
        if ((a > b) == up) {
          sk[lo] = b;
          sk[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  // segment starts, then an inclusive max-scan gives each element its segment start
  for (int j = tid; j < CH; j += SORT_THREADS)
    start[j] = (j == 0 || (sk[j] >> 32) != (sk[j - 1] >> 32)) ? j : 0;
  __syncthreads();
  for (int off = 1; off < CH; off <<= 1) {
    int32_t vals[CH / SORT_THREADS];
#pragma unroll
    for (int q = 0; q < CH / SORT_THREADS; ++q) {
      const int j = tid + q * SORT_THREADS;
      vals[q] = j >= off ? max(start[j], start[j - off]) : start[j];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < CH / SORT_THREADS; ++q) start[tid + q * SORT_THREADS] = vals[q];
    __syncthreads();
  }
}

__global__ __launch_bounds__(SORT_THREADS) void sort_chunks_kernel(
    const int32_t *__restrict__ keys, const int32_t *__restrict__ aux, int64_t aux_bound, int64_t N,
    int nbins, int32_t *__restrict__ chunk_counts, int32_t *__restrict__ s_key,
    int32_t *__restrict__ s_idx, int32_t *__restrict__ s_rank) {
  __shared__ uint64_t sk[CH];
  __shared__ int32_t start[CH];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * CH;
  int32_t *row = chunk_counts + (int64_t)blockIdx.x * (nbins + 1);
  for (int b = tid; b <= nbins; b += SORT_THREADS) row[b] = 0;
  sort_chunk_lds(keys, aux, aux_bound, N, nbins, blockIdx.x, sk, start);
  const int64_t nreal = min((int64_t)CH, N - base);
  for (int j = tid; j < nreal; j += SORT_THREADS) {
    const uint64_t v = sk[j];
    const uint32_t key = (uint32_t)(v >> 32);
    const int32_t rank = j - start[j];
    s_key[base + j] = (int32_t)key;
    s_idx[base + j] = (int32_t)(uint32_t)v;
    s_rank[base + j] = rank;
    const bool last = (j == nreal - 1) || ((uint32_t)(sk[j + 1] >> 32) != key);
    if (last) row[key] = rank + 1;
  }
}

// Column c of bin b: exclusive scan over the chunks in place, returning the
// bin's total.  Loads go out in batches of 16 so that their latencies overlap
// (a load of the next chunk may not pass the store of the previous one).
constexpr int SCAN_BATCH = 16;
__device__ __forceinline__ int32_t column_exclusive_scan(int32_t *__restrict__ cc, int64_t ld, int b, int nchunk) {
  int32_t run = 0;
  for (int c0 = 0; c0 < nchunk; c0 += SCAN_BATCH) {
    int32_t v[SCAN_BATCH];
#pragma unroll
    for (int u = 0; u < SCAN_BATCH; ++u) v[u] = c0 + u < nchunk ? cc[(c0 + u) * ld + b] : 0;
#pragma unroll
    for (int u = 0; u < SCAN_BATCH; ++u) {
      if (c0 + u < nchunk) cc[(c0 + u) * ld + b] = run;
      run += v[u];
    }
  }
  return run;
}
// cc[c][b] += o for every chunk c, in batches of 16 loads.
__device__ __forceinline__ void column_add(int32_t *__restrict__ cc, int64_t ld, int b, int nchunk, int32_t o) {
  for (int c0 = 0; c0 < nchunk; c0 += SCAN_BATCH) {
    int32_t v[SCAN_BATCH];
#pragma unroll
    for (int u = 0; u < SCAN_BATCH; ++u) v[u] = c0 + u < nchunk ? cc[(c0 + u) * ld + b] : 0;
#pragma unroll
    for (int u = 0; u < SCAN_BATCH; ++u)
      if (c0 + u < nchunk) cc[(c0 + u) * ld + b] = v[u] + o;
  }
}

// One workgroup: bases[c][b] = offsets[b] + sum_{c' < c} counts[c'][b].
__global__ __launch_bounds__(1024) void scan_counts_kernel(int32_t *__restrict__ cc, int nchunk, int nbins,
                                                           int32_t *__restrict__ offsets) {
  __shared__ int32_t buf[1024];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  const int64_t ld = nbins + 1;
  // per bin: exclusive scan over chunks; the total goes to offsets[b] for now
  for (int b = tid; b < nbins; b += 1024) offsets[b] = column_exclusive_scan(cc, ld, b, nchunk);
  if (tid == 0) carry = 0;
  __syncthreads();
  // exclusive scan of the totals over bins, 1024 at a time
  for (int b0 = 0; b0 < nbins; b0 += 1024) {
    const int b = b0 + tid;
    const int32_t own = b < nbins ? offsets[b] : 0;
    buf[tid] = own;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t add = tid >= off ? buf[tid - off] : 0;
      __syncthreads();
      buf[tid] += add;
      __syncthreads();
    }
    const int32_t excl = carry + buf[tid] - own;
    if (b < nbins) offsets[b] = excl;
    __syncthreads();
    if (tid == 1023) carry = excl + own;
    __syncthreads();
  }
  if (tid == 0) offsets[nbins] = carry;
  __syncthreads();
  for (int b = tid; b < nbins; b += 1024) column_add(cc, ld, b, nchunk, offsets[b]);
}

// Multi-workgroup variant for many bins (e.g. one bin per token).
// Pass 1: per bin, exclusive scan over chunks in place; bin totals to offsets[b]
// and per-block sums of the totals to bsum[block].
__global__ __launch_bounds__(SCAN_BLOCK) void scan_bins_pass1(int32_t *__restrict__ cc, int nchunk, int nbins,
                                                              int32_t *__restrict__ offsets, int32_t *__restrict__ bsum) {
  __shared__ int32_t red[SCAN_BLOCK];
  const int b = blockIdx.x * SCAN_BLOCK + threadIdx.x;
  const int64_t ld = nbins + 1;
  int32_t run = 0;
  if (b < nbins) {
    run = column_exclusive_scan(cc, ld, b, nchunk);
    offsets[b] = run;
  }
  red[threadIdx.x] = run;
  __syncthreads();
  for (int o = SCAN_BLOCK / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) bsum[blockIdx.x] = red[0];
}

// Pass 2 (one workgroup): exclusive scan of the block sums; total to offsets[nbins].
__global__ __launch_bounds__(1024) void scan_bins_pass2(int32_t *__restrict__ bsum, int nblocks, int nbins,
                                                        int32_t *__restrict__ offsets) {
  __shared__ int32_t buf[1024];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int b0 = 0; b0 < nblocks; b0 += 1024) {
    const int b = b0 + tid;
    const int32_t own = b < nblocks ? bsum[b] : 0;
    buf[tid] = own;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t add = tid >= off ? buf[tid - off] : 0;
      __syncthreads();
      buf[tid] += add;
      __syncthreads();
    }
    const int32_t excl = carry + buf[tid] - own;
    if (b < nblocks) bsum[b] = excl;
    __syncthreads();
    if (tid == 1023) carry = excl + own;
    __syncthreads();
  }
  if (tid == 0) offsets[nbins] = carry;
}

// Pass 3: exclusive scan of the bin totals inside each block plus the block's
// base gives offsets[b]; every chunk's base for the bin adds it.
__global__ __launch_bounds__(SCAN_BLOCK) void scan_bins_pass3(int32_t *__restrict__ cc, int nchunk, int nbins,
                                                              int32_t *__restrict__ offsets,
                                                              const int32_t *__restrict__ bsum) {
  __shared__ int32_t buf[SCAN_BLOCK];
  const int tid = threadIdx.x;
  const int b = blockIdx.x * SCAN_BLOCK + tid;
  const int32_t own = b < nbins ? offsets[b] : 0;
  buf[tid] = own;
  __syncthreads();
  for (int off = 1; off < SCAN_BLOCK; off <<= 1) {
    const int32_t add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  if (b >= nbins) return;
  const int32_t o = bsum[blockIdx.x] + buf[tid] - own;
  offsets[b] = o;
  column_add(cc, nbins + 1, b, nchunk, o);
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t *__restrict__ cc, int nbins, int64_t N,
                                                      const int32_t *__restrict__ s_key,
                                                      const int32_t *__restrict__ s_idx,
                                                      const int32_t *__restrict__ s_rank,
                                                      int32_t *__restrict__ perm_src,
                                                      int32_t *__restrict__ perm_pos) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= N) return;
  const int32_t key = s_key[j];
  const int32_t i = s_idx[j];
  if (key >= nbins) {
    if (perm_pos) perm_pos[i] = -1;
    return;
  }
  const int64_t c = j / CH;
  const int32_t pos = cc[c * (nbins + 1) + key] + s_rank[j];
  if (perm_src) perm_src[pos] = i;
  if (perm_pos) perm_pos[i] = pos;
}

// The whole sort in one workgroup when every key fits one chunk (N <= 512,
// e.g. a decode step) and the bins fit LDS: chunk sort, bin counts, their
// exclusive scan and the scatter, with the same results as the general path.
constexpr int ONE_CHUNK_BINS = 4096;
__global__ __launch_bounds__(SORT_THREADS) void sort_one_chunk_kernel(
    const int32_t *__restrict__ keys, const int32_t *__restrict__ aux, int64_t aux_bound, int64_t N, int nbins,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm_src, int32_t *__restrict__ perm_pos) {
  __shared__ uint64_t sk[CH];
  __shared__ int32_t start[CH];
  __shared__ int32_t off[ONE_CHUNK_BINS + 1];
  __shared__ int32_t part[SORT_THREADS];
  const int tid = threadIdx.x;
  for (int b = tid; b <= nbins; b += SORT_THREADS) off[b] = 0;
  sort_chunk_lds(keys, aux, aux_bound, N, nbins, 0, sk, start);
  const int nreal = (int)min((int64_t)CH, N);
  for (int j = tid; j < nreal; j += SORT_THREADS) {
    const uint32_t key = (uint32_t)(sk[j] >> 32);
    const bool last = (j == nreal - 1) || ((uint32_t)(sk[j + 1] >> 32) != key);
    if (last) off[key] = j - start[j] + 1;   // count of the bin (the dropped bin nbins included)
  }
  __syncthreads();
  // exclusive scan of off[0 .. nbins-1]: thread t sums bins [per*t, per*t + per)
  const int per = (nbins + SORT_THREADS - 1) / SORT_THREADS;
  const int b0 = min(tid * per, nbins), b1 = min(b0 + per, nbins);
  int32_t sum = 0;
  for (int b = b0; b < b1; ++b) sum += off[b];
  part[tid] = sum;
  __syncthreads();
  for (int o = 1; o < SORT_THREADS; o <<= 1) {
    const int32_t add = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int32_t run = part[tid] - sum;
  for (int b = b0; b < b1; ++b) {
    const int32_t c = off[b];
    off[b] = run;
    offsets[b] = run;
    run += c;
  }
  if (tid == SORT_THREADS - 1) offsets[nbins] = part[SORT_THREADS - 1];
  __syncthreads();
  for (int j = tid; j < nreal; j += SORT_THREADS) {
    const uint64_t v = sk[j];
    const int32_t key = (int32_t)(v >> 32);
    const int32_t i = (int32_t)(uint32_t)v;
    if (key >= nbins) {
      if (perm_pos) perm_pos[i] = -1;
      continue;
    }
    const int32_t pos = off[key] + (j - start[j]);
    if (perm_src) perm_src[pos] = i;
    if (perm_pos) perm_pos[i] = pos;
  }
}

hipError_t launch_counting_sort(const int32_t *keys, const int32_t *aux, int64_t aux_bound, int64_t N,
                                int64_t nbins, int32_t *offsets, int32_t *perm_src, int32_t *perm_pos,
                                int32_t *ws, hipStream_t st) {
  const int64_t nchunk = cdiv(N, CH);
  int32_t *cc = ws;
  int32_t *s_key = cc + nchunk * (nbins + 1);
  int32_t *s_idx = s_key + nchunk * CH;
  int32_t *s_rank = s_idx + nchunk * CH;
  timing_before(2, st);
  if (N <= CH && nbins <= ONE_CHUNK_BINS) {
    sort_one_chunk_kernel<<<1, SORT_THREADS, 0, st>>>(keys, aux, aux_bound, N, (int)nbins, offsets, perm_src,
                                                     perm_pos);
    timing_after(2, st);
    return hipGetLastError();
  }
  if (N > 0)
    sort_chunks_kernel<<<(unsigned)nchunk, SORT_THREADS, 0, st>>>(keys, aux, aux_bound, N, (int)nbins, cc,
                                                                  s_key, s_idx, s_rank);
  if (nbins <= SINGLE_SCAN_BINS) {
    scan_counts_kernel<<<1, 1024, 0, st>>>(cc, (int)nchunk, (int)nbins, offsets);
  } else {
    int32_t *bsum = s_rank + nchunk * CH;
    const unsigned nb = (unsigned)cdiv(nbins, SCAN_BLOCK);
    scan_bins_pass1<<<nb, SCAN_BLOCK, 0, st>>>(cc, (int)nchunk, (int)nbins, offsets, bsum);
    scan_bins_pass2<<<1, 1024, 0, st>>>(bsum, (int)nb, (int)nbins, offsets);
    scan_bins_pass3<<<nb, SCAN_BLOCK, 0, st>>>(cc, (int)nchunk, (int)nbins, offsets, bsum);
  }
  if (N > 0)
    scatter_kernel<<<(unsigned)cdiv(N, 256), 256, 0, st>>>(cc, (int)nbins, N, s_key, s_idx, s_rank, perm_src,
                                                          perm_pos);
  timing_after(2, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------- gather

// One wave per output row.  bf16: 16-byte copies.  fp8: a 1x128 group is 16
// lanes x 8 values; amax over the 16 lanes, s = amax/448 (IEEE division),
// code = RNE(v / s), 8 codes per lane stored as 8 bytes.
template <bool FP8>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *__restrict__ x, int H,
                                                          const int32_t *__restrict__ perm_src,
                                                          const int32_t *__restrict__ tok, int k, int64_t N,
                                                          const int32_t *__restrict__ offsets_end,
                                                          void *__restrict__ x_perm,
                                                          float *__restrict__ x_scale) {
  const int lane = lane_id();
  const int64_t p = (int64_t)blockIdx.x * 4 + wave_id();
  if (p >= N || (offsets_end && p >= offsets_end[0])) return;
  const int64_t i = perm_src ? perm_src[p] : p;   // no permutation: quantise rows in place order
  const int64_t t = tok ? tok[i] : i / k;
  const uint16_t *src = x + t * H;
  // row segments of 512 values (8 per lane), four at a time: the loads of a
  // batch are issued before any of them is used
  constexpr int BATCH = 4;
  if constexpr (!FP8) {
    uint16_t *dst = reinterpret_cast<uint16_t *>(x_perm) + p * H;
    for (int c0 = lane * 8; c0 < H; c0 += 512 * BATCH) {
      i32x4 raw[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
        if (c0 + 512 * u < H) raw[u] = load16(src + c0 + 512 * u);
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
        if (c0 + 512 * u < H) store16(dst + c0 + 512 * u, raw[u]);
    }
  } else {
    uint8_t *dst = reinterpret_cast<uint8_t *>(x_perm) + p * H;
    for (int c0 = lane * 8; c0 < H; c0 += 512 * BATCH) {
      i32x4 rawb[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
        if (c0 + 512 * u < H) rawb[u] = load16(src + c0 + 512 * u);
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int c = c0 + 512 * u;
        if (c >= H) break;
        const i32x4 raw = rawb[u];
        float v[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t wv = (uint32_t)raw[q];
          v[2 * q] = bf16_to_f32(wv & 0xFFFFu);
          v[2 * q + 1] = bf16_to_f32(wv >> 16);
        }
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[q]));
        amax = wave_xor_max(amax, 16);
        const float s = group_scale(amax);
        uint32_t lo = f32x4_to_e4m3(__fdiv_rn(v[0], s), __fdiv_rn(v[1], s), __fdiv_rn(v[2], s), __fdiv_rn(v[3], s));
        uint32_t hi = f32x4_to_e4m3(__fdiv_rn(v[4], s), __fdiv_rn(v[5], s), __fdiv_rn(v[6], s), __fdiv_rn(v[7], s));
        *reinterpret_cast<uint2 *>(dst + c) = make_uint2(lo, hi);
        if ((lane & 15) == 0) x_scale[p * (H / 128) + c / 128] = s;
      }
    }
  }
}

hipError_t launch_gather_rows(const uint16_t *x, int64_t H, const int32_t *perm_src, const int32_t *tok,
                              int k, int64_t N, const int32_t *offsets_end, bool fp8, void *x_perm,
                              float *x_scale, hipStream_t st) {
  if (N == 0) return hipSuccess;
  const unsigned g = (unsigned)cdiv(N, 4);
  timing_before(3, st);
  if (fp8)
    gather_rows_kernel<true><<<g, 256, 0, st>>>(x, (int)H, perm_src, tok, k, N, offsets_end, x_perm, x_scale);
  else
    gather_rows_kernel<false><<<g, 256, 0, st>>>(x, (int)H, perm_src, tok, k, N, offsets_end, x_perm, x_scale);
  timing_after(3, st);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t *x, int64_t H, int64_t T, uint8_t *xq, float *x_scale,
                                hipStream_t st) {
  if (T == 0) return hipSuccess;
  const unsigned g = (unsigned)cdiv(T, 4);
  timing_before(3, st);
  gather_rows_kernel<true><<<g, 256, 0, st>>>(x, (int)H, nullptr, nullptr, 1, T, nullptr, xq, x_scale);
  timing_after(3, st);
  return hipGetLastError();
}

}  // namespace moe
