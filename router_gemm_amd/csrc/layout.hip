// layout.hip -- repacking of expert weights into the 16-row tile layout that
// the grouped expert GEMMs read with whole-kilobyte loads (a permutation of
// bytes: no arithmetic).

#include <algorithm>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

// One thread per 16-byte piece of the packed matrices: piece p is lane
// l = p % 64 of load q = (p / 64) % 2 of tile n = p / 128, which is tile
// (t, c) = (n % (rows/16), n / (rows/16)) of matrix n / (rows/16 * nchunk);
// it holds bytes 32 g + 16 q .. +15 of chunk c of row 16 t + i, with
// i = l % 16, g = l / 16.
__global__ __launch_bounds__(256) void pack_tile16_kernel(const uint8_t *src, uint8_t *dst, int64_t count,
                                                          int64_t rows, int64_t row_bytes) {
  const int64_t npieces = count * rows * row_bytes / 16;
  const int64_t nchunk = row_bytes / 128, ntile = rows / 16;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < npieces; p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tile = p >> 7;
    const int w = (int)(p & 127), q = w >> 6, l = w & 63, i = l & 15, g = l >> 4;
    const int64_t m = tile / (ntile * nchunk), in = tile - m * ntile * nchunk;
    const int64_t c = in / ntile, t = in - c * ntile;
    const int64_t s = m * rows * row_bytes + (16 * t + i) * row_bytes + 128 * c + 32 * g + 16 * q;
    store16(dst + p * 16, load16(src + s));
  }
}

hipError_t launch_pack_tile16(const uint8_t *src, uint8_t *dst, int64_t count, int64_t rows, int64_t row_bytes,
                              hipStream_t st) {
  const int64_t npieces = count * rows * row_bytes / 16;
  if (npieces == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(cdiv(npieces, 256), 65536);
  pack_tile16_kernel<<<(unsigned)blocks, 256, 0, st>>>(src, dst, count, rows, row_bytes);
  return hipGetLastError();
}

}  // namespace moe
