// Weight preparation: a row-major matrix re-laid into the tiled fp16 layout that the products'
// operand loads read as whole 1 KiB blocks (16 rows x 32 columns per tile).
#include "common.h"
#include "kernels.h"

namespace q3 {

// One thread per 16-byte chunk of the output, in output order: chunk i is tile i / 64, row
// (i % 64) / 4 of that tile, columns 8 * (i % 4) .. + 7 of the tile. A wave writes one whole tile.
template <int DT>
__global__ __launch_bounds__(256) void tile_matrix_kernel(const void* __restrict__ src, int cols,
                                                          int64_t chunks, uint16_t* __restrict__ dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= chunks) return;
  const int64_t tile = i >> 6;
  const int in_tile = static_cast<int>(i & 63);
  const int tiles_per_group = cols >> 5;
  const int64_t g = tile / tiles_per_group;
  const int kt = static_cast<int>(tile - g * tiles_per_group);
  const int64_t r = g * 16 + (in_tile >> 2);
  const int c = kt * 32 + (in_tile & 3) * 8;
  float v[8];
  load8<DT>(src, r * cols + c, v);
  store8<DT_F16>(dst, i * 8, v);
}

hipError_t launch_tile_matrix(const void* src, int src_dt, int rows, int cols, uint16_t* dst, hipStream_t s) {
  if (rows <= 0 || cols <= 0 || rows % 16 != 0 || cols % 32 != 0) return hipErrorInvalidValue;
  const int64_t chunks = static_cast<int64_t>(rows) * cols / 8;
  const int64_t blocks = (chunks + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>(blocks);
  switch (src_dt) {
    case DT_F32: tile_matrix_kernel<DT_F32><<<grid, 256, 0, s>>>(src, cols, chunks, dst); break;
    case DT_BF16: tile_matrix_kernel<DT_BF16><<<grid, 256, 0, s>>>(src, cols, chunks, dst); break;
    case DT_F16: tile_matrix_kernel<DT_F16><<<grid, 256, 0, s>>>(src, cols, chunks, dst); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace q3
