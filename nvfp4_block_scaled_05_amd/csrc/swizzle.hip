// Compact -> GEMM-swizzled scales for shapes with partial scale tiles.
//
// "Fuse NVFP4 scale swizzling on SM120 and SM121" (Description): when rows or
// columns are not multiples of 128 the quantize call keeps compact scales and
// a separate pass lays them out for the GEMM. Here that pass pads the scale
// matrix with zeros to whole 128-row x 4-column tiles (512 bytes each, in
// row-major tile order; scale (r, c) at (r%32)*16 + (r%128)/32*4 + c%4 inside
// its tile).
//
// One thread per output word: the four scales c0..c0+3 of one row, which sit
// next to each other in both layouts. Consecutive threads write consecutive
// words, so the stores are fully coalesced; the loads are 4-byte pieces of
// rows r, r + 32, r + 64, r + 96, r + 1, ... of one 128-row band.
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_swizzle(const uint8_t *__restrict__ compact, uint32_t rows,
                                                      uint32_t scale_cols, uint32_t tiles_per_row, uint64_t words,
                                                      uint32_t *__restrict__ out) {
  const uint64_t word = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (word >= words) return;
  const uint64_t tile = word >> 7;     // 128 words per 512-byte tile
  const uint32_t w = word & 127u;      // word in the tile = (r % 32) * 4 + (r % 128) / 32
  const uint32_t r = static_cast<uint32_t>(tile / tiles_per_row) * 128 + (w >> 2) + 32 * (w & 3);
  const uint32_t c0 = static_cast<uint32_t>(tile % tiles_per_row) * 4;
  uint32_t v = 0;
  if (r < rows) {
    const uint8_t *src = compact + static_cast<uint64_t>(r) * scale_cols + c0;
    if ((scale_cols & 3u) == 0) {  // c0 + 4 <= scale_cols and 4-byte aligned
      v = *reinterpret_cast<const uint32_t *>(src);
    } else {
#pragma unroll
      for (uint32_t i = 0; i < 4; ++i)
        if (c0 + i < scale_cols) v |= static_cast<uint32_t>(src[i]) << (8 * i);
    }
  }
  out[word] = v;
}

}  // namespace

uint64_t swizzled_scales_bytes(uint64_t rows, uint64_t scale_cols) {
  return (rows + 127) / 128 * 128 * ((scale_cols + 3) / 4 * 4);
}

hipError_t launch_swizzle(const uint8_t *compact, uint32_t rows, uint32_t scale_cols, uint8_t *out, hipStream_t s) {
  const uint64_t words = swizzled_scales_bytes(rows, scale_cols) / 4;
  if (words == 0) return hipSuccess;
  const uint32_t tiles_per_row = (scale_cols + 3) / 4;
  hipLaunchKernelGGL(k_swizzle, dim3(static_cast<uint32_t>((words + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                     compact, rows, scale_cols, tiles_per_row, words, reinterpret_cast<uint32_t *>(out));
  return hipGetLastError();
}

}  // namespace nvfp4
