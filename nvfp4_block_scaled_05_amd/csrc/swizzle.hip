// Compact -> GEMM-swizzled scales for shapes with partial scale tiles.
//
// "Fuse NVFP4 scale swizzling on SM120 and SM121" (Description): when rows or
// columns are not multiples of 128 the quantize call keeps compact scales and
// a separate pass lays them out for the GEMM. Here that pass pads the scale
// matrix with zeros to whole 128-row x 4-column tiles (512 bytes each, in
// row-major tile order; scale (r, c) at (r%32)*16 + (r%128)/32*4 + c%4 inside
// its tile).
//
// One workgroup per 128-row band and 128 scale columns (32 tiles): the
// band's compact scales go to LDS by coalesced loads (eight lanes per row,
// 16 bytes each: one 16-byte load where rows and buffer allow it, else four
// 4-byte loads, else single bytes), and the 32 tiles, 16 KiB contiguous in
// the output, leave as 16-byte pieces: piece r32 of tile j holds rows r32,
// r32 + 32, r32 + 64 and r32 + 96 of the band, four codes each (4-byte
// stores when the output is not 16-byte aligned). Past the scale matrix
// every byte is zero.
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kBand = 128;                  // rows per band (one tile high)
constexpr uint32_t kChunk = 128;                 // scale columns per workgroup (32 tiles)
constexpr uint32_t kRowWords = kChunk / 4 + 1;   // LDS words per band row (one pad word: no bank conflicts)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void k_swizzle(const uint8_t *__restrict__ compact, uint32_t rows,
                                                      uint32_t scale_cols, uint32_t tiles_per_row, uint32_t chunks,
                                                      uint8_t *__restrict__ out) {
  __shared__ uint32_t lds[kBand * kRowWords];
  const uint32_t t = threadIdx.x;
  const uint32_t band = blockIdx.x / chunks, chunk = blockIdx.x - band * chunks;  // one-dimensional grid
  const uint32_t r0 = band * kBand, c0 = chunk * kChunk;
  const bool in16 = (scale_cols & 15u) == 0 && (reinterpret_cast<uintptr_t>(compact) & 15u) == 0;  // uniform
  const bool in4 = (scale_cols & 3u) == 0;  // rows 4-byte aligned (the buffer is)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t i = t + kThreads * k;  // piece i: band row i / 8, bytes 16 (i % 8) .. + 15 of the chunk
    const uint32_t lr = i >> 3, part = i & 7;
    const uint32_t r = r0 + lr, c = c0 + 16 * part;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (r < rows && c < scale_cols) {
      const uint8_t *src = compact + static_cast<uint64_t>(r) * scale_cols + c;
      if (in16 && c + 16 <= scale_cols) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(src);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
      } else if (in4) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (c + 4 * q < scale_cols) w[q] = reinterpret_cast<const uint32_t *>(src)[q];
      } else {
        for (uint32_t b = 0; b < 16 && c + b < scale_cols; ++b) w[b >> 2] |= static_cast<uint32_t>(src[b]) << (8 * (b & 3));
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) lds[lr * kRowWords + 4 * part + q] = w[q];
  }
  __syncthreads();
  const bool out16 = (reinterpret_cast<uintptr_t>(out) & 15u) == 0;  // uniform
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t p = t + kThreads * k;  // piece r32 = p % 32 of tile j = p / 32
    const uint32_t j = p >> 5, r32 = p & 31;
    const uint32_t tile_c = chunk * (kChunk / 4) + j;
    if (tile_c >= tiles_per_row) continue;
    const uint32_t v[4] = {lds[r32 * kRowWords + j], lds[(r32 + 32) * kRowWords + j], lds[(r32 + 64) * kRowWords + j],
                           lds[(r32 + 96) * kRowWords + j]};
    uint8_t *dst = out + (static_cast<uint64_t>(band) * tiles_per_row + tile_c) * 512 + 16 * r32;
    if (out16) {
      *reinterpret_cast<u32x4 *>(dst) = u32x4{v[0], v[1], v[2], v[3]};
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) reinterpret_cast<uint32_t *>(dst)[q] = v[q];
    }
  }
}

}  // namespace

uint64_t swizzled_scales_bytes(uint64_t rows, uint64_t scale_cols) {
  return (rows + 127) / 128 * 128 * ((scale_cols + 3) / 4 * 4);
}

hipError_t launch_swizzle(const uint8_t *compact, uint32_t rows, uint32_t scale_cols, uint8_t *out, hipStream_t s) {
  const uint64_t words = swizzled_scales_bytes(rows, scale_cols) / 4;
  if (words == 0) return hipSuccess;
  const uint32_t tiles_per_row = (scale_cols + 3) / 4;
  const uint32_t chunks = (scale_cols + kChunk - 1) / kChunk;
  const uint64_t grid = static_cast<uint64_t>(chunks) * ((rows + kBand - 1) / kBand);  // < 2^27: the padded matrix is < 2^34 bytes
  hipLaunchKernelGGL(k_swizzle, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, s, compact, rows, scale_cols,
                     tiles_per_row, chunks, out);
  return hipGetLastError();
}

}  // namespace nvfp4
