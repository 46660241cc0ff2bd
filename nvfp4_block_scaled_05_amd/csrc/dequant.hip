// NVFP4 dequantization of one orientation for gfx950.
//
// y = (value(code) * value(scale)) / S, where the product is exact and S is
// the global encode scale of the tensor amax, or of the row's amax for
// row-scaled tensors ("Implement row-scaled NVFP4 fprop recipe", Changes:
// the dequantize kernel picks the per-row amax). Each thread turns one
// 32-bit word of codes (8 elements) into two 128-bit stores.
#include "codec.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

// E2M1 code -> value: magnitude 0.5 * m for exponent 0, else
// (1 + m / 2) * 2^(e - 1); bit 3 is the sign.
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  const uint32_t e = (code >> 1) & 3u;
  const uint32_t m = code & 1u;
  const float mag = e == 0 ? (m ? 0.5f : 0.0f) : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return (code & 8u) ? -mag : mag;
}

__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t *__restrict__ data,
                                                      const uint8_t *__restrict__ scales,
                                                      const float *__restrict__ amax, uint32_t rows, uint32_t cols,
                                                      uint32_t swizzled, uint32_t row_scaled, uint32_t ue5m3,
                                                      float *__restrict__ y) {
  const uint64_t i = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const uint32_t units_per_row = cols >> 3;
  if (i >= static_cast<uint64_t>(rows) * units_per_row) return;
  const uint32_t r = static_cast<uint32_t>(i / units_per_row);
  const uint32_t c = static_cast<uint32_t>(i % units_per_row) * 8;
  const float S = global_encode_scale(amax[row_scaled ? r : 0], ue5m3 != 0);
  const uint32_t scale_cols = cols >> 4;
  const uint64_t soff = swizzled ? swizzled_scale_offset(r, c >> 4, scale_cols)
                                 : static_cast<uint64_t>(r) * scale_cols + (c >> 4);
  const float sf = scale_decode(scales[soff], ue5m3 != 0);
  const uint32_t word = *reinterpret_cast<const uint32_t *>(data + static_cast<uint64_t>(r) * (cols >> 1) + (c >> 1));
  float out[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) out[q] = (e2m1_value((word >> (4 * q)) & 15u) * sf) / S;
  float4 *dst = reinterpret_cast<float4 *>(y + static_cast<uint64_t>(r) * cols + c);
  dst[0] = make_float4(out[0], out[1], out[2], out[3]);
  dst[1] = make_float4(out[4], out[5], out[6], out[7]);
}

}  // namespace

hipError_t launch_dequant(const uint8_t *data, const uint8_t *scales, const float *amax, uint32_t rows,
                          uint32_t cols, bool swizzled, bool row_scaled, bool ue5m3, float *y, hipStream_t s) {
  const uint64_t units = static_cast<uint64_t>(rows) * (cols >> 3);
  if (units == 0) return hipSuccess;
  const uint32_t blocks = static_cast<uint32_t>((units + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(k_dequant, dim3(blocks), dim3(kThreads), 0, s, data, scales, amax, rows, cols,
                     swizzled ? 1u : 0u, row_scaled ? 1u : 0u, ue5m3 ? 1u : 0u, y);
  return hipGetLastError();
}

}  // namespace nvfp4
