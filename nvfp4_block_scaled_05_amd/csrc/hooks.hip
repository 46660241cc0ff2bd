// Test hook: the E2M1 encoders of the quantize kernels applied to given
// (already scaled) values and random words, so that the GPU tests can check
// them against the CPU definition on chosen inputs, thresholds included.
#include "codec.h"
#include "launch.h"

namespace nvfp4 {
namespace {

// Thread t encodes pairs 4t .. 4t+3 (fewer at the end).
__global__ void k_debug_e2m1(const float *__restrict__ v, const uint32_t *__restrict__ r, uint8_t *__restrict__ out,
                             uint64_t n, bool sr, bool pairwise) {
  const uint64_t g = (static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (g >= n) return;
  const int cnt = n - g < 4 ? static_cast<int>(n - g) : 4;
  float a[8];
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool in = q < cnt;
    a[2 * q] = in ? v[2 * (g + q)] : 0.0f;
    a[2 * q + 1] = in ? v[2 * (g + q) + 1] : 0.0f;
    w[q] = in && sr ? r[g + q] : 0u;
  }
  uint32_t word = 0;
  if (!pairwise) {
    word = sr ? e2m1_sr_x8(a, w) : e2m1_rne_x8(a);
  } else if (sr) {
    word = e2m1_sr_pair_into(word, a[0], a[1], w[0], 0);
    word = e2m1_sr_pair_into(word, a[2], a[3], w[1], 1);
    word = e2m1_sr_pair_into(word, a[4], a[5], w[2], 2);
    word = e2m1_sr_pair_into(word, a[6], a[7], w[3], 3);
  } else {
    word = e2m1_rne_pair_into(word, a[0], a[1], 0);
    word = e2m1_rne_pair_into(word, a[2], a[3], 1);
    word = e2m1_rne_pair_into(word, a[4], a[5], 2);
    word = e2m1_rne_pair_into(word, a[6], a[7], 3);
  }
  for (int q = 0; q < cnt; ++q) out[g + q] = static_cast<uint8_t>(word >> (8 * q));
}

}  // namespace

hipError_t launch_debug_e2m1(const float *v, const uint32_t *r, uint8_t *out, uint64_t n, bool sr, bool pairwise,
                             hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(k_debug_e2m1, dim3(static_cast<uint32_t>((threads + 255) / 256)), dim3(256), 0, s, v, r, out, n,
                     sr, pairwise);
  return hipGetLastError();
}

}  // namespace nvfp4
