// Internal launch interface between the C ABI (validation, dispatch) and the
// gfx950 kernels. Every launcher assumes its arguments were validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

enum InType : int { kBF16 = 0, kFP32 = 1 };

// Arguments of the fused cast(-transpose) kernels. A direction whose data
// pointer is NULL is not written.
struct CastArgs {
  const void *x;
  uint32_t rows, cols;
  uint8_t *row_data, *row_scales;
  const float *row_amax;
  uint8_t *col_data, *col_scales;
  const float *col_amax;
  uint32_t swizzled;
  uint32_t sr_seed;
  uint32_t sign_mask;
  const float *noop;
};

// Arguments of the row-scaled (per-row amax) kernel: row-wise output only.
struct RowScaledArgs {
  const void *x;
  uint32_t rows, cols;
  uint8_t *data, *scales;  // NULL data: only compute the per-row amax
  float *amax;             // [rows]
  uint32_t sr_seed;
  const float *noop;
};

hipError_t launch_zero_amax(float *a, float *b, const float *noop, hipStream_t s);
hipError_t launch_amax(const void *x, int dtype, uint64_t n, float *a, float *b, const float *noop,
                       hipStream_t s);
hipError_t launch_rht_amax(const void *x, int dtype, uint32_t rows, uint32_t cols, uint32_t mask,
                           float *row_amax, float *col_amax, const float *noop, hipStream_t s);
hipError_t launch_cast(const CastArgs &a, int dtype, bool block_2d, bool rht, bool sr, hipStream_t s);
// compute_amax: reduce each row's amax in the kernel (else read a.amax).
hipError_t launch_rowscaled(const RowScaledArgs &a, int dtype, bool sr, bool compute_amax, hipStream_t s);
hipError_t launch_dequant(const uint8_t *data, const uint8_t *scales, const float *amax, uint32_t rows,
                          uint32_t cols, bool swizzled, bool row_scaled, float *y, hipStream_t s);
hipError_t launch_debug_rht(const void *x, int dtype, uint32_t rows, uint32_t cols, uint32_t mask, float *t,
                            hipStream_t s);

}  // namespace nvfp4
