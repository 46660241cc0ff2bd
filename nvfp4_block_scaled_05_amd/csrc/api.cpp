// C ABI of the NVFP4 quantize library: host-side validation and dispatch.
//
// Every argument is checked before anything is queued, so a rejected call
// writes nothing. The gates follow the pages: swizzled scales need 128x128
// alignment and partial tiles are rejected ("Fuse NVFP4 scale swizzling on
// SM120 and SM121", Changes and Validation); row-scaled NVFP4 is 1x16,
// compact and not combined with the RHT ("Implement row-scaled NVFP4 fprop
// recipe", Changes; "Fuse NVFP4 scale swizzling ...", Changes), its
// column-wise side taking one amax per input column (the quantizer
// prototype in the review thread of "Write both NVFP4 amax buffers"); an
// RHT quantize cannot share one float between its two amaxes ("Write both
// NVFP4 amax buffers", review thread).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "launch.h"
#include "nvfp4.h"

namespace {

thread_local std::string g_last_error;

nvfp4_status_t fail(nvfp4_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned(const void *p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

nvfp4_config_t config_or_default(const nvfp4_config_t *cfg) {
  if (cfg) return *cfg;
  nvfp4_config_t c{};
  c.compute_amax = 1;
  return c;
}

// The RHT kernels' mask word: the 16 sign bits, and the BF16 option above them.
uint32_t rht_word(const nvfp4_config_t &c) {
  return (c.rht_sign_mask & 0xFFFFu) | (c.rht_bf16 ? nvfp4::kRhtBf16 : 0u);
}

nvfp4_status_t hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return NVFP4_OK;
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// For non-negative a, b: a * b >= limit, or either is 2^32 or more (no size
// argument of the kernels may reach 2^32); computed without overflow.
bool product_at_least(int64_t a, int64_t b, uint64_t limit) {
  if (a == 0 || b == 0) return false;
  if (a >= (int64_t{1} << 32) || b >= (int64_t{1} << 32)) return true;
  return static_cast<uint64_t>(a) * static_cast<uint64_t>(b) >= limit;
}

// Shared checks of an input matrix.
nvfp4_status_t check_input(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t cols) {
  if (dtype != NVFP4_IN_BF16 && dtype != NVFP4_IN_FP32)
    return fail(NVFP4_ERR_UNSUPPORTED, "input dtype %d is not BF16 (0) or FP32 (1)", static_cast<int>(dtype));
  if (rows < 0 || cols < 0) return fail(NVFP4_ERR_SHAPE, "negative shape %lld x %lld", (long long)rows, (long long)cols);
  if (cols % 16 != 0) return fail(NVFP4_ERR_SHAPE, "cols = %lld is not a multiple of 16", (long long)cols);
  if (product_at_least(rows, cols, uint64_t{1} << 32))
    return fail(NVFP4_ERR_SHAPE, "rows * cols (%lld x %lld) must be below 2^32", (long long)rows, (long long)cols);
  if (rows * cols > 0 && x == nullptr) return fail(NVFP4_ERR_NULL, "input pointer is NULL");
  if (x != nullptr && !aligned(x, 16)) return fail(NVFP4_ERR_ALIGN, "input pointer is not 16-byte aligned");
  return NVFP4_OK;
}

// An empty tensor may come with NULL data and scales; amax is always written.
nvfp4_status_t check_out(const nvfp4_out_t *o, const char *name, bool empty) {
  if (o->amax == nullptr) return fail(NVFP4_ERR_NULL, "%s output has a NULL amax pointer", name);
  if (!empty && (o->data == nullptr || o->scales == nullptr))
    return fail(NVFP4_ERR_NULL, "%s output has a NULL data or scales pointer", name);
  if (!aligned(o->data, 16)) return fail(NVFP4_ERR_ALIGN, "%s data is not 16-byte aligned", name);
  if (!aligned(o->scales, 4)) return fail(NVFP4_ERR_ALIGN, "%s scales are not 4-byte aligned", name);
  if (!aligned(o->amax, 4)) return fail(NVFP4_ERR_ALIGN, "%s amax is not 4-byte aligned", name);
  return NVFP4_OK;
}

}  // namespace

extern "C" const char *nvfp4_last_error(void) { return g_last_error.c_str(); }

extern "C" uint64_t nvfp4_workspace_bytes(void) { return NVFP4_WORKSPACE_BYTES; }
static_assert(NVFP4_WORKSPACE_BYTES == nvfp4::kWorkspaceWords * 4, "workspace layout and ABI size agree");

extern "C" nvfp4_status_t nvfp4_debug_set_wait_ticks(uint32_t ticks) {
  nvfp4::set_resident_wait_ticks(ticks);
  return NVFP4_OK;
}

extern "C" nvfp4_status_t nvfp4_debug_set_resident_variant(uint32_t tiles_per_workgroup) {
  if (!nvfp4::set_resident_variant(tiles_per_workgroup))
    return fail(NVFP4_ERR_UNSUPPORTED, "unknown single-pass variant %u (0: the library's choice, 1 .. 6)",
                tiles_per_workgroup);
  return NVFP4_OK;
}

extern "C" nvfp4_status_t nvfp4_debug_set_rht_unit(uint32_t unit) {
  if (unit > 2)
    return fail(NVFP4_ERR_UNSUPPORTED, "unknown RHT unit %u (0: default, 1: vector ALU, 2: matrix cores)", unit);
  nvfp4::set_rht_unit(unit);
  return NVFP4_OK;
}

extern "C" uint64_t nvfp4_swizzled_scales_bytes(int64_t rows, int64_t scale_cols) {
  if (rows <= 0 || scale_cols <= 0 || rows >= (int64_t{1} << 32) || scale_cols >= (int64_t{1} << 32)) return 0;
  return nvfp4::swizzled_scales_bytes(static_cast<uint64_t>(rows), static_cast<uint64_t>(scale_cols));
}

extern "C" nvfp4_status_t nvfp4_swizzle_scales(const uint8_t *compact, int64_t rows, int64_t scale_cols,
                                               uint8_t *swizzled, void *stream) {
  if (rows < 0 || scale_cols < 0) return fail(NVFP4_ERR_SHAPE, "negative shape %lld x %lld", (long long)rows,
                                              (long long)scale_cols);
  if (product_at_least((rows + 127) / 128 * 128, (scale_cols + 3) / 4 * 4, uint64_t{1} << 34))
    return fail(NVFP4_ERR_SHAPE, "scale matrix %lld x %lld is too large", (long long)rows, (long long)scale_cols);
  if (rows * scale_cols == 0) return NVFP4_OK;
  if (compact == nullptr || swizzled == nullptr) return fail(NVFP4_ERR_NULL, "a scale pointer is NULL");
  if (!aligned(compact, 4) || !aligned(swizzled, 4))
    return fail(NVFP4_ERR_ALIGN, "scale buffers must be 4-byte aligned");
  return hip_status(nvfp4::launch_swizzle(compact, static_cast<uint32_t>(rows), static_cast<uint32_t>(scale_cols),
                                          swizzled, static_cast<hipStream_t>(stream)),
                    "swizzle launch");
}

extern "C" nvfp4_status_t nvfp4_compute_amax(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t cols,
                                             float *row_amax, float *col_amax, const nvfp4_config_t *cfg_in,
                                             void *stream) {
  nvfp4_status_t st = check_input(x, dtype, rows, cols);
  if (st != NVFP4_OK) return st;
  const nvfp4_config_t cfg = config_or_default(cfg_in);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (row_amax == nullptr && col_amax == nullptr) return fail(NVFP4_ERR_NULL, "both amax pointers are NULL");
  if ((row_amax && !aligned(row_amax, 4)) || (col_amax && !aligned(col_amax, 4)))
    return fail(NVFP4_ERR_ALIGN, "amax pointers must be 4-byte aligned");
  if (cfg.row_scaled && cfg.rht) return fail(NVFP4_ERR_UNSUPPORTED, "row-scaled amax cannot be combined with the RHT");
  if (cfg.rht_bf16 && !cfg.rht) return fail(NVFP4_ERR_UNSUPPORTED, "rht_bf16 needs rht");
  if (cfg.row_scaled) {
    if (row_amax != nullptr && row_amax == col_amax)
      return fail(NVFP4_ERR_UNSUPPORTED, "row-scaled per-row and per-column amaxes need two distinct buffers");
    const uint32_t R = static_cast<uint32_t>(rows), C = static_cast<uint32_t>(cols);
    if (col_amax == nullptr) {  // per-row only: one workgroup per row, no atomics
      nvfp4::RowScaledArgs a{x, R, C, nullptr, nullptr, row_amax, 0u, cfg.noop};
      return hip_status(nvfp4::launch_rowscaled(a, dtype, false, true, s), "row amax launch");
    }
    return hip_status(nvfp4::launch_dual_amax(x, dtype, R, C, row_amax, col_amax, cfg.noop, s), "row-scaled amax launch");
  }
  if (cfg.rht) {
    if (rows % 16 != 0) return fail(NVFP4_ERR_SHAPE, "the RHT needs rows %% 16 == 0 (rows = %lld)", (long long)rows);
    if (row_amax != nullptr && row_amax == col_amax)
      return fail(NVFP4_ERR_UNSUPPORTED, "the RHT amax pair needs two distinct buffers");
  }
  float *b = (col_amax == row_amax) ? nullptr : col_amax;
  float *a = row_amax ? row_amax : col_amax;
  if (a == col_amax) b = nullptr;
  st = hip_status(nvfp4::launch_zero_amax(a, b, cfg.noop, s), "zero amax launch");
  if (st != NVFP4_OK || rows * cols == 0) return st;
  if (cfg.rht)
    return hip_status(nvfp4::launch_rht_amax(x, dtype, static_cast<uint32_t>(rows), static_cast<uint32_t>(cols),
                                             rht_word(cfg), row_amax, col_amax, nullptr, nullptr, cfg.noop, s),
                      "RHT amax launch");
  return hip_status(
      nvfp4::launch_amax(x, dtype, static_cast<uint64_t>(rows * cols), a, b, nullptr, nullptr, cfg.noop, s),
      "amax launch");
}

namespace {

// nvfp4_quantize's validation and, unless check_only, its launches.
nvfp4_status_t quantize_impl(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t cols, const nvfp4_out_t *row,
                             const nvfp4_out_t *col, const nvfp4_config_t &cfg, hipStream_t s, bool check_only) {
  nvfp4_status_t st = check_input(x, dtype, rows, cols);
  if (st != NVFP4_OK) return st;
  if (row == nullptr && col == nullptr) return fail(NVFP4_ERR_NULL, "neither a row-wise nor a column-wise output");
  if (cfg.cast_events != nullptr && (cfg.cast_events[0] == nullptr || cfg.cast_events[1] == nullptr))
    return fail(NVFP4_ERR_NULL, "cast_events holds a NULL event");
  const bool empty = rows * cols == 0;
  if (row && (st = check_out(row, "row-wise", empty)) != NVFP4_OK) return st;
  if (col && (st = check_out(col, "column-wise", empty)) != NVFP4_OK) return st;
  if (cfg.scale_fmt != NVFP4_SCALE_E4M3 && cfg.scale_fmt != NVFP4_SCALE_UE5M3)
    return fail(NVFP4_ERR_UNSUPPORTED, "unknown scale format %u", cfg.scale_fmt);
  if (cfg.scale_layout != NVFP4_SCALES_COMPACT && cfg.scale_layout != NVFP4_SCALES_GEMM_SWIZZLED)
    return fail(NVFP4_ERR_UNSUPPORTED, "unknown scale layout %u", cfg.scale_layout);
  const bool swz = cfg.scale_layout == NVFP4_SCALES_GEMM_SWIZZLED;
  if (cfg.workspace != nullptr && !aligned(cfg.workspace, 16))
    return fail(NVFP4_ERR_ALIGN, "the workspace is not 16-byte aligned");
  if (cfg.amax_path > NVFP4_AMAX_PATH_SINGLE_PASS)
    return fail(NVFP4_ERR_UNSUPPORTED, "unknown amax path %u", cfg.amax_path);
  if (cfg.row_scaled) {
    if (row && col && row->amax == col->amax)
      return fail(NVFP4_ERR_UNSUPPORTED, "row-scaled per-row and per-column amaxes need two distinct buffers");
    if (cfg.block_2d) return fail(NVFP4_ERR_UNSUPPORTED, "row-scaled NVFP4 uses 1x16 blocks");
    if (cfg.rht) return fail(NVFP4_ERR_UNSUPPORTED, "row-scaled NVFP4 cannot be combined with the RHT");
    if (swz) return fail(NVFP4_ERR_UNSUPPORTED, "row-scaled NVFP4 keeps compact scales");
  }
  if (cfg.rht && cfg.block_2d) return fail(NVFP4_ERR_UNSUPPORTED, "the RHT is defined for 1x16 blocks only");
  if (cfg.rht_bf16 && !cfg.rht) return fail(NVFP4_ERR_UNSUPPORTED, "rht_bf16 needs rht");
  if (cfg.rht && row && col && row->amax == col->amax)
    return fail(NVFP4_ERR_UNSUPPORTED, "the RHT quantize needs distinct row-wise and column-wise amax buffers");
  if ((col || cfg.block_2d) && rows % 16 != 0)
    return fail(NVFP4_ERR_SHAPE, "rows = %lld must be a multiple of 16 for %s", (long long)rows,
                cfg.block_2d ? "16x16 blocks" : "the column-wise output");
  if (swz && (rows % 128 != 0 || cols % 128 != 0))
    return fail(NVFP4_ERR_SHAPE, "GEMM-swizzled scales need rows and cols that are multiples of 128 (got %lld x %lld)",
                (long long)rows, (long long)cols);
  if (check_only) return NVFP4_OK;

  const uint32_t R = static_cast<uint32_t>(rows), C = static_cast<uint32_t>(cols);
  const bool sr = cfg.stochastic != 0;
  // optional events around the cast launch (rows * cols == 0 launches nothing)
  const bool timed = cfg.cast_events != nullptr && rows * cols > 0;
  auto record = [&](int i) -> nvfp4_status_t {
    return timed ? hip_status(hipEventRecord(static_cast<hipEvent_t>(cfg.cast_events[i]), s), "cast event record")
                 : NVFP4_OK;
  };
  if (cfg.row_scaled) {
    const uint32_t ue = cfg.scale_fmt == NVFP4_SCALE_UE5M3;
    if ((st = record(0)) != NVFP4_OK) return st;
    if (!col) {  // row-wise only: one launch that reduces each row and encodes it from registers
      nvfp4::RowScaledArgs a{x, R, C, row->data, row->scales, row->amax, cfg.sr_seed, cfg.noop, ue};
      st = hip_status(nvfp4::launch_rowscaled(a, dtype, sr, cfg.compute_amax != 0, s), "row-scaled quantize launch");
      return st != NVFP4_OK ? st : record(1);
    }
    // column-wise output: the per-row and per-column amax in one read, then
    // both orientations by register tiles in a second read
    if (cfg.compute_amax)
      st = hip_status(nvfp4::launch_dual_amax(x, dtype, R, C, row ? row->amax : nullptr, col->amax, cfg.noop, s),
                      "row-scaled amax launch");
    if (st == NVFP4_OK) {
      nvfp4::CastArgs a{x,  R,          C,           row ? row->data : nullptr, row ? row->scales : nullptr,
                        row ? row->amax : nullptr, col->data, col->scales, col->amax, 0u, cfg.sr_seed,
                        0u, cfg.noop,  nullptr,    0u};
      a.ue5m3 = ue;
      st = hip_status(nvfp4::launch_cast_rowscaled(a, dtype, sr, s), "row-scaled quantize launch");
    }
    return st != NVFP4_OK ? st : record(1);
  }
  float *ra = row ? row->amax : nullptr;
  float *ca = col ? col->amax : nullptr;
  // With a workspace the amax pass leaves per-workgroup maxima there and the
  // cast kernel finishes the reduction. An empty input takes the zeroing
  // pass, which is all it needs.
  uint32_t *partials = nullptr;
  uint32_t npartials = 0;
  // single pass: one launch that reads the input once (K tiles per workgroup)
  const nvfp4::ResidentPlan plan = cfg.compute_amax && cfg.workspace != nullptr && !cfg.rht &&
                                           cfg.amax_path != NVFP4_AMAX_PATH_TWO_PASS
                                       ? nvfp4::resident_plan(dtype, cfg.block_2d != 0, sr, R, C,
                                                              cfg.amax_path == NVFP4_AMAX_PATH_AUTO, s)
                                       : nvfp4::ResidentPlan{0, 0};
  const bool resident = plan.variant > 0;
  if (cfg.compute_amax && !resident) {
    float *a = ra ? ra : ca;
    float *b = (ca == a) ? nullptr : ca;
    if (cfg.workspace != nullptr && rows * cols > 0) {
      partials = static_cast<uint32_t *>(cfg.workspace);
      if (cfg.rht)
        st = hip_status(
            nvfp4::launch_rht_amax(x, dtype, R, C, rht_word(cfg), ra, ca, partials, &npartials, cfg.noop, s),
            "RHT amax launch");
      else
        st = hip_status(nvfp4::launch_amax(x, dtype, static_cast<uint64_t>(rows * cols), a, b, partials, &npartials,
                                           cfg.noop, s),
                        "amax launch");
      if (st != NVFP4_OK) return st;
    } else {
      st = hip_status(nvfp4::launch_zero_amax(a, b, cfg.noop, s), "zero amax launch");
      if (st != NVFP4_OK) return st;
      if (rows * cols > 0) {
        if (cfg.rht)
          st = hip_status(
              nvfp4::launch_rht_amax(x, dtype, R, C, rht_word(cfg), ra, ca, nullptr, nullptr, cfg.noop, s),
              "RHT amax launch");
        else
          st = hip_status(nvfp4::launch_amax(x, dtype, static_cast<uint64_t>(rows * cols), a, b, nullptr, nullptr,
                                             cfg.noop, s),
                          "amax launch");
        if (st != NVFP4_OK) return st;
      }
    }
  }
  nvfp4::CastArgs a{x,  R,        C,    row ? row->data : nullptr, row ? row->scales : nullptr, ra,
                    col ? col->data : nullptr, col ? col->scales : nullptr, ca, swz ? 1u : 0u, cfg.sr_seed,
                    rht_word(cfg), cfg.noop, partials, npartials};
  a.ue5m3 = cfg.scale_fmt == NVFP4_SCALE_UE5M3;
  if (resident) {
    if ((st = record(0)) != NVFP4_OK) return st;
    st = hip_status(nvfp4::launch_cast_resident(a, static_cast<uint32_t *>(cfg.workspace), dtype,
                                                cfg.block_2d != 0, sr, plan, s),
                    "single-pass quantize launch");
    return st != NVFP4_OK ? st : record(1);
  }
  if ((st = record(0)) != NVFP4_OK) return st;
  st = hip_status(nvfp4::launch_cast(a, dtype, cfg.block_2d != 0, cfg.rht != 0, sr, s), "quantize launch");
  return st != NVFP4_OK ? st : record(1);
}

}  // namespace

extern "C" nvfp4_status_t nvfp4_quantize(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t cols,
                                         const nvfp4_out_t *row, const nvfp4_out_t *col,
                                         const nvfp4_config_t *cfg_in, void *stream) {
  return quantize_impl(x, dtype, rows, cols, row, col, config_or_default(cfg_in), static_cast<hipStream_t>(stream),
                       false);
}

// ---------------------------------------------------------------------------
// Allocation-free quantize: nvfp4_quantize with the library's own copy of
// the workspace, a file-scope device array that each GPU holds until the
// process ends. Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is passed to kernels.
// ---------------------------------------------------------------------------
namespace {

constexpr uint32_t kScratchWords = nvfp4::kWorkspaceWords;  // NVFP4_WORKSPACE_BYTES / 4
static_assert(kScratchWords * 4 == NVFP4_WORKSPACE_BYTES, "scratch holds one quantize workspace");
__device__ __align__(256) uint32_t scratch[kScratchWords];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
uint32_t *g_scratch_ptr[kMaxScratchDevices];   // device address of each GPU's copy
bool g_scratch_cleared[kMaxScratchDevices];    // its clearing kernel has been queued

// Zero-fills n words (a kernel rather than hipMemsetAsync: calls may be
// captured in a HIP graph).
__global__ void k_clear_scratch(uint32_t *p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The scratch address on the device that `s` runs on; on the first call for
// that device it also queues, on `s`, the clearing kernel that the
// workspace's first use needs.
nvfp4_status_t device_scratch(hipStream_t s, uint32_t **out) {
  hipDevice_t dev = -1;
  nvfp4_status_t st = hip_status(hipStreamGetDevice(s, &dev), "hipStreamGetDevice");
  if (st != NVFP4_OK) return st;
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(NVFP4_ERR_UNSUPPORTED, "device %d: the allocation-free quantize supports devices 0..%d",
                static_cast<int>(dev), kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if ((st = hip_status(hipGetDevice(&cur), "hipGetDevice")) != NVFP4_OK) return st;
    if (cur != dev && (st = hip_status(hipSetDevice(dev), "hipSetDevice")) != NVFP4_OK) return st;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if ((st = hip_status(e, "hipGetSymbolAddress(scratch)")) != NVFP4_OK) return st;
    if (p == nullptr) return fail(NVFP4_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = static_cast<uint32_t *>(p);
  }
  if (!g_scratch_cleared[dev]) {
    hipLaunchKernelGGL(k_clear_scratch, dim3(kScratchWords / 256), dim3(256), 0, s, g_scratch_ptr[dev], kScratchWords);
    if ((st = hip_status(hipGetLastError(), "scratch clearing launch")) != NVFP4_OK) return st;
    g_scratch_cleared[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}

}  // namespace

extern "C" nvfp4_status_t nvfp4_quantize_noalloc(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t cols,
                                                 const nvfp4_out_t *row, const nvfp4_out_t *col,
                                                 const nvfp4_config_t *cfg_in, void *stream) {
  nvfp4_config_t cfg = config_or_default(cfg_in);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cfg.workspace != nullptr)
    return fail(NVFP4_ERR_UNSUPPORTED, "nvfp4_quantize_noalloc uses its own scratch: config.workspace must be NULL");
  // The workspace the call needs is NVFP4_WORKSPACE_BYTES whatever the
  // input's size (the amax pass grid-strides beyond its largest grid), so
  // the scratch covers every input nvfp4_quantize accepts; the check keeps
  // that promise explicit.
  if (nvfp4_workspace_bytes() > uint64_t{kScratchWords} * 4)
    return fail(NVFP4_ERR_UNSUPPORTED, "the call needs %llu bytes of scratch, more than the %llu held",
                (unsigned long long)nvfp4_workspace_bytes(), (unsigned long long)kScratchWords * 4);
  nvfp4_status_t st = quantize_impl(x, dtype, rows, cols, row, col, cfg, s, true);  // validation only
  if (st != NVFP4_OK) return st;
  uint32_t *ws = nullptr;
  if ((st = device_scratch(s, &ws)) != NVFP4_OK) return st;
  cfg.workspace = ws;
  return quantize_impl(x, dtype, rows, cols, row, col, cfg, s, false);
}

extern "C" nvfp4_status_t nvfp4_quantize_grouped(const void *x, nvfp4_dtype_t dtype, int64_t num_groups,
                                                 const int64_t *group_rows, int64_t cols, const nvfp4_out_t *row,
                                                 const nvfp4_out_t *col, const nvfp4_config_t *cfg_in,
                                                 void *stream) {
  if (num_groups < 1 || num_groups > NVFP4_MAX_GROUPS)
    return fail(NVFP4_ERR_SHAPE, "num_groups = %lld must be in [1, %d]", (long long)num_groups, NVFP4_MAX_GROUPS);
  if (group_rows == nullptr) return fail(NVFP4_ERR_NULL, "group_rows is NULL");
  int64_t rows = 0;
  for (int64_t g = 0; g < num_groups; ++g) {
    if (group_rows[g] < 0 || group_rows[g] >= (int64_t{1} << 32))
      return fail(NVFP4_ERR_SHAPE, "group %lld has %lld rows", (long long)g, (long long)group_rows[g]);
    rows += group_rows[g];
    if (rows >= (int64_t{1} << 32)) return fail(NVFP4_ERR_SHAPE, "too many rows");
  }
  nvfp4_status_t st = check_input(x, dtype, rows, cols);
  if (st != NVFP4_OK) return st;
  const nvfp4_config_t cfg = config_or_default(cfg_in);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (row == nullptr && col == nullptr) return fail(NVFP4_ERR_NULL, "neither a row-wise nor a column-wise output");
  const bool empty = rows * cols == 0;
  if (row && (st = check_out(row, "row-wise", empty)) != NVFP4_OK) return st;
  if (col && (st = check_out(col, "column-wise", empty)) != NVFP4_OK) return st;
  if (cfg.row_scaled) {
    if (col) return fail(NVFP4_ERR_UNSUPPORTED, "grouped row-scaled NVFP4 is row-wise only");
    if (cfg.block_2d) return fail(NVFP4_ERR_UNSUPPORTED, "row-scaled NVFP4 uses 1x16 blocks");
    if (cfg.rht) return fail(NVFP4_ERR_UNSUPPORTED, "row-scaled NVFP4 cannot be combined with the RHT");
    if (cfg.scale_layout == NVFP4_SCALES_GEMM_SWIZZLED)
      return fail(NVFP4_ERR_UNSUPPORTED, "row-scaled NVFP4 keeps compact scales");
  }
  if (cfg.scale_fmt != NVFP4_SCALE_E4M3 && cfg.scale_fmt != NVFP4_SCALE_UE5M3)
    return fail(NVFP4_ERR_UNSUPPORTED, "unknown scale format %u", cfg.scale_fmt);
  if (cfg.scale_layout != NVFP4_SCALES_COMPACT && cfg.scale_layout != NVFP4_SCALES_GEMM_SWIZZLED)
    return fail(NVFP4_ERR_UNSUPPORTED, "unknown scale layout %u", cfg.scale_layout);
  const bool swz = cfg.scale_layout == NVFP4_SCALES_GEMM_SWIZZLED;
  if (cfg.workspace != nullptr && !aligned(cfg.workspace, 16))
    return fail(NVFP4_ERR_ALIGN, "the workspace is not 16-byte aligned");
  if (cfg.rht && cfg.block_2d) return fail(NVFP4_ERR_UNSUPPORTED, "the RHT is defined for 1x16 blocks only");
  if (cfg.rht_bf16 && !cfg.rht) return fail(NVFP4_ERR_UNSUPPORTED, "rht_bf16 needs rht");
  if (cfg.rht && row && col && row->amax == col->amax)
    return fail(NVFP4_ERR_UNSUPPORTED, "the RHT quantize needs distinct row-wise and column-wise amax buffers");
  const int64_t mult = swz ? 128 : ((col || cfg.block_2d || cfg.rht) ? 16 : 1);
  for (int64_t g = 0; g < num_groups; ++g)
    if (group_rows[g] % mult != 0)
      return fail(NVFP4_ERR_SHAPE, "group %lld: %lld rows is not a multiple of %lld", (long long)g,
                  (long long)group_rows[g], (long long)mult);
  if (swz && cols % 128 != 0)
    return fail(NVFP4_ERR_SHAPE, "GEMM-swizzled scales need cols %% 128 == 0 (got %lld)", (long long)cols);

  uint32_t row_start[nvfp4::kMaxGroups + 1];
  row_start[0] = 0;
  for (int64_t g = 0; g < num_groups; ++g) row_start[g + 1] = row_start[g] + static_cast<uint32_t>(group_rows[g]);
  const uint32_t G = static_cast<uint32_t>(num_groups), C = static_cast<uint32_t>(cols);
  const bool sr = cfg.stochastic != 0;
  if (cfg.row_scaled) {  // one fused launch over all rows; amax has one entry per row
    nvfp4::RowScaledArgs a{x, static_cast<uint32_t>(rows), C, row->data, row->scales, row->amax, cfg.sr_seed, cfg.noop};
    a.ue5m3 = cfg.scale_fmt == NVFP4_SCALE_UE5M3;
    return hip_status(nvfp4::launch_rowscaled_grouped(a, row_start, G, dtype, sr, cfg.compute_amax != 0, s),
                      "grouped row-scaled quantize launch");
  }
  float *ra = row ? row->amax : nullptr;
  float *ca = col ? col->amax : nullptr;
  if (cfg.amax_path > NVFP4_AMAX_PATH_SINGLE_PASS)
    return fail(NVFP4_ERR_UNSUPPORTED, "unknown amax path %u", cfg.amax_path);
  // With a workspace (no RHT) and groups of at most kMaxFusedGroupTiles
  // tiles, one launch: each group's tiles hand their maxima to the group's
  // head workgroup and encode from registers (the input is read once).
  uint64_t most_tiles = 0;
  for (uint32_t g = 0; g < G; ++g) {
    const uint64_t n = (uint64_t{row_start[g + 1] - row_start[g]} + 127) / 128 * ((uint64_t{C} + 127) / 128);
    most_tiles = n > most_tiles ? n : most_tiles;
  }
  if (cfg.compute_amax && cfg.workspace != nullptr && !cfg.rht && !empty && cfg.amax_path != NVFP4_AMAX_PATH_TWO_PASS &&
      most_tiles <= nvfp4::kMaxFusedGroupTiles) {
    nvfp4::CastArgs a{x, static_cast<uint32_t>(rows), C, row ? row->data : nullptr, row ? row->scales : nullptr, ra,
                      col ? col->data : nullptr, col ? col->scales : nullptr, ca, swz ? 1u : 0u, cfg.sr_seed,
                      rht_word(cfg), cfg.noop, nullptr, 0};
    a.ue5m3 = cfg.scale_fmt == NVFP4_SCALE_UE5M3;
    return hip_status(nvfp4::launch_grouped_fused(a, row_start, G, dtype, cfg.block_2d != 0, sr,
                                                  static_cast<uint32_t *>(cfg.workspace), s),
                      "grouped one-launch quantize");
  }
  // With a workspace each group's amax workgroups leave their maxima in a
  // range of it (part_start) that the group's cast tiles reduce; without
  // one, the slots are zeroed and reduced by atomic max.
  uint32_t *partials = nullptr;
  uint32_t part_start[nvfp4::kMaxGroups + 1];
  if (cfg.compute_amax) {
    float *a = ra ? ra : ca;
    float *b = (ca == a) ? nullptr : ca;
    if (cfg.workspace != nullptr && !empty) partials = static_cast<uint32_t *>(cfg.workspace);
    else if ((st = hip_status(nvfp4::launch_zero_amax_n(a, b, G, cfg.noop, s), "zero amax launch")) != NVFP4_OK)
      return st;
    if (!empty) {
      uint32_t *ps = partials ? part_start : nullptr;
      if (cfg.rht)
        st = hip_status(nvfp4::launch_rht_amax_grouped(x, dtype, C, row_start, G, rht_word(cfg), ra, ca, partials,
                                                       ps, cfg.noop, s),
                        "RHT amax launch");
      else
        st = hip_status(nvfp4::launch_amax_grouped(x, dtype, C, row_start, G, a, b, partials, ps, cfg.noop, s),
                        "amax launch");
      if (st != NVFP4_OK) return st;
    }
  }
  if (empty) return NVFP4_OK;
  nvfp4::CastArgs a{x, static_cast<uint32_t>(rows), C, row ? row->data : nullptr, row ? row->scales : nullptr, ra,
                    col ? col->data : nullptr, col ? col->scales : nullptr, ca, swz ? 1u : 0u, cfg.sr_seed,
                    rht_word(cfg), cfg.noop, partials, 0};
  a.ue5m3 = cfg.scale_fmt == NVFP4_SCALE_UE5M3;
  return hip_status(nvfp4::launch_cast_grouped(a, row_start, partials ? part_start : nullptr, G, dtype,
                                               cfg.block_2d != 0, cfg.rht != 0, sr, s),
                    "grouped quantize launch");
}

extern "C" nvfp4_status_t nvfp4_dequantize(const nvfp4_out_t *q, int64_t rows, int64_t cols, uint32_t scale_layout,
                                           uint32_t scale_fmt, uint32_t row_scaled, float *y, void *stream) {
  if (q == nullptr || y == nullptr) return fail(NVFP4_ERR_NULL, "NULL quantized tensor or output");
  if (rows < 0 || cols < 0) return fail(NVFP4_ERR_SHAPE, "negative shape");
  if (cols % 16 != 0) return fail(NVFP4_ERR_SHAPE, "cols = %lld is not a multiple of 16", (long long)cols);
  if (product_at_least(rows, cols, uint64_t{1} << 32)) return fail(NVFP4_ERR_SHAPE, "rows * cols must be below 2^32");
  if (rows * cols == 0) return NVFP4_OK;
  if (q->data == nullptr || q->scales == nullptr || q->amax == nullptr)
    return fail(NVFP4_ERR_NULL, "quantized tensor has a NULL data, scales or amax pointer");
  if (!aligned(q->data, 4) || !aligned(q->amax, 4)) return fail(NVFP4_ERR_ALIGN, "data and amax must be 4-byte aligned");
  if (!aligned(y, 16)) return fail(NVFP4_ERR_ALIGN, "output must be 16-byte aligned");
  if (scale_layout != NVFP4_SCALES_COMPACT && scale_layout != NVFP4_SCALES_GEMM_SWIZZLED)
    return fail(NVFP4_ERR_UNSUPPORTED, "unknown scale layout %u", scale_layout);
  if (scale_fmt != NVFP4_SCALE_E4M3 && scale_fmt != NVFP4_SCALE_UE5M3)
    return fail(NVFP4_ERR_UNSUPPORTED, "unknown scale format %u", scale_fmt);
  const bool swz = scale_layout == NVFP4_SCALES_GEMM_SWIZZLED;
  if (swz && (rows % 128 != 0 || cols % 128 != 0))
    return fail(NVFP4_ERR_SHAPE, "GEMM-swizzled scales need rows and cols that are multiples of 128");
  if (row_scaled && swz) return fail(NVFP4_ERR_UNSUPPORTED, "row-scaled NVFP4 keeps compact scales");
  return hip_status(nvfp4::launch_dequant(q->data, q->scales, q->amax, static_cast<uint32_t>(rows),
                                          static_cast<uint32_t>(cols), swz, row_scaled != 0,
                                          scale_fmt == NVFP4_SCALE_UE5M3, y,
                                          static_cast<hipStream_t>(stream)),
                    "dequantize launch");
}

extern "C" nvfp4_status_t nvfp4_debug_rht_colwise(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t cols,
                                                  uint32_t sign_mask, float *t, void *stream) {
  nvfp4_status_t st = check_input(x, dtype, rows, cols);
  if (st != NVFP4_OK) return st;
  if (rows % 16 != 0) return fail(NVFP4_ERR_SHAPE, "the RHT needs rows %% 16 == 0");
  if (rows * cols > 0 && t == nullptr) return fail(NVFP4_ERR_NULL, "output pointer is NULL");
  if (t != nullptr && !aligned(t, 16)) return fail(NVFP4_ERR_ALIGN, "output must be 16-byte aligned");
  return hip_status(nvfp4::launch_debug_rht(x, dtype, static_cast<uint32_t>(rows), static_cast<uint32_t>(cols),
                                            sign_mask & (0xFFFFu | nvfp4::kRhtBf16), t,
                                            static_cast<hipStream_t>(stream)),
                    "RHT launch");
}

extern "C" nvfp4_status_t nvfp4_debug_e2m1_pack(const float *v, const uint32_t *r, uint8_t *out, int64_t n,
                                                uint32_t flags, void *stream) {
  if (n < 0 || n >= (int64_t{1} << 32)) return fail(NVFP4_ERR_SHAPE, "pair count %lld out of range", (long long)n);
  if (flags & ~(NVFP4_DEBUG_SR | NVFP4_DEBUG_PAIRWISE)) return fail(NVFP4_ERR_UNSUPPORTED, "unknown flags %#x", flags);
  const bool sr = (flags & NVFP4_DEBUG_SR) != 0;
  if (n > 0 && (v == nullptr || out == nullptr || (sr && r == nullptr)))
    return fail(NVFP4_ERR_NULL, "a required pointer is NULL");
  if (!aligned(v, 4) || !aligned(r, 4)) return fail(NVFP4_ERR_ALIGN, "v and r must be 4-byte aligned");
  return hip_status(nvfp4::launch_debug_e2m1(v, r, out, static_cast<uint64_t>(n), sr, (flags & NVFP4_DEBUG_PAIRWISE) != 0,
                                             static_cast<hipStream_t>(stream)),
                    "debug e2m1 launch");
}
