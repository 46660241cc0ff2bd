// Amax kernels: the zeroing pass, the per-tensor max|x| reduction that fills
// both amax buffers, and the RHT pair (max|x| and max|RHT(x)|) from one read;
// each also in a grouped form (one amax per row slice of the input, group
// table in the kernel arguments).
//
// "Write both NVFP4 amax buffers" (Description, Changes): the zeroing kernel
// clears both buffers and each block's atomic max goes into both, so no
// copy and no second read are needed. Max is exact and order-free; on
// non-negative binary32 values an unsigned integer max of the bit patterns
// is the float max, so each workgroup ends with one global_atomic_umax per
// buffer on the +0.0 that the zeroing pass wrote. With a caller workspace
// the workgroups store their maxima there instead and the cast kernel
// reduces them, which needs neither the zeroing pass nor atomics.

#include <atomic>

#include "codec.h"
#include "launch.h"

namespace nvfp4 {

namespace {
std::atomic<uint32_t> g_rht_unit{0};
}  // namespace

void set_rht_unit(uint32_t unit) { g_rht_unit.store(unit, std::memory_order_relaxed); }
bool rht_cast_on_matrix_cores() { return g_rht_unit.load(std::memory_order_relaxed) != 1; }
bool rht_amax_on_matrix_cores() { return g_rht_unit.load(std::memory_order_relaxed) == 2; }

namespace {

constexpr int kThreads = 256;

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bool noop_set(const float *noop) { return noop != nullptr && *noop == 1.0f; }

// max over the NT threads of a workgroup (values are float bit patterns of
// non-negative numbers, so unsigned max == float max). Result valid in all
// threads; lds holds one word per wave.
template <int NT>
__device__ __forceinline__ uint32_t block_umax(uint32_t v, uint32_t *lds) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64)));
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
  __syncthreads();
  v = lds[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) v = max(v, lds[i]);
  return v;
}

// Apply a workgroup's maximum to an amax buffer. Same-address atomics from
// thousands of workgroups serialize at the memory side across the XCDs, so a
// workgroup first reads the buffer (system scope: past every cache) and
// issues the atomic max only when its value is larger. The buffer only grows
// during the reduction (from the +0 of the zeroing pass), so a value that is
// not larger than one already there cannot change the result.
__device__ __forceinline__ void publish_max(float *dst, uint32_t m) {
  if (dst == nullptr) return;
  unsigned int *u = reinterpret_cast<unsigned int *>(dst);
  if (m > __hip_atomic_load(u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)) atomicMax(u, m);
}

__global__ void k_zero_amax(float *a, float *b, const float *noop) {
  if (noop_set(noop)) return;
  if (threadIdx.x == 0) {
    if (a) *a = 0.0f;
    if (b) *b = 0.0f;
  }
}

// Per-tensor amax. nvec = number of 16-byte vectors of x. The grid reads x
// in passes of VPT grid-wide contiguous spans: in each pass thread t of the
// grid loads vectors t, t + span, ..., t + (VPT - 1) * span (span = grid size
// in threads), all issued before any is used, so every wave keeps VPT
// 16-byte loads in flight and consecutive waves read consecutive memory.
// The workgroup's maximum then goes either to partials[blockIdx.x] (plain
// store; the cast kernel finishes the reduction) or, with partials == NULL,
// into a and b by atomic max.
constexpr int kAmaxThreads = 256;     // RHT amax pair (512 and 1024 measured slower, 64 and 128 the same)
constexpr int kMaxThreads = 256;      // per-tensor amax
constexpr int kMaxVecPerThread = 8;   // loads in flight per thread and pass
constexpr uint32_t kMaxGrid = 1280;   // 5 workgroups per CU on 256 CUs
// The form that publishes by atomics takes workgroups four times as large
// (the same threads and loads in flight): every workgroup's publish reads
// the amax word past the caches, and those reads of one word serialize
// (8192x5120 BF16: 23.5 -> 19.6 us per nvfp4_compute_amax call; half as many
// of these workgroups, 23.2 us). The form with a workspace stays at 256
// threads, where it measured faster (the two-pass 8192x5120 16x16 call:
// 36.4 against 38.1 us).
constexpr int kMaxThreadsAtomic = 1024;
constexpr uint32_t kMaxGridAtomic = kMaxGrid * kMaxThreads / kMaxThreadsAtomic;
// RHT amax pair without a workspace: workgroups loop over 16-row units
// (8192x5120 BF16 nvfp4_compute_amax: 38.2 us with a workgroup per unit,
// 35.6 with at most 2048 workgroups, 27.8 with 1024, 20.5-21.3 with 512,
// 21.4-21.7 with 384, 27.1 with 256)
constexpr uint32_t kMaxGridRhtAtomic = 512;
static_assert(kMaxGroups <= kMaxGridRhtAtomic, "one workgroup per group fits the grouped atomic grid");

template <int DT, int NT>
__global__ __launch_bounds__(NT) void k_amax(const uint4 *__restrict__ x, uint64_t nvec, float *a, float *b,
                                             uint32_t *partials, const float *noop) {
  constexpr int VPT = kMaxVecPerThread;
  __shared__ uint32_t lds[NT / 64];
  if (noop_set(noop)) return;
  uint32_t m32 = 0;        // FP32: max of |x| bit patterns
  ushort2_t m16 = {0, 0};  // BF16: max of 15-bit magnitudes, two lanes
  const uint64_t span = static_cast<uint64_t>(gridDim.x) * NT;
  for (uint64_t i0 = static_cast<uint64_t>(blockIdx.x) * NT + threadIdx.x; i0 < nvec; i0 += span * VPT) {
    uint4 v[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const uint64_t i = i0 + k * span;
      v[k] = i < nvec ? x[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (DT == kBF16)
          m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(ushort2_t, w[j] & 0x7FFF7FFFu));
        else
          m32 = max(m32, w[j] & 0x7FFFFFFFu);
      }
    }
  }
  uint32_t m = DT == kBF16 ? (static_cast<uint32_t>(max(m16.x, m16.y)) << 16) : m32;
  m = block_umax<NT>(m, lds);
  if (threadIdx.x == 0) {
    if (partials != nullptr) {
      partials[blockIdx.x] = m;
    } else {
      publish_max(a, m);
      if (b != a) publish_max(b, m);
    }
  }
}

// Load the 16 x VEC values of one thread's column strip (rows g*16 .. +15,
// columns c .. c+VEC-1) as floats v[col][row].
template <int DT, int VEC>
__device__ __forceinline__ void load_strip(const void *x, uint32_t cols, uint32_t r0, uint32_t c,
                                           float (&v)[VEC][16]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint64_t off = static_cast<uint64_t>(r0 + r) * cols + c;
    if (DT == kBF16) {
      const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + off);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k][r] = bf16_lo(w[k]);
        v[2 * k + 1][r] = bf16_hi(w[k]);
      }
    } else {
      const float4 q = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + off);
      v[0][r] = q.x;
      v[1][r] = q.y;
      v[2][r] = q.z;
      v[3][r] = q.w;
    }
  }
}

// One RHT amax unit: this thread's 4 columns c .. c+3 of rows 16 by .. +15.
// Accumulates max|x| (mx16 / mx32 by input type) and max|unnormalized
// transform| (ms).
// MFMA (BF16 only): the transform on the matrix cores (fwht16_mfma, with the
// lane's operands a1 / a2 for the mask), else butterflies on the vector ALU.
template <int DT, bool MFMA>
__device__ __forceinline__ void rht_amax_unit(const void *__restrict__ x, uint32_t cols, uint32_t by, uint32_t c,
                                              uint32_t mask, const uint32_t (&a1)[4][2], const float (&a2)[4],
                                              ushort2_t &mx16, uint32_t &mx32, uint32_t &ms) {
  static_assert(!MFMA || DT == kBF16, "the matrix-core transform takes BF16 input");
  constexpr int VEC = 4;
  constexpr int W = DT == kBF16 ? 2 : 4;  // 32-bit words per 4-column row piece
  constexpr uint32_t kAbs = DT == kBF16 ? 0x7FFF7FFFu : 0x7FFFFFFFu;
  constexpr uint32_t kSign = DT == kBF16 ? 0x80008000u : 0x80000000u;
  uint32_t w[16][W];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint8_t *src = static_cast<const uint8_t *>(x) +
                         (static_cast<uint64_t>(by * 16 + r) * cols + c) * (DT == kBF16 ? 2 : 4);
    if constexpr (DT == kBF16) {
      const uint2 t = *reinterpret_cast<const uint2 *>(src);
      w[r][0] = t.x;
      w[r][1] = t.y;
    } else {
      const uint4 t = *reinterpret_cast<const uint4 *>(src);
      w[r][0] = t.x;
      w[r][1] = t.y;
      w[r][2] = t.z;
      w[r][3] = t.w;
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
#pragma unroll
    for (int q = 0; q < W; ++q) {
      if constexpr (DT == kBF16)
        mx16 = __builtin_elementwise_max(mx16, __builtin_bit_cast(ushort2_t, w[r][q] & kAbs));
      else
        mx32 = max(mx32, w[r][q] & kAbs);
      if constexpr (!MFMA) w[r][q] ^= ((mask >> r) & 1u) ? kSign : 0u;  // uniform select
    }
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    float v[16];
    if constexpr (MFMA) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;  // column j's halves, rows paired
      uint32_t x2[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        x2[g][0] = __builtin_amdgcn_perm(w[4 * g + 1][j >> 1], w[4 * g][j >> 1], sel);
        x2[g][1] = __builtin_amdgcn_perm(w[4 * g + 3][j >> 1], w[4 * g + 2][j >> 1], sel);
      }
      fwht16_mfma(x2, a1, a2, v);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (DT == kBF16)
          v[r] = (j & 1) ? bf16_hi(w[r][j >> 1]) : bf16_lo(w[r][j >> 1]);
        else
          v[r] = __uint_as_float(w[r][j]);
      }
      fwht16(v);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) ms = max(ms, __float_as_uint(v[r]) & 0x7FFFFFFFu);  // NaN stays NaN
  }
}

// One unit at column c of every lane of the wave (c >= cols: nothing). With
// the matrix cores every lane takes part in the transform (a lane that sat
// out would leave its block of four lanes without its operands), so a lane
// past the end transforms a clamped column and keeps its maxima.
template <int DT, bool MFMA>
__device__ __forceinline__ void rht_amax_step(const void *__restrict__ x, uint32_t cols, uint32_t by, uint32_t c,
                                              uint32_t mask, const uint32_t (&a1)[4][2], const float (&a2)[4],
                                              ushort2_t &mx16, uint32_t &mx32, uint32_t &ms) {
  if constexpr (MFMA) {
    ushort2_t mx16_u = mx16;
    uint32_t ms_u = ms;
    rht_amax_unit<DT, MFMA>(x, cols, by, c < cols ? c : 0u, mask, a1, a2, mx16_u, mx32, ms_u);
    if (c < cols) {
      mx16 = mx16_u;
      ms = ms_u;
    }
  } else {
    if (c < cols) rht_amax_unit<DT, MFMA>(x, cols, by, c, mask, a1, a2, mx16, mx32, ms);
  }
}

// Workgroup maxima of an RHT amax pass: (max|x|, max|t|) as float bits, in
// every thread.
template <int DT>
__device__ __forceinline__ void rht_amax_finish(ushort2_t mx16, uint32_t mx32, uint32_t ms, uint32_t mask, uint32_t *lds,
                                                uint32_t &mx, uint32_t &mt) {
  mx = DT == kBF16 ? (static_cast<uint32_t>(max(mx16.x, mx16.y)) << 16) : mx32;
  float t = __uint_as_float(ms) * 0.25f;
  if (mask & kRhtBf16) {  // rounding is monotonic: max|bf16(t)| == bf16(max|t|)
    float unused = 0.0f;
    bf16_round_pair(t, unused);
  }
  mt = __float_as_uint(t);
  mx = block_umax<kAmaxThreads>(mx, lds);
  __syncthreads();
  mt = block_umax<kAmaxThreads>(mt, lds);
}

// RHT amax pair. The input is cut into units of 16 rows x (kAmaxThreads * 4)
// columns, gx units across; a workgroup reduces units blockIdx.x,
// blockIdx.x + gridDim.x, ... Each thread loads 4 adjacent columns of one
// 16-row group as raw words: max|x| comes from the words themselves, the
// sign flips of the transform are applied to whole words (one sign per row),
// and each column's 16 values then go through the unnormalized transform.
// max|t| = fl(max|sum| / 4): scaling by 1/4 is exact up to rounding in the
// denormal range, and rounding is monotonic, so this is the maximum of the
// transformed values t = fl(sum / 4) themselves. Results go to
// partials[blockIdx.x] and partials[kMaxPartials + blockIdx.x], or with
// partials == NULL (one unit per workgroup) into row_amax and col_amax by
// atomic max.
template <int DT, bool MFMA>
__global__ __launch_bounds__(kAmaxThreads) void k_rht_amax(const void *__restrict__ x, uint32_t rows, uint32_t cols,
                                                       uint32_t gx, uint32_t units, uint32_t mask, float *row_amax,
                                                       float *col_amax, uint32_t *partials, const float *noop) {
  __shared__ uint32_t lds[kAmaxThreads / 64];
  if (noop_set(noop)) return;
  ushort2_t mx16 = {0, 0};  // BF16 max|x|, two lanes
  uint32_t mx32 = 0;        // FP32 max|x| bits
  uint32_t ms = 0;          // max |unnormalized transform| (bit pattern)
  uint32_t a1[4][2] = {};
  float a2[4] = {};
  if constexpr (MFMA) fwht16_mfma_operands(mask, a1, a2);
  for (uint32_t u = blockIdx.x; u < units; u += gridDim.x) {
    const uint32_t by = u / gx;
    const uint32_t c = ((u - by * gx) * kAmaxThreads + threadIdx.x) * 4;
    rht_amax_step<DT, MFMA>(x, cols, by, c, mask, a1, a2, mx16, mx32, ms);
  }
  uint32_t mx, mt;
  rht_amax_finish<DT>(mx16, mx32, ms, mask, lds, mx, mt);
  if (threadIdx.x == 0) {
    if (partials != nullptr) {
      partials[blockIdx.x] = mx;
      partials[kMaxPartials + blockIdx.x] = mt;
    } else {
      publish_max(row_amax, mx);
      publish_max(col_amax, mt);
    }
  }
}

// Slots of empty groups: in the workspace form no cast tile writes them.
__device__ __forceinline__ void zero_empty_groups(const GroupTable &t, float *a, float *b) {
  for (uint32_t g = threadIdx.x; g < t.ngroups; g += blockDim.x) {
    if (t.row_start[g + 1] == t.row_start[g]) {
      if (a) a[g] = 0.0f;
      if (b) b[g] = 0.0f;
    }
  }
}

// Grouped RHT amax pair. Workgroup b of group g (b in unit_start[g] ..
// unit_start[g + 1] - 1) takes `per_wg` consecutive units of that group
// (gx across, m_g / 16 down; units past the group's end are empty). Results
// go to partials[b] and partials[kMaxPartials + b], or with partials == NULL
// into the group's slots by atomic max.
template <int DT, bool MFMA>
__global__ __launch_bounds__(kAmaxThreads) void k_rht_amax_grouped(const void *__restrict__ x, uint32_t cols,
                                                               uint32_t gx, GroupTable t, uint32_t per_wg,
                                                               uint32_t mask, float *row_amax, float *col_amax,
                                                               uint32_t *partials, const float *noop) {
  __shared__ uint32_t lds[kAmaxThreads / 64];
  if (noop_set(noop)) return;
  if (partials != nullptr && blockIdx.x == 0) zero_empty_groups(t, row_amax, col_amax);
  const uint32_t g = group_of(t, blockIdx.x);
  const uint32_t units = gx * ((t.row_start[g + 1] - t.row_start[g]) / 16);
  const void *xg = static_cast<const uint8_t *>(x) + static_cast<uint64_t>(t.row_start[g]) * cols * (DT == kBF16 ? 2 : 4);
  ushort2_t mx16 = {0, 0};
  uint32_t mx32 = 0;
  uint32_t ms = 0;
  uint32_t a1[4][2] = {};
  float a2[4] = {};
  if constexpr (MFMA) fwht16_mfma_operands(mask, a1, a2);
  const uint32_t u0 = (blockIdx.x - t.unit_start[g]) * per_wg;
  for (uint32_t u = u0; u < u0 + per_wg && u < units; ++u) {
    const uint32_t by = u / gx;
    const uint32_t c = ((u - by * gx) * kAmaxThreads + threadIdx.x) * 4;
    rht_amax_step<DT, MFMA>(xg, cols, by, c, mask, a1, a2, mx16, mx32, ms);
  }
  uint32_t mx, mt;
  rht_amax_finish<DT>(mx16, mx32, ms, mask, lds, mx, mt);
  if (threadIdx.x == 0) {
    if (partials != nullptr) {
      partials[blockIdx.x] = mx;
      partials[kMaxPartials + blockIdx.x] = mt;
    } else {
      if (row_amax) publish_max(row_amax + g, mx);
      if (col_amax) publish_max(col_amax + g, mt);
    }
  }
}

// Grouped per-tensor amax. The n_g = unit_start[g + 1] - unit_start[g]
// workgroups of group g read its rows as k_amax reads a tensor: grid-wide
// (here group-wide) contiguous spans, kMaxVecPerThread loads per thread in
// flight. Result to partials[b], or with partials == NULL into the group's
// slots by atomic max.
template <int DT, int NT>
__global__ __launch_bounds__(NT) void k_amax_grouped(const uint4 *__restrict__ x, uint32_t vec_per_row, GroupTable t,
                                                     float *a, float *b, uint32_t *partials, const float *noop) {
  constexpr int VPT = kMaxVecPerThread;
  __shared__ uint32_t lds[NT / 64];
  if (noop_set(noop)) return;
  if (partials != nullptr && blockIdx.x == 0) zero_empty_groups(t, a, b);
  const uint32_t g = group_of(t, blockIdx.x);
  const uint64_t first = static_cast<uint64_t>(t.row_start[g]) * vec_per_row;
  const uint64_t nvec = static_cast<uint64_t>(t.row_start[g + 1] - t.row_start[g]) * vec_per_row;
  const uint64_t span = static_cast<uint64_t>(t.unit_start[g + 1] - t.unit_start[g]) * NT;
  uint32_t m32 = 0;
  ushort2_t m16 = {0, 0};
  for (uint64_t i0 = static_cast<uint64_t>(blockIdx.x - t.unit_start[g]) * NT + threadIdx.x; i0 < nvec;
       i0 += span * VPT) {
    // all loads in flight at once: past the group's end the index is
    // clamped to its last vector, which cannot change a maximum
    uint4 v[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) v[k] = x[first + min(i0 + k * span, nvec - 1)];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (DT == kBF16)
          m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(ushort2_t, w[j] & 0x7FFF7FFFu));
        else
          m32 = max(m32, w[j] & 0x7FFFFFFFu);
      }
    }
  }
  uint32_t m = DT == kBF16 ? (static_cast<uint32_t>(max(m16.x, m16.y)) << 16) : m32;
  m = block_umax<NT>(m, lds);
  if (threadIdx.x == 0) {
    if (partials != nullptr) {
      partials[blockIdx.x] = m;
    } else {
      if (a) publish_max(a + g, m);
      if (b && b != a) publish_max(b + g, m);
    }
  }
}

__global__ void k_zero_amax_n(float *a, float *b, uint32_t n, const float *noop) {
  if (noop_set(noop)) return;
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
    if (a) a[i] = 0.0f;
    if (b) b[i] = 0.0f;
  }
}

// Column-wise RHT image t[cols][rows] (test hook; same transform code).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_debug_rht(const void *__restrict__ x, uint32_t rows, uint32_t cols,
                                                        uint32_t mask, float *__restrict__ t) {
  constexpr int VEC = DT == kBF16 ? 8 : 4;
  const uint32_t c = (blockIdx.x * kThreads + threadIdx.x) * VEC;
  const uint32_t r0 = blockIdx.y * 16;
  if (c >= cols) return;
  float v[VEC][16];
  load_strip<DT, VEC>(x, cols, r0, c, v);
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    rht16(v[j], mask);
    if (mask & kRhtBf16) bf16_round16(v[j]);
    float4 *dst = reinterpret_cast<float4 *>(t + static_cast<uint64_t>(c + j) * rows + r0);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_float4(v[j][4 * q], v[j][4 * q + 1], v[j][4 * q + 2], v[j][4 * q + 3]);
  }
}

}  // namespace

hipError_t launch_zero_amax(float *a, float *b, const float *noop, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_amax, dim3(1), dim3(64), 0, s, a, b, noop);
  return hipGetLastError();
}

namespace {

// Grid of a reduction over `work` units: one unit per workgroup for the
// atomic form; for the workspace form at most kMaxPartials workgroups, padded
// to a multiple of kPartialsGrain (the extra workgroups store +0).
uint32_t reduction_grid(uint64_t work, bool to_partials) {
  // the form without a workspace publishes each workgroup's maximum by a
  // read of the amax word past the caches, and those reads of one word
  // serialize: at most kMaxGridRhtAtomic workgroups there
  if (!to_partials) return static_cast<uint32_t>(work < kMaxGridRhtAtomic ? work : kMaxGridRhtAtomic);
  const uint64_t g = (work + kPartialsGrain - 1) / kPartialsGrain * kPartialsGrain;
  return static_cast<uint32_t>(g < kMaxPartials ? g : kMaxPartials);
}

}  // namespace

hipError_t launch_amax(const void *x, int dtype, uint64_t n, float *a, float *b, uint32_t *partials,
                       uint32_t *npartials, const float *noop, hipStream_t s) {
  const uint64_t nvec = n * (dtype == kBF16 ? 2 : 4) / 16;
  if (nvec == 0) return hipSuccess;
  // one pass of kMaxVecPerThread loads per thread covers the input when it
  // fits; at most kMaxGrid (kMaxGridAtomic) workgroups
  const uint32_t nt = partials != nullptr ? kMaxThreads : kMaxThreadsAtomic;
  const uint32_t cap = partials != nullptr ? kMaxGrid : kMaxGridAtomic;
  const uint64_t want = (nvec + uint64_t{nt} * kMaxVecPerThread - 1) / (uint64_t{nt} * kMaxVecPerThread);
  uint32_t grid = static_cast<uint32_t>(want < cap ? want : cap);
  if (partials != nullptr) grid = reduction_grid(grid, true);
  if (npartials) *npartials = grid;
  const uint4 *xv = static_cast<const uint4 *>(x);
  if (partials != nullptr) {
    if (dtype == kBF16)
      hipLaunchKernelGGL((k_amax<kBF16, kMaxThreads>), dim3(grid), dim3(nt), 0, s, xv, nvec, a, b, partials, noop);
    else
      hipLaunchKernelGGL((k_amax<kFP32, kMaxThreads>), dim3(grid), dim3(nt), 0, s, xv, nvec, a, b, partials, noop);
  } else {
    if (dtype == kBF16)
      hipLaunchKernelGGL((k_amax<kBF16, kMaxThreadsAtomic>), dim3(grid), dim3(nt), 0, s, xv, nvec, a, b, partials,
                         noop);
    else
      hipLaunchKernelGGL((k_amax<kFP32, kMaxThreadsAtomic>), dim3(grid), dim3(nt), 0, s, xv, nvec, a, b, partials,
                         noop);
  }
  return hipGetLastError();
}

hipError_t launch_rht_amax(const void *x, int dtype, uint32_t rows, uint32_t cols, uint32_t mask,
                           float *row_amax, float *col_amax, uint32_t *partials, uint32_t *npartials,
                           const float *noop, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const uint32_t gx = (cols + kAmaxThreads * 4 - 1) / (kAmaxThreads * 4);
  const uint32_t units = gx * (rows / 16);  // < 2^32: rows * cols < 2^32
  const uint32_t grid = reduction_grid(units, partials != nullptr);
  if (npartials) *npartials = grid;
  if (dtype == kBF16 && rht_amax_on_matrix_cores())
    hipLaunchKernelGGL((k_rht_amax<kBF16, true>), dim3(grid), dim3(kAmaxThreads), 0, s, x, rows, cols, gx, units,
                       mask, row_amax, col_amax, partials, noop);
  else if (dtype == kBF16)
    hipLaunchKernelGGL((k_rht_amax<kBF16, false>), dim3(grid), dim3(kAmaxThreads), 0, s, x, rows, cols, gx, units,
                       mask, row_amax, col_amax, partials, noop);
  else
    hipLaunchKernelGGL((k_rht_amax<kFP32, false>), dim3(grid), dim3(kAmaxThreads), 0, s, x, rows, cols, gx, units,
                       mask, row_amax, col_amax, partials, noop);
  return hipGetLastError();
}

hipError_t launch_zero_amax_n(float *a, float *b, uint32_t n, const float *noop, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_amax_n, dim3(1), dim3(256), 0, s, a, b, n, noop);
  return hipGetLastError();
}

namespace {

// Work units per group for a grouped amax pass: `work[g]` units of group g,
// `per` of them per workgroup. `per` doubles until the workgroups fit:
// kMaxPartials in total for the workspace form (each group's count padded to
// a multiple of kPartialsGrain), kMaxGridRhtAtomic for the atomic form.
uint32_t plan_groups(const uint64_t *work, uint32_t ngroups, bool to_partials, GroupTable &t) {
  uint32_t per = 1;
  for (;;) {
    uint64_t total = 0;
    t.unit_start[0] = 0;
    for (uint32_t g = 0; g < ngroups; ++g) {
      uint64_t n = (work[g] + per - 1) / per;
      if (to_partials) n = (n + kPartialsGrain - 1) / kPartialsGrain * kPartialsGrain;
      total += n;
      t.unit_start[g + 1] = static_cast<uint32_t>(total < 0xFFFFFFFFull ? total : 0xFFFFFFFFull);
    }
    // the workspace form's workgroups fit its slots; the atomic form's stay
    // few, since their publishes serialize (ngroups <= kMaxGroups keeps both
    // reachable with one workgroup per group)
    if (total <= (to_partials ? kMaxPartials : kMaxGridRhtAtomic)) return per;
    per *= 2;
  }
}

// Workgroups per group for the per-tensor amax: shares of about `target`
// (the pass's grid cap) in proportion to each group's chunks (at least one,
// at most its chunk count), so that the whole pass runs as one k_amax over
// the tensor would.
// The workspace form pads each share to a multiple of kPartialsGrain and
// lowers the target so that the sum stays within kMaxPartials:
// sum <= target + ngroups (rounding up) + 3 ngroups (padding).
void share_groups(const uint64_t *work, uint32_t ngroups, bool to_partials, GroupTable &t,
                  uint64_t target = kMaxGrid) {
  uint64_t total = 0;
  for (uint32_t g = 0; g < ngroups; ++g) total += work[g];
  if (to_partials && target + 4ull * ngroups > kMaxPartials) target = kMaxPartials - 4ull * ngroups;
  t.unit_start[0] = 0;
  for (uint32_t g = 0; g < ngroups; ++g) {
    uint64_t n = 0;
    if (work[g] > 0) {
      n = (target * work[g] + total - 1) / total;
      n = n < 1 ? 1 : (n > work[g] ? work[g] : n);
      if (to_partials) n = (n + kPartialsGrain - 1) / kPartialsGrain * kPartialsGrain;
    }
    t.unit_start[g + 1] = t.unit_start[g] + static_cast<uint32_t>(n);
  }
}

}  // namespace

hipError_t launch_amax_grouped(const void *x, int dtype, uint32_t cols, const uint32_t *row_start, uint32_t ngroups,
                               float *a, float *b, uint32_t *partials, uint32_t *part_start, const float *noop,
                               hipStream_t s) {
  GroupTable t{};
  t.ngroups = ngroups;
  const uint32_t vec_per_row = cols * (dtype == kBF16 ? 2 : 4) / 16;
  // the form without a workspace takes the per-tensor pass's larger
  // workgroups (fewer publishes: the groups' amax words share a few lines)
  const bool atomic = partials == nullptr;
  const uint32_t nt = atomic ? kMaxThreadsAtomic : kMaxThreads;
  const uint64_t chunk = uint64_t{nt} * kMaxVecPerThread;
  uint64_t work[kMaxGroups];
  for (uint32_t g = 0; g <= ngroups; ++g) t.row_start[g] = row_start[g];
  for (uint32_t g = 0; g < ngroups; ++g)
    work[g] = (static_cast<uint64_t>(row_start[g + 1] - row_start[g]) * vec_per_row + chunk - 1) / chunk;
  share_groups(work, ngroups, !atomic, t, atomic ? kMaxGridAtomic : kMaxGrid);
  if (part_start)
    for (uint32_t g = 0; g <= ngroups; ++g) part_start[g] = t.unit_start[g];
  const uint32_t grid = t.unit_start[ngroups] > 0 ? t.unit_start[ngroups] : (partials ? 1u : 0u);
  if (grid == 0) return hipSuccess;
  const uint4 *xv = static_cast<const uint4 *>(x);
  if (!atomic) {
    if (dtype == kBF16)
      hipLaunchKernelGGL((k_amax_grouped<kBF16, kMaxThreads>), dim3(grid), dim3(nt), 0, s, xv, vec_per_row, t, a, b,
                         partials, noop);
    else
      hipLaunchKernelGGL((k_amax_grouped<kFP32, kMaxThreads>), dim3(grid), dim3(nt), 0, s, xv, vec_per_row, t, a, b,
                         partials, noop);
  } else {
    if (dtype == kBF16)
      hipLaunchKernelGGL((k_amax_grouped<kBF16, kMaxThreadsAtomic>), dim3(grid), dim3(nt), 0, s, xv, vec_per_row, t, a,
                         b, partials, noop);
    else
      hipLaunchKernelGGL((k_amax_grouped<kFP32, kMaxThreadsAtomic>), dim3(grid), dim3(nt), 0, s, xv, vec_per_row, t, a,
                         b, partials, noop);
  }
  return hipGetLastError();
}

hipError_t launch_rht_amax_grouped(const void *x, int dtype, uint32_t cols, const uint32_t *row_start,
                                   uint32_t ngroups, uint32_t mask, float *row_amax, float *col_amax,
                                   uint32_t *partials, uint32_t *part_start, const float *noop, hipStream_t s) {
  GroupTable t{};
  t.ngroups = ngroups;
  const uint32_t gx = (cols + kAmaxThreads * 4 - 1) / (kAmaxThreads * 4);
  uint64_t work[kMaxGroups];
  for (uint32_t g = 0; g <= ngroups; ++g) t.row_start[g] = row_start[g];
  for (uint32_t g = 0; g < ngroups; ++g) work[g] = static_cast<uint64_t>(gx) * ((row_start[g + 1] - row_start[g]) / 16);
  const uint32_t per_wg = plan_groups(work, ngroups, partials != nullptr, t);
  if (part_start)
    for (uint32_t g = 0; g <= ngroups; ++g) part_start[g] = t.unit_start[g];
  const uint32_t grid = t.unit_start[ngroups] > 0 ? t.unit_start[ngroups] : (partials ? 1u : 0u);
  if (grid == 0) return hipSuccess;
  if (dtype == kBF16 && rht_amax_on_matrix_cores())
    hipLaunchKernelGGL((k_rht_amax_grouped<kBF16, true>), dim3(grid), dim3(kAmaxThreads), 0, s, x, cols, gx, t, per_wg,
                       mask, row_amax, col_amax, partials, noop);
  else if (dtype == kBF16)
    hipLaunchKernelGGL((k_rht_amax_grouped<kBF16, false>), dim3(grid), dim3(kAmaxThreads), 0, s, x, cols, gx, t,
                       per_wg, mask, row_amax, col_amax, partials, noop);
  else
    hipLaunchKernelGGL((k_rht_amax_grouped<kFP32, false>), dim3(grid), dim3(kAmaxThreads), 0, s, x, cols, gx, t,
                       per_wg, mask, row_amax, col_amax, partials, noop);
  return hipGetLastError();
}

hipError_t launch_debug_rht(const void *x, int dtype, uint32_t rows, uint32_t cols, uint32_t mask, float *t,
                            hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const uint32_t vec = dtype == kBF16 ? 8 : 4;
  dim3 grid((cols + kThreads * vec - 1) / (kThreads * vec), rows / 16);
  if (dtype == kBF16)
    hipLaunchKernelGGL(k_debug_rht<kBF16>, grid, dim3(kThreads), 0, s, x, rows, cols, mask, t);
  else
    hipLaunchKernelGGL(k_debug_rht<kFP32>, grid, dim3(kThreads), 0, s, x, rows, cols, mask, t);
  return hipGetLastError();
}

}  // namespace nvfp4
