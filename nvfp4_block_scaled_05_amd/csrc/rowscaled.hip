// Row-scaled (per-token) NVFP4 quantize for gfx950: one workgroup per row.
//
// "Implement row-scaled NVFP4 fprop recipe" (Changes, Greptile summary): each
// row gets its own FP32 amax and the E4M3 block scales are taken relative to
// it; output is row-wise only with compact scales. There the row amax is a
// separate kernel run before the quantize kernel. Here the two are one
// kernel: a row of up to 256 x 4 units of 8 elements (8192 elements) stays
// in registers between the reduction and the cast, so the input is read from
// HBM once. Longer rows re-read the part beyond that from cache.
#include "codec.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kRegUnits = 4;  // units of 8 elements kept in registers per thread

template <int DT>
struct Unit {
  static constexpr int kWords = DT == kBF16 ? 4 : 8;
  uint32_t w[kWords];
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// NT: non-temporal (the part of a row that stays in registers is read once);
// the part beyond that is read twice and goes through the caches.
template <int DT, bool NT>
__device__ __forceinline__ Unit<DT> load_unit(const void *x, uint64_t elem_off) {
  Unit<DT> u;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(x) + elem_off * (DT == kBF16 ? 2 : 4));
#pragma unroll
  for (int q = 0; q < Unit<DT>::kWords / 4; ++q) {
    const u32x4 t = NT ? __builtin_nontemporal_load(src + q) : src[q];
    u.w[4 * q] = t.x;
    u.w[4 * q + 1] = t.y;
    u.w[4 * q + 2] = t.z;
    u.w[4 * q + 3] = t.w;
  }
  return u;
}

template <int DT>
__device__ __forceinline__ void unit_values(const Unit<DT> &u, float (&v)[8]) {
  if (DT == kBF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_lo(u.w[k]);
      v[2 * k + 1] = bf16_hi(u.w[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __uint_as_float(u.w[k]);
  }
}

template <int DT>
__device__ __forceinline__ uint32_t unit_max_bits(const Unit<DT> &u) {
  float v[8];
  unit_values<DT>(u, v);
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = max(m, __float_as_uint(v[k]) & 0x7FFFFFFFu);
  return m;
}

// Encode one unit (8 elements = half a 1x16 block; the other half is in the
// neighbouring lane) and store its 4 data bytes and, on every 8th lane, the
// group of 4 block scales. Executed by all lanes (shuffles), stores predicated.
template <int DT, bool SR>
__device__ __forceinline__ void encode_unit(const Unit<DT> &u, bool valid, uint32_t uidx, uint32_t row,
                                            const RowScaledArgs &p, float S, uint32_t key) {
  float v[8];
  unit_values<DT>(u, v);
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = max(m, __float_as_uint(v[k]) & 0x7FFFFFFFu);
  m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 1, 64)));
  const BlockScale bs = block_scale(__uint_as_float(m), S);
  const uint32_t byte0 = row * (p.cols >> 1) + uidx * 4;
  float s[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) s[k] = v[k] * bs.mult;
  uint32_t word;
  if (SR) {
    uint32_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = fmix32(key ^ (byte0 + q));
    word = e2m1_sr_x8(s, r);
  } else {
    word = e2m1_rne_x8(s);
  }
  if (valid) __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(p.data + byte0));
  const uint32_t c1 = static_cast<uint32_t>(__shfl_down(static_cast<int>(bs.code), 2, 64));
  const uint32_t c2 = static_cast<uint32_t>(__shfl_down(static_cast<int>(bs.code), 4, 64));
  const uint32_t c3 = static_cast<uint32_t>(__shfl_down(static_cast<int>(bs.code), 6, 64));
  if (valid && (uidx & 7u) == 0) {
    const uint32_t scale_cols = p.cols >> 4;
    const uint32_t sc = uidx >> 1;
    const uint64_t off = static_cast<uint64_t>(row) * scale_cols + sc;
    const uint32_t group = bs.code | (c1 << 8) | (c2 << 16) | (c3 << 24);
    if ((scale_cols & 3u) == 0 && sc + 4 <= scale_cols) {
      __builtin_nontemporal_store(group, reinterpret_cast<uint32_t *>(p.scales + off));
    } else {
#pragma unroll
      for (uint32_t i = 0; i < 4; ++i)
        if (sc + i < scale_cols) p.scales[off + i] = static_cast<uint8_t>(group >> (8 * i));
    }
  }
}

template <int DT, bool SR, bool COMPUTE>
__global__ __launch_bounds__(kThreads) void k_rowscaled(RowScaledArgs p) {
  __shared__ uint32_t lds_w[kThreads / 64];
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  const uint32_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const uint32_t units = p.cols >> 3;
  const uint64_t row_off = static_cast<uint64_t>(row) * p.cols;

  Unit<DT> reg[kRegUnits];
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < kRegUnits; ++k) {
    const uint32_t u = tid + kThreads * k;
    if (u < units) {
      reg[k] = load_unit<DT, true>(p.x, row_off + 8ull * u);
      if (COMPUTE) m = max(m, unit_max_bits<DT>(reg[k]));
    } else {
#pragma unroll
      for (int q = 0; q < Unit<DT>::kWords; ++q) reg[k].w[q] = 0;
    }
  }
  float amax;
  if (COMPUTE) {
    for (uint32_t u = tid + kThreads * kRegUnits; u < units; u += kThreads)
      m = max(m, unit_max_bits<DT>(load_unit<DT, false>(p.x, row_off + 8ull * u)));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off, 64)));
    if ((tid & 63) == 0) lds_w[tid >> 6] = m;
    __syncthreads();
    m = lds_w[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) m = max(m, lds_w[w]);
    amax = __uint_as_float(m);
    if (tid == 0) p.amax[row] = amax;
  } else {
    amax = p.amax[row];
  }
  if (p.data == nullptr) return;

  const float S = global_encode_scale(amax);
  const uint32_t key = SR ? sr_key(p.sr_seed, 0) : 0u;
#pragma unroll
  for (int k = 0; k < kRegUnits; ++k) {
    const uint32_t u = tid + kThreads * k;
    encode_unit<DT, SR>(reg[k], u < units, u, row, p, S, key);
  }
  for (uint32_t base = kThreads * kRegUnits; base < units; base += kThreads) {
    const uint32_t u = base + tid;
    Unit<DT> cur;
    if (u < units) {
      cur = load_unit<DT, false>(p.x, row_off + 8ull * u);
    } else {
#pragma unroll
      for (int q = 0; q < Unit<DT>::kWords; ++q) cur.w[q] = 0;
    }
    encode_unit<DT, SR>(cur, u < units, u, row, p, S, key);
  }
}

template <int DT, bool SR, bool COMPUTE>
hipError_t launch_one(const RowScaledArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((k_rowscaled<DT, SR, COMPUTE>), dim3(a.rows), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const RowScaledArgs &a, bool sr, bool compute, hipStream_t s) {
  if (compute) return sr ? launch_one<DT, true, true>(a, s) : launch_one<DT, false, true>(a, s);
  return sr ? launch_one<DT, true, false>(a, s) : launch_one<DT, false, false>(a, s);
}

}  // namespace

hipError_t launch_rowscaled(const RowScaledArgs &a, int dtype, bool sr, bool compute_amax, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  return dtype == kBF16 ? launch_dt<kBF16>(a, sr, compute_amax, s) : launch_dt<kFP32>(a, sr, compute_amax, s);
}

}  // namespace nvfp4
