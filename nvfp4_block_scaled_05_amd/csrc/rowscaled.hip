// Row-scaled (per-token) NVFP4 quantize for gfx950: one workgroup per row.
//
// "Implement row-scaled NVFP4 fprop recipe" (Changes, Greptile summary): each
// row gets its own FP32 amax and the E4M3 block scales are taken relative to
// it; output is row-wise only with compact scales. There the row amax is a
// separate kernel run before the quantize kernel. Here the two are one
// kernel: thread t keeps 1x16 blocks t and t + 256 of a row in registers (up
// to 8192 elements per row) between the reduction and the cast, so the input
// is read from HBM once; longer rows re-read the part beyond that from cache.
//
// With whole blocks per thread, a block's maximum needs no other lane; the
// four scale codes of an aligned group (four consecutive threads) are
// gathered with DPP, and the row maximum is a DPP wave reduction plus one
// barrier.
#include "codec.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRegBlocks = 2;  // 1x16 blocks per thread kept in registers

template <int DT>
struct Block {
  static constexpr int kWords = DT == kBF16 ? 8 : 16;
  uint32_t w[kWords];
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

// NT: non-temporal (the part of a row that stays in registers is read once);
// the part beyond that is read twice and goes through the caches.
template <int DT, bool NT>
__device__ __forceinline__ Block<DT> load_block(const void *x, uint64_t elem_off) {
  Block<DT> b;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(x) + elem_off * (DT == kBF16 ? 2 : 4));
#pragma unroll
  for (int q = 0; q < Block<DT>::kWords / 4; ++q) {
    const u32x4 t = NT ? __builtin_nontemporal_load(src + q) : src[q];
    b.w[4 * q] = t.x;
    b.w[4 * q + 1] = t.y;
    b.w[4 * q + 2] = t.z;
    b.w[4 * q + 3] = t.w;
  }
  return b;
}

template <int DT>
__device__ __forceinline__ void zero_block(Block<DT> &b) {
#pragma unroll
  for (int q = 0; q < Block<DT>::kWords; ++q) b.w[q] = 0;
}

// max |x| of a block as the bit pattern of a non-negative float
template <int DT>
__device__ __forceinline__ uint32_t block_max_bits(const Block<DT> &b) {
  if (DT == kBF16) {
    ushort2_t h = {0, 0};
#pragma unroll
    for (int q = 0; q < 8; ++q) h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2_t, b.w[q] & 0x7FFF7FFFu));
    return static_cast<uint32_t>(max(h.x, h.y)) << 16;
  }
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) m = max(m, b.w[q] & 0x7FFFFFFFu);
  return m;
}

template <int DT>
__device__ __forceinline__ float block_value(const Block<DT> &b, int k) {
  if (DT == kBF16) return (k & 1) ? bf16_hi(b.w[k >> 1]) : bf16_lo(b.w[k >> 1]);
  return __uint_as_float(b.w[k]);
}

// Encode block `blk` of `row` (16 elements, block max bits m) and store its 8
// data bytes; lane 0 of each group of four stores the group's 4 scale codes.
// Executed by all lanes (DPP), stores predicated on `valid`.
template <int DT, bool SR>
__device__ __forceinline__ void encode_block(const Block<DT> &b, uint32_t m, bool valid, uint32_t blk, uint32_t row,
                                             const RowScaledArgs &p, float S, uint32_t key, uint64_t sr_base) {
  const BlockScale bs = block_scale(__uint_as_float(m), S, p.ue5m3 != 0);
  float s[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) s[k] = block_value<DT>(b, k) * bs.mult;
  const uint64_t byte0 = static_cast<uint64_t>(row) * (p.cols >> 1) + 8ull * blk;
  uint32_t lo, hi;
  if (SR) {
    uint32_t r[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) r[q] = fmix32(key ^ static_cast<uint32_t>(byte0 - sr_base + q));
    lo = e2m1_sr_x8(s, r);
    hi = e2m1_sr_x8(s + 8, r + 4);
  } else {
    lo = e2m1_rne_x8(s);
    hi = e2m1_rne_x8(s + 8);
  }
  if (valid) __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2 *>(p.data + byte0));
  const uint32_t group = quad_bcast(bs.code, 0) | (quad_bcast(bs.code, 1) << 8) | (quad_bcast(bs.code, 2) << 16) |
                         (quad_bcast(bs.code, 3) << 24);
  if (valid && (blk & 3u) == 0) {
    const uint32_t scale_cols = p.cols >> 4;
    const uint64_t off = static_cast<uint64_t>(row) * scale_cols + blk;
    if ((scale_cols & 3u) == 0 && blk + 4 <= scale_cols) {
      __builtin_nontemporal_store(group, reinterpret_cast<uint32_t *>(p.scales + off));
    } else {
#pragma unroll
      for (uint32_t i = 0; i < 4; ++i)
        if (blk + i < scale_cols) p.scales[off + i] = static_cast<uint8_t>(group >> (8 * i));
    }
  }
}

// The register part of one row (blocks t, t + kThreads, ...), zero past the
// row's end.
template <int DT>
__device__ __forceinline__ void load_row(const RowScaledArgs &p, uint32_t row, Block<DT> (&r)[kRegBlocks]) {
  const uint32_t nblk = p.cols >> 4;
  const uint64_t row_off = static_cast<uint64_t>(row) * p.cols;
#pragma unroll
  for (int k = 0; k < kRegBlocks; ++k) {
    const uint32_t blk = threadIdx.x + kThreads * k;
    if (blk < nblk)
      r[k] = load_block<DT, true>(p.x, row_off + 16ull * blk);
    else
      zero_block<DT>(r[k]);
  }
}

// One row: amax (or the given one), then encode and store.
template <int DT, bool SR, bool COMPUTE>
__device__ __forceinline__ void process_row(const RowScaledArgs &p, uint32_t row, const Block<DT> (&reg)[kRegBlocks],
                                            uint32_t *lds_w, uint32_t key, uint64_t sr_base) {
  const int tid = threadIdx.x;
  const uint32_t nblk = p.cols >> 4;
  const uint64_t row_off = static_cast<uint64_t>(row) * p.cols;
  uint32_t bm[kRegBlocks];
#pragma unroll
  for (int k = 0; k < kRegBlocks; ++k) bm[k] = block_max_bits<DT>(reg[k]);
  float amax;
  if (COMPUTE) {
    uint32_t m = bm[0];
#pragma unroll
    for (int k = 1; k < kRegBlocks; ++k) m = max(m, bm[k]);
    for (uint32_t blk = tid + kThreads * kRegBlocks; blk < nblk; blk += kThreads)
      m = max(m, block_max_bits<DT>(load_block<DT, false>(p.x, row_off + 16ull * blk)));
    m = wave_max(m);
    if ((tid & 63) == 0) lds_w[tid >> 6] = m;
    __syncthreads();
    m = lds_w[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = max(m, lds_w[w]);
    amax = __uint_as_float(m);
    if (tid == 0) p.amax[row] = amax;
  } else {
    amax = p.amax[row];
  }
  if (p.data == nullptr) return;

  const float S = global_encode_scale(amax, p.ue5m3 != 0);
#pragma unroll
  for (int k = 0; k < kRegBlocks; ++k) {
    const uint32_t blk = tid + kThreads * k;
    encode_block<DT, SR>(reg[k], bm[k], blk < nblk, blk, row, p, S, key, sr_base);
  }
  for (uint32_t base = kThreads * kRegBlocks; base < nblk; base += kThreads) {  // uniform loop
    const uint32_t blk = base + tid;
    Block<DT> cur;
    if (blk < nblk)
      cur = load_block<DT, false>(p.x, row_off + 16ull * blk);
    else
      zero_block<DT>(cur);
    encode_block<DT, SR>(cur, block_max_bits<DT>(cur), blk < nblk, blk, row, p, S, key, sr_base);
  }
}

// One row per workgroup. A whole grid of these is about two rounds of
// resident workgroups (8 per CU) at the sizes of interest, so the second
// round's loads overlap the first round's encoding and stores; two rows per
// workgroup (one round) measured 8% slower.
template <int DT, bool SR, bool COMPUTE>
__global__ __launch_bounds__(kThreads) void k_rowscaled(RowScaledArgs p) {
  __shared__ uint32_t lds_w[kWaves];
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  const uint32_t key = SR ? sr_key(p.sr_seed, 0) : 0u;
  Block<DT> a[kRegBlocks];
  load_row<DT>(p, blockIdx.x, a);
  process_row<DT, SR, COMPUTE>(p, blockIdx.x, a, lds_w, key, 0);
}

// Grouped form (row slices, each a row-scaled tensor of its own): the same
// rows, with the stochastic-rounding byte indices counted from the start of
// the row's group (t.unit_start holds the groups' first rows). Only
// stochastic rounding needs it; nearest even runs the plain kernel.
template <int DT, bool COMPUTE>
__global__ __launch_bounds__(kThreads) void k_rowscaled_grouped(RowScaledArgs p, GroupTable t) {
  __shared__ uint32_t lds_w[kWaves];
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  const uint32_t key = sr_key(p.sr_seed, 0);
  const uint32_t g = group_of(t, blockIdx.x);
  Block<DT> a[kRegBlocks];
  load_row<DT>(p, blockIdx.x, a);
  process_row<DT, true, COMPUTE>(p, blockIdx.x, a, lds_w, key,
                                 static_cast<uint64_t>(t.unit_start[g]) * (p.cols >> 1));
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

hipError_t launch_rowscaled_grouped(const RowScaledArgs &a, const uint32_t *row_start, uint32_t ngroups, int dtype,
                                    bool sr, bool compute_amax, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (!sr) return launch_rowscaled(a, dtype, false, compute_amax, s);  // grouping changes nothing then
  GroupTable t{};
  t.ngroups = ngroups;
  for (uint32_t g = 0; g <= ngroups; ++g) t.unit_start[g] = t.row_start[g] = row_start[g];
  const dim3 grid(a.rows), block(kThreads);
  if (dtype == kBF16) {
    if (compute_amax)
      hipLaunchKernelGGL((k_rowscaled_grouped<kBF16, true>), grid, block, 0, s, a, t);
    else
      hipLaunchKernelGGL((k_rowscaled_grouped<kBF16, false>), grid, block, 0, s, a, t);
  } else {
    if (compute_amax)
      hipLaunchKernelGGL((k_rowscaled_grouped<kFP32, true>), grid, block, 0, s, a, t);
    else
      hipLaunchKernelGGL((k_rowscaled_grouped<kFP32, false>), grid, block, 0, s, a, t);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
