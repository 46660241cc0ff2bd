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
#include <atomic>

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

// ---------------------------------------------------------------------------
// Column-wise side of a row-scaled quantize. The column-wise tensor's rows
// are the input's columns, so it is scaled along them: one amax per input
// column, and each column's 1x16 blocks (16 consecutive rows) take their
// E4M3 scales relative to that column's global scale (the quantizer
// prototype in the review thread of "Write both NVFP4 amax buffers" sizes
// the column-wise amax of a row-scaled tensor as one float per input
// column). Two launches: a column reduction (HBM-bound, one read of
// the input) and the encode (one more read, the transpose written out).
// ---------------------------------------------------------------------------
constexpr uint32_t kColAmaxCols = 512;  // 64 lanes x 8 columns: one wave reads 1 KiB (BF16) of a row
constexpr uint32_t kColAmaxRows = 128;  // rows per workgroup of the reduction
constexpr uint32_t kColStrip = 64;      // columns per encode workgroup (8 lanes x 8 columns)
constexpr uint32_t kColRows = 512;      // rows per encode unit (32 lane groups x 16 rows)
#ifndef NVFP4_COL_WGS_PER_CU
#define NVFP4_COL_WGS_PER_CU 2
#endif
constexpr int kColWgsPerCu = NVFP4_COL_WGS_PER_CU;  // encode workgroups kept per compute unit

template <int DT>
struct Piece8 {  // 8 consecutive elements of one row
  static constexpr int kWords = DT == kBF16 ? 4 : 8;
  uint32_t w[kWords];
};

template <int DT>
__device__ __forceinline__ Piece8<DT> load_piece8(const void *x, uint64_t elem_off) {
  Piece8<DT> b;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(x) + elem_off * (DT == kBF16 ? 2 : 4));
#pragma unroll
  for (int q = 0; q < Piece8<DT>::kWords / 4; ++q) {
    const u32x4 t = __builtin_nontemporal_load(src + q);
    b.w[4 * q] = t.x;
    b.w[4 * q + 1] = t.y;
    b.w[4 * q + 2] = t.z;
    b.w[4 * q + 3] = t.w;
  }
  return b;
}

// Running max |x| of 8 columns, read back per column as the bit pattern of
// a non-negative float. BF16 keeps both columns of a word in one packed
// 16-bit max (one AND and one max per word).
template <int DT>
struct ColMax {
  uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  __device__ __forceinline__ void fold(const Piece8<DT> &b) {
#pragma unroll
    for (int c = 0; c < 8; ++c) m[c] = max(m[c], b.w[c] & 0x7FFFFFFFu);
  }
  __device__ __forceinline__ uint32_t get(int c) const { return m[c]; }
};

template <>
struct ColMax<kBF16> {
  ushort2_t h[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
  __device__ __forceinline__ void fold(const Piece8<kBF16> &b) {
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = __builtin_elementwise_max(h[q], __builtin_bit_cast(ushort2_t, b.w[q] & 0x7FFF7FFFu));
  }
  // element 2q is the word's low half, 2q + 1 its high half
  __device__ __forceinline__ uint32_t get(int c) const {
    return static_cast<uint32_t>((c & 1) ? h[c >> 1].y : h[c >> 1].x) << 16;
  }
};

template <int DT>
__device__ __forceinline__ float piece8_value(const Piece8<DT> &b, int c) {
  if (DT == kBF16) return (c & 1) ? bf16_hi(b.w[c >> 1]) : bf16_lo(b.w[c >> 1]);
  return __uint_as_float(b.w[c]);
}

__global__ __launch_bounds__(kThreads) void k_colamax_zero(float *amax, uint32_t n, const float *noop) {
  if (noop != nullptr && *noop == 1.0f) return;
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) amax[i] = 0.0f;
}

// amax[j] = max over rows of |x[i][j]|, after k_colamax_zero: each
// workgroup reduces kColAmaxRows rows of kColAmaxCols columns (wave v takes
// rows v, v + 4, ...) and folds its maxima in with one atomic max per
// column (non-negative floats order as their bit patterns).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_colamax(RowScaledArgs p) {
  __shared__ uint32_t lds_m[kWaves][kColAmaxCols];
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // one-dimensional grid (either extent alone may pass 65535): column strip
  // fastest, so consecutive workgroups read neighbouring parts of a row
  const uint32_t nstrip = (p.cols + kColAmaxCols - 1) / kColAmaxCols;
  const uint32_t chunk = blockIdx.x / nstrip, strip = blockIdx.x - chunk * nstrip;
  const uint32_t c0 = strip * kColAmaxCols + 8 * lane;
  const uint32_t rbeg = chunk * kColAmaxRows;
  const uint32_t rend = min(rbeg + kColAmaxRows, p.rows);
  ColMax<DT> acc;
  if (c0 < p.cols) {  // cols % 16 == 0: a lane's 8 columns are all inside or all outside
    constexpr int kUnroll = 16;
    uint32_t r = rbeg + wave;
    for (; r + kWaves * (kUnroll - 1) < rend; r += kWaves * kUnroll) {
      Piece8<DT> b[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) b[u] = load_piece8<DT>(p.x, static_cast<uint64_t>(r + kWaves * u) * p.cols + c0);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc.fold(b[u]);
    }
    for (; r < rend; r += kWaves) acc.fold(load_piece8<DT>(p.x, static_cast<uint64_t>(r) * p.cols + c0));
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) lds_m[wave][8 * lane + c] = acc.get(c);
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t k = tid + kThreads * h;
    const uint32_t j = strip * kColAmaxCols + k;
    uint32_t v = lds_m[0][k];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v = max(v, lds_m[w][k]);
    if (j < p.cols && v != 0) atomicMax(reinterpret_cast<unsigned int *>(p.amax) + j, v);
  }
}

// Column-wise encode with the per-column amax. A unit is 512 rows x 64
// columns: thread (lane group g = tid / 8, column piece tid % 8) owns 8
// columns x 16 rows of it, one 1x16 block of each of its 8 columns, and
// writes each block's 8 data bytes and scale to the transposed arrays
// ([cols][rows / 2], [cols][rows / 16]). The grid is what stays resident and
// each workgroup walks units with the next unit's loads issued before the
// current unit is encoded, so the encode overlaps the reads; a grid of one
// unit per workgroup would load everything first and encode afterwards.
template <int DT>
__device__ __forceinline__ void load_unit(const RowScaledArgs &p, uint32_t unit, uint32_t nstrip, Piece8<DT> (&b)[16],
                                          uint32_t &c0, uint32_t &r0, bool &ok) {
  const uint32_t chunk = unit / nstrip, strip = unit - chunk * nstrip;
  c0 = strip * kColStrip + 8 * (threadIdx.x & 7);
  r0 = chunk * kColRows + 16 * (threadIdx.x >> 3);
  ok = c0 < p.cols && r0 < p.rows;  // rows % 16 == 0, cols % 16 == 0: whole blocks
  // a lane outside the input loads (and later discards) the first 16 rows,
  // which exist: rows >= 16
  const uint64_t base = ok ? static_cast<uint64_t>(r0) * p.cols + c0 : 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) b[k] = load_piece8<DT>(p.x, base + static_cast<uint64_t>(k) * p.cols);
}

template <int DT, bool SR>
__device__ __forceinline__ void encode_unit(const RowScaledArgs &p, const Piece8<DT> (&b)[16], uint32_t c0,
                                            uint32_t r0, bool ok) {
  if (!ok) return;
  const bool ue = p.ue5m3 != 0;
  const uint32_t key = SR ? sr_key(p.sr_seed, 1) : 0u;
  const uint64_t half_rows = p.rows >> 1;
  ColMax<DT> acc;
#pragma unroll
  for (int k = 0; k < 16; ++k) acc.fold(b[k]);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t j = c0 + c;
    const float S = global_encode_scale(p.amax[j], ue);
    const BlockScale bs = block_scale(__uint_as_float(acc.get(c)), S, ue);
    float s[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) s[k] = piece8_value<DT>(b[k], c) * bs.mult;
    const uint64_t byte0 = j * half_rows + (r0 >> 1);
    uint32_t lo, hi;
    if (SR) {
      uint32_t r[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) r[q] = fmix32(key ^ static_cast<uint32_t>(byte0 + q));
      lo = e2m1_sr_x8(s, r);
      hi = e2m1_sr_x8(s + 8, r + 4);
    } else {
      lo = e2m1_rne_x8(s);
      hi = e2m1_rne_x8(s + 8);
    }
    // plain stores: a wave writes 64-byte halves of output lines, which the
    // L2 merges (non-temporal stores of them measured 7% slower)
    *reinterpret_cast<u32x2 *>(p.data + byte0) = u32x2{lo, hi};
    p.scales[static_cast<uint64_t>(j) * (p.rows >> 4) + (r0 >> 4)] = static_cast<uint8_t>(bs.code);
  }
}

template <int DT, bool SR>
__global__ __launch_bounds__(kThreads) void k_colscaled(RowScaledArgs p, uint32_t units) {
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  const uint32_t nstrip = (p.cols + kColStrip - 1) / kColStrip;  // strip fastest: neighbouring row parts
  uint32_t u = blockIdx.x;  // < units (the grid is at most one workgroup per unit)
  Piece8<DT> cur[16];
  uint32_t c0, r0;
  bool ok;
  load_unit<DT>(p, u, nstrip, cur, c0, r0, ok);
  for (;;) {  // no barrier inside: lanes may leave at different units only through `ok`
    const uint32_t next = u + gridDim.x;
    if (next >= units) break;  // uniform
    Piece8<DT> nxt[16];
    uint32_t nc0, nr0;
    bool nok;
    load_unit<DT>(p, next, nstrip, nxt, nc0, nr0, nok);
    encode_unit<DT, SR>(p, cur, c0, r0, ok);
#pragma unroll
    for (int k = 0; k < 16; ++k) cur[k] = nxt[k];
    c0 = nc0;
    r0 = nr0;
    ok = nok;
    u = next;
  }
  encode_unit<DT, SR>(p, cur, c0, r0, ok);
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

hipError_t launch_colscaled(const RowScaledArgs &a, int dtype, bool sr, bool compute_amax, hipStream_t s) {
  if (a.cols == 0) return hipSuccess;
  if (compute_amax) {
    hipLaunchKernelGGL(k_colamax_zero, dim3((a.cols + kThreads - 1) / kThreads), dim3(kThreads), 0, s, a.amax, a.cols,
                       a.noop);
    if (a.rows > 0) {
      const dim3 grid(((a.cols + kColAmaxCols - 1) / kColAmaxCols) * ((a.rows + kColAmaxRows - 1) / kColAmaxRows));
      if (dtype == kBF16)
        hipLaunchKernelGGL(k_colamax<kBF16>, grid, dim3(kThreads), 0, s, a);
      else
        hipLaunchKernelGGL(k_colamax<kFP32>, grid, dim3(kThreads), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.data == nullptr || a.rows == 0) return hipSuccess;
  const uint32_t units = ((a.cols + kColStrip - 1) / kColStrip) * ((a.rows + kColRows - 1) / kColRows);
  const void *fn = dtype == kBF16 ? (sr ? reinterpret_cast<const void *>(&k_colscaled<kBF16, true>)
                                        : reinterpret_cast<const void *>(&k_colscaled<kBF16, false>))
                                  : (sr ? reinterpret_cast<const void *>(&k_colscaled<kFP32, true>)
                                        : reinterpret_cast<const void *>(&k_colscaled<kFP32, false>));
  // resident workgroups: compute units x what one holds (the latter depends
  // on the kernel's registers only, so it is taken once per kernel)
  static std::atomic<int> occupancy[2][2];
  hipDevice_t dev = 0;
  int cus = 0;
  hipError_t e = hipStreamGetDevice(s, &dev);  // the device the work runs on
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int per_cu = occupancy[dtype == kBF16][sr].load(std::memory_order_relaxed);
  if (per_cu == 0) {
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0)) != hipSuccess) return e;
    occupancy[dtype == kBF16][sr].store(per_cu, std::memory_order_relaxed);
  }
  const uint32_t resident = static_cast<uint32_t>(max(cus, 1)) * static_cast<uint32_t>(min(max(per_cu, 1), kColWgsPerCu));
  const dim3 grid(min(units, resident));
  if (dtype == kBF16) {
    if (sr)
      hipLaunchKernelGGL((k_colscaled<kBF16, true>), grid, dim3(kThreads), 0, s, a, units);
    else
      hipLaunchKernelGGL((k_colscaled<kBF16, false>), grid, dim3(kThreads), 0, s, a, units);
  } else {
    if (sr)
      hipLaunchKernelGGL((k_colscaled<kFP32, true>), grid, dim3(kThreads), 0, s, a, units);
    else
      hipLaunchKernelGGL((k_colscaled<kFP32, false>), grid, dim3(kThreads), 0, s, a, units);
  }
  return hipGetLastError();
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
