// Row-scaled (per-token) NVFP4 quantize for gfx950: one workgroup per row.
//
// "Implement row-scaled NVFP4 fprop recipe" (Changes, Greptile summary): each
// row gets its own FP32 amax and the E4M3 block scales are taken relative to
// it; output is row-wise only with compact scales. There the row amax is a
// separate kernel run before the quantize kernel. Here the two are one
// kernel: each thread keeps two whole 1x16 blocks of a row in registers (up
// to 8192 elements per row) between the reduction and the cast, so the input
// is read from HBM once; longer rows re-read the part beyond that from cache.
//
// With whole blocks per thread, a block's maximum needs no other lane; the
// four scale codes of an aligned group are gathered by lane exchanges
// (DPP or swizzles, see reg_block), and the row maximum is a DPP wave
// reduction plus one barrier.
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

// One block of the part of a row beyond the register part (rows longer than
// 8192 elements): read twice, for the reduction and for the encode, so
// through the caches.
template <int DT>
__device__ __forceinline__ Block<DT> load_block(const void *x, uint64_t elem_off) {
  Block<DT> b;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(x) + elem_off * (DT == kBF16 ? 2 : 4));
#pragma unroll
  for (int q = 0; q < Block<DT>::kWords / 4; ++q) {
    const u32x4 t = src[q];
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

// The four scale codes of an aligned group of blocks, for the lane that
// holds its first block: the group's blocks are in lanes t, t + STRIDE,
// t + 2 STRIDE, t + 3 STRIDE (1: a lane quad; 2 and 4: the BF16 and FP32
// register blocks, see reg_block).
template <int STRIDE>
__device__ __forceinline__ uint32_t scale_group(uint32_t code) {
  static_assert(STRIDE == 1 || STRIDE == 2 || STRIDE == 4, "lane strides of the register layouts");
  if (STRIDE == 1)
    return quad_bcast(code, 0) | (quad_bcast(code, 1) << 8) | (quad_bcast(code, 2) << 16) |
           (quad_bcast(code, 3) << 24);
  // bit-mask swizzles within 32 lanes: lane (t with the stride's two bits
  // cleared) | STRIDE i
  constexpr int kAnd = STRIDE == 2 ? 0x19 : 0x13;
  const auto from = [](uint32_t x, auto pattern) {
    return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(x), decltype(pattern)::value));
  };
  return from(code, std::integral_constant<int, kAnd>{}) |
         (from(code, std::integral_constant<int, kAnd | ((1 * STRIDE) << 5)>{}) << 8) |
         (from(code, std::integral_constant<int, kAnd | ((2 * STRIDE) << 5)>{}) << 16) |
         (from(code, std::integral_constant<int, kAnd | ((3 * STRIDE) << 5)>{}) << 24);
}

// Encode block `blk` of `row` (16 elements, block max bits m) and store its 8
// data bytes; the lane holding the first block of an aligned group of four
// stores the group's 4 scale codes. Executed by all lanes (lane exchanges),
// stores predicated on `valid`.
template <int DT, bool SR, int STRIDE = 1>
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
  const uint32_t group = scale_group<STRIDE>(bs.code);
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

// Block index of the thread's register block k. The row is loaded in
// 16-byte pieces, load j taking piece j * 256 + t, so that each load
// instruction of a wave reads 1 KiB contiguous (a layout with whole blocks
// per thread measured about 1 us slower per 4096x8192 BF16 call in a
// traffic-only probe); lanes then exchange pieces so that each holds whole
// blocks. BF16 (2 pieces per block, 4 loads): lanes 2m and 2m + 1 swap
// halves, lane 2m taking the blocks of loads 0 and 2 (blocks m and
// 256 + m), lane 2m + 1 those of loads 1 and 3 (128 + m and 384 + m). FP32
// (4 pieces per block, 8 loads): the lanes 4m + i of a quad transpose each
// group of four loads, lane 4m + i taking the block of load 4k + i, block
// (4k + i) * 64 + m.
template <int DT>
__device__ __forceinline__ uint32_t reg_block(int k) {
  const uint32_t t = threadIdx.x;
  if (DT == kBF16) return kThreads * k + ((t & 1) ? kThreads / 2 + (t >> 1) : (t >> 1));
  return (4 * k + (t & 3)) * (kThreads / 4) + (t >> 2);
}

// Lane stride between consecutive register blocks (scale_group)
template <int DT>
constexpr int kRegStride = DT == kBF16 ? 2 : 4;

// The register part of one row (blocks reg_block(k)), zero past the row's
// end.
template <int DT>
__device__ __forceinline__ void load_row(const RowScaledArgs &p, uint32_t row, Block<DT> (&r)[kRegBlocks]) {
  const uint32_t nblk = p.cols >> 4;
  const uint64_t row_off = static_cast<uint64_t>(row) * p.cols;
  if constexpr (DT == kBF16) {
    static_assert(kRegBlocks == 2, "two pairs of piece loads");
    const uint32_t t = threadIdx.x;
    const uint32_t npieces = p.cols >> 3;  // even: cols % 16 == 0
    const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(p.x) + row_off * 2);
    u32x4 v[2 * kRegBlocks];
#pragma unroll
    for (int j = 0; j < 2 * kRegBlocks; ++j) {
      const uint32_t q = kThreads * j + t;
      v[j] = q < npieces ? __builtin_nontemporal_load(src + q) : u32x4{0u, 0u, 0u, 0u};
    }
    // a block's two pieces are valid together (block b: pieces 2b, 2b + 1)
    const bool odd = (t & 1) != 0;
#pragma unroll
    for (int k = 0; k < kRegBlocks; ++k) {
      const u32x4 a = v[2 * k], b = v[2 * k + 1];
      // the even lane needs its neighbour's piece of load 2k, the odd lane
      // its neighbour's piece of load 2k + 1
      const uint32_t send[4] = {odd ? a.x : b.x, odd ? a.y : b.y, odd ? a.z : b.z, odd ? a.w : b.w};
      uint32_t got[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) got[c] = dpp_mov<kQuadXor1>(send[c]);
      const uint32_t own_lo[4] = {a.x, a.y, a.z, a.w};
      const uint32_t own_hi[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        r[k].w[c] = odd ? got[c] : own_lo[c];
        r[k].w[4 + c] = odd ? own_hi[c] : got[c];
      }
    }
  } else {
    const uint32_t t = threadIdx.x;
    const uint32_t npieces = p.cols >> 2;  // a multiple of 4: cols % 16 == 0
    const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(p.x) + row_off * 4);
    u32x4 v[4 * kRegBlocks];
#pragma unroll
    for (int j = 0; j < 4 * kRegBlocks; ++j) {
      const uint32_t q = kThreads * j + t;
      v[j] = q < npieces ? __builtin_nontemporal_load(src + q) : u32x4{0u, 0u, 0u, 0u};
    }
    // per group of four loads and per dword, a 4x4 transpose over the lane
    // quad in two exchange stages (lane ^ 1, then lane ^ 2): afterwards lane
    // i of the quad holds, as its piece j, what lane j loaded in load 4k + i
    const uint32_t i = t & 3;
#pragma unroll
    for (int k = 0; k < kRegBlocks; ++k) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t m[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] = v[4 * k + j][d];
        uint32_t n[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t other = dpp_mov<kQuadXor1>(m[j ^ 1]);
          n[j] = ((static_cast<uint32_t>(j) ^ i) & 1u) ? other : m[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t other = dpp_mov<kQuadXor2>(n[j ^ 2]);
          r[k].w[4 * j + d] = ((static_cast<uint32_t>(j) ^ i) & 2u) ? other : n[j];
        }
      }
    }
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
      m = max(m, block_max_bits<DT>(load_block<DT>(p.x, row_off + 16ull * blk)));
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
    const uint32_t blk = reg_block<DT>(k);
    encode_block<DT, SR, kRegStride<DT>>(reg[k], bm[k], blk < nblk, blk, row, p, S, key, sr_base);
  }
  for (uint32_t base = kThreads * kRegBlocks; base < nblk; base += kThreads) {  // uniform loop
    const uint32_t blk = base + tid;
    Block<DT> cur;
    if (blk < nblk)
      cur = load_block<DT>(p.x, row_off + 16ull * blk);
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
// Per-row and per-column amax of a row-scaled quantize with both
// orientations. The column-wise tensor's rows are the input's columns, so it
// is scaled along them: one amax per input column, and each column's 1x16
// blocks (16 consecutive rows) take their scales relative to that column's
// global scale (the quantizer prototype in the review thread of "Write both
// NVFP4 amax buffers" sizes the column-wise amax of a row-scaled tensor as
// one float per input column). Both orientations then take one read each:
// this reduction of both amax arrays, and the register-tile encode of both
// orientations with per-row and per-column global scales (cast.hip).
// ---------------------------------------------------------------------------
constexpr uint32_t kColAmaxCols = 512;  // 64 lanes x 8 columns: one wave reads 1 KiB (BF16) of a row
constexpr uint32_t kColAmaxRows = 64;   // rows per workgroup of the reduction: one batch per wave

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
    const u32x4 t = src[q];
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

// max |x| of a piece as the bit pattern of a non-negative float
template <int DT>
__device__ __forceinline__ uint32_t piece8_max(const Piece8<DT> &b) {
  if (DT == kBF16) {
    ushort2_t h = {0, 0};
#pragma unroll
    for (int q = 0; q < 4; ++q) h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2_t, b.w[q] & 0x7FFF7FFFu));
    return static_cast<uint32_t>(max(h.x, h.y)) << 16;
  }
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < Piece8<DT>::kWords; ++q) m = max(m, b.w[q] & 0x7FFFFFFFu);
  return m;
}

__global__ __launch_bounds__(kThreads) void k_amax_zero2(float *a, uint32_t na, float *b, uint32_t nb,
                                                       const float *noop) {
  if (noop != nullptr && *noop == 1.0f) return;
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (a != nullptr && i < na) a[i] = 0.0f;
  if (b != nullptr && i < nb) b[i] = 0.0f;
}

// One batch of the reduction: rows r, r + 4, ..., r + 4 (N - 1) of the
// lane's 8 columns (KEEP: a lane outside the input reads column 0 and
// discards it). The column maxima fold into acc; with row_amax, each row's
// maximum over the wave's 512 columns goes to the row's slot by atomic max:
// the lanes' row maxima are transposed through LDS (lds_r, the wave's
// [64][17] words), lane l reduces row l % 16 over lanes 16 (l / 16) ..
// 16 (l / 16) + 15, two lane exchanges combine the four quarters, and lanes
// 0 .. N - 1 issue the atomics in one instruction.
template <int DT, int N, bool KEEP>
__device__ __forceinline__ void dual_amax_rows(const RowScaledArgs &p, float *row_amax, uint32_t r, uint32_t c0,
                                               bool lane_ok, ColMax<DT> &acc, uint32_t *lds_r) {
  Piece8<DT> b[N];
#pragma unroll
  for (int u = 0; u < N; ++u) b[u] = load_piece8<DT>(p.x, static_cast<uint64_t>(r + kWaves * u) * p.cols + c0);
  if (KEEP) {
    const uint32_t keep = lane_ok ? ~0u : 0u;
#pragma unroll
    for (int u = 0; u < N; ++u)
#pragma unroll
      for (int q = 0; q < Piece8<DT>::kWords; ++q) b[u].w[q] &= keep;
  }
#pragma unroll
  for (int u = 0; u < N; ++u) acc.fold(b[u]);
  if (row_amax != nullptr) {  // uniform
    static_assert(N <= 16, "one row per lane of a quarter wave");
    const uint32_t lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < N; ++u) lds_r[lane * 17 + u] = piece8_max<DT>(b[u]);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
    const uint32_t u = lane & 15, q = lane >> 4;
    uint32_t m = 0;
    if (u < N) {
#pragma unroll
      for (int k = 0; k < 16; ++k) m = max(m, lds_r[(16 * q + k) * 17 + u]);
    }
    m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 16)));
    m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 32)));
    if (lane < N && m != 0) atomicMax(reinterpret_cast<unsigned int *>(row_amax) + r + kWaves * lane, m);
    __builtin_amdgcn_wave_barrier();  // the reads above are done before a later batch writes lds_r
  }
}

// Per-column maxima (p.amax, when not NULL) and per-row maxima (row_amax,
// when not NULL) in one read of the input, after k_amax_zero2: each
// workgroup reduces kColAmaxRows rows of kColAmaxCols columns (wave v takes
// rows v, v + 4, ...) and folds its maxima in with one atomic max per
// column and per row (non-negative floats order as their bit patterns).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_dual_amax(RowScaledArgs p, float *row_amax) {
  __shared__ uint32_t lds_m[kWaves][kColAmaxCols];
  __shared__ uint32_t lds_r[kWaves][64 * 17];
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // one-dimensional grid (either extent alone may pass 65535): column strip
  // fastest, so consecutive workgroups read neighbouring parts of a row
  const uint32_t nstrip = (p.cols + kColAmaxCols - 1) / kColAmaxCols;
  const uint32_t chunk = blockIdx.x / nstrip, strip = blockIdx.x - chunk * nstrip;
  const bool full = (strip + 1) * kColAmaxCols <= p.cols;  // uniform
  // cols % 16 == 0: a lane's 8 columns are all inside or all outside
  const bool lane_ok = strip * kColAmaxCols + 8 * lane < p.cols;
  const uint32_t c0 = lane_ok ? strip * kColAmaxCols + 8 * lane : 0u;
  const uint32_t rbeg = chunk * kColAmaxRows;
  const uint32_t rend = min(rbeg + kColAmaxRows, p.rows);
  ColMax<DT> acc;
  constexpr int kUnroll = DT == kBF16 ? 16 : 8;  // 256 bytes of loads in flight per lane
  uint32_t r = rbeg + wave;
  for (; r + kWaves * (kUnroll - 1) < rend; r += kWaves * kUnroll) {
    if (full) dual_amax_rows<DT, kUnroll, false>(p, row_amax, r, c0, lane_ok, acc, lds_r[wave]);
    else dual_amax_rows<DT, kUnroll, true>(p, row_amax, r, c0, lane_ok, acc, lds_r[wave]);
  }
  for (; r < rend; r += kWaves) dual_amax_rows<DT, 1, true>(p, row_amax, r, c0, lane_ok, acc, lds_r[wave]);
  if (p.amax == nullptr) return;  // uniform
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

hipError_t launch_dual_amax(const void *x, int dtype, uint32_t rows, uint32_t cols, float *row_amax, float *col_amax,
                            const float *noop, hipStream_t s) {
  if (row_amax == nullptr && col_amax == nullptr) return hipSuccess;
  const uint32_t n = max(row_amax ? rows : 0u, col_amax ? cols : 0u);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_amax_zero2, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s, row_amax, rows, col_amax,
                     cols, noop);
  if (rows > 0 && cols > 0) {
    RowScaledArgs a{x, rows, cols, nullptr, nullptr, col_amax, 0u, noop};
    const dim3 grid(((cols + kColAmaxCols - 1) / kColAmaxCols) * ((rows + kColAmaxRows - 1) / kColAmaxRows));
    if (dtype == kBF16)
      hipLaunchKernelGGL(k_dual_amax<kBF16>, grid, dim3(kThreads), 0, s, a, row_amax);
    else
      hipLaunchKernelGGL(k_dual_amax<kFP32>, grid, dim3(kThreads), 0, s, a, row_amax);
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
