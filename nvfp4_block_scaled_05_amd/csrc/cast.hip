// Fused NVFP4 cast-transpose for gfx950.
//
// One workgroup (256 threads, 4 waves of 64) owns a tile of TR x 128 input
// elements (TR = 128 for BF16, 64 for FP32) and writes, for that tile:
//   row-wise:    FP4 data [rows][cols/2] and E4M3 scales, 1x16 blocks along
//                each input row (or the shared 16x16 block scale);
//   column-wise: the same for the transposed tensor, 1x16 blocks along each
//                input column, optionally after a 16-point RHT of each
//                16-row column group.
// "Write both NVFP4 amax buffers" (Changes) and "Fuse NVFP4 scale swizzling
// on SM120 and SM121" (Description, Changes) describe one kernel writing
// both orientations, and scales stored directly in the GEMM layout with one
// 32-bit store per aligned group of four.
//
// Data flow per tile:
//   1. each thread loads TR/16 row units of 8 elements with 128-bit loads
//      (a wave reads 4 rows x 256 contiguous bytes per instruction) and, if
//      the column-wise side is wanted, copies them to a padded LDS tile;
//   2. 16x16 mode: block maxima via lane shuffles + LDS, one scale per block;
//   3. row-wise: a 1x16 block is two adjacent lanes' units; the block max is
//      one lane exchange; each lane writes one 32-bit word of 8 codes, and
//      every 8th lane gathers four scales into one 32-bit store;
//   4. column-wise: each thread reads 16 rows x 8 bytes from LDS (2 or 4
//      columns), encodes each column block into 8 bytes (one 64-bit store),
//      and the scales go through LDS so each column's run of scales leaves
//      as 32-bit words.
#include "codec.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kTC = 128;

template <int DT>
struct Tile {
  static constexpr int kElem = DT == kBF16 ? 2 : 4;   // bytes per input element
  static constexpr int kTR = DT == kBF16 ? 128 : 64;  // tile rows
  static constexpr int kUPT = kTR / 16;                // row units per thread
  static constexpr int kUW = 8 * kElem / 4;            // 32-bit words per unit
  static constexpr int kPad = 16 / kElem;              // 16 bytes of padding per LDS row
  static constexpr int kStride = kTC + kPad;           // LDS row stride in elements
  static constexpr int kCPT = 8 / kElem;               // columns per thread in the column phase
  static constexpr int kNCQ = kTC / kCPT;              // column groups per tile
  static constexpr int kNRB = kTR / 16;                // 16-row blocks per tile
  static_assert(kNCQ * kNRB == kThreads, "column phase covers the tile");
};

template <int DT>
__device__ __forceinline__ void unit_values(const uint32_t (&w)[Tile<DT>::kUW], float (&v)[8]) {
  if (DT == kBF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_lo(w[k]);
      v[2 * k + 1] = bf16_hi(w[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __uint_as_float(w[k]);
  }
}

template <int N>
__device__ __forceinline__ uint32_t max_abs_bits(const float (&v)[N]) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < N; ++k) m = max(m, __float_as_uint(v[k]) & 0x7FFFFFFFu);
  return m;
}

// Codes of 8 consecutive values of one output row, packed little-endian
// (element 2i in the low nibble of byte i). byte0 = index of the first byte
// in the orientation's data array (stochastic-rounding counter).
template <bool SR>
__device__ __forceinline__ uint32_t encode8(const float *v, float e, uint32_t key, uint32_t byte0) {
  uint32_t word = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a = v[2 * q] * e;
    const float b = v[2 * q + 1] * e;
    uint32_t lo, hi;
    if (SR) {
      const uint32_t r = fmix32(key ^ (byte0 + q));
      lo = e2m1_sr(a, r & 0xFFFFu);
      hi = e2m1_sr(b, r >> 16);
    } else {
      lo = e2m1_rne(a);
      hi = e2m1_rne(b);
    }
    word |= (lo | (hi << 4)) << (8 * q);
  }
  return word;
}

// Four scales (c .. c+3 of scale row r, c % 4 == 0) packed in `word`.
__device__ __forceinline__ void store_scale_group(uint8_t *base, uint32_t r, uint32_t c, uint32_t scale_cols,
                                                  bool swizzled, uint32_t word) {
  if (swizzled) {
    *reinterpret_cast<uint32_t *>(base + swizzled_scale_offset(r, c, scale_cols)) = word;
    return;
  }
  const uint64_t off = static_cast<uint64_t>(r) * scale_cols + c;
  if ((scale_cols & 3u) == 0 && c + 4 <= scale_cols) {
    *reinterpret_cast<uint32_t *>(base + off) = word;
  } else {
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i)
      if (c + i < scale_cols) base[off + i] = static_cast<uint8_t>(word >> (8 * i));
  }
}

template <int DT, bool B2D, bool RHT, bool SR>
__global__ __launch_bounds__(kThreads) void k_cast(CastArgs p) {
  using T = Tile<DT>;
  __shared__ __align__(16) uint8_t lds_tile[T::kTR * T::kStride * T::kElem];
  __shared__ __align__(4) uint8_t lds_cs[kTC][T::kNRB];  // column-wise scale codes
  __shared__ uint32_t lds_m2d[4][T::kUPT][8];            // 16x16: per-wave partial block max
  __shared__ uint32_t lds_s2d[2][T::kUPT][8];            // 16x16: codes (row, col)
  __shared__ float lds_e2d[2][T::kUPT][8];               // 16x16: multipliers (row, col)

  if (p.noop != nullptr && *p.noop == 1.0f) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ucol = tid & 15;
  const int rsub = tid >> 4;
  const uint32_t r0 = blockIdx.y * T::kTR;
  const uint32_t c0 = blockIdx.x * kTC;
  const uint32_t col = c0 + ucol * 8;
  const bool col_ok = col < p.cols;
  const bool do_row = p.row_data != nullptr;
  const bool do_col = p.col_data != nullptr;

  // 1. load the tile's row units; stage them in LDS for the column phase.
  uint32_t w[T::kUPT][T::kUW];
#pragma unroll
  for (int k = 0; k < T::kUPT; ++k) {
    const uint32_t row = r0 + rsub + 16 * k;
    if (col_ok && row < p.rows) {
      const uint64_t off = static_cast<uint64_t>(row) * p.cols + col;
      const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(p.x) + off * T::kElem);
#pragma unroll
      for (int q = 0; q < T::kUW / 4; ++q) {
        const uint4 t = src[q];
        w[k][4 * q] = t.x;
        w[k][4 * q + 1] = t.y;
        w[k][4 * q + 2] = t.z;
        w[k][4 * q + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < T::kUW; ++q) w[k][q] = 0;
    }
  }
  if (do_col) {
#pragma unroll
    for (int k = 0; k < T::kUPT; ++k) {
      uint4 *dst = reinterpret_cast<uint4 *>(lds_tile + ((rsub + 16 * k) * T::kStride + ucol * 8) * T::kElem);
#pragma unroll
      for (int q = 0; q < T::kUW / 4; ++q)
        dst[q] = make_uint4(w[k][4 * q], w[k][4 * q + 1], w[k][4 * q + 2], w[k][4 * q + 3]);
    }
  }

  const float S_row = do_row ? global_encode_scale(*p.row_amax) : 1.0f;
  const float S_col = do_col ? global_encode_scale(*p.col_amax) : 1.0f;

  // 2. 16x16 blocks: block (k, b) covers tile rows 16k..16k+15 and columns
  //    16b..16b+15, i.e. units held by lanes with ucol in {2b, 2b+1} over all
  //    16 values of rsub (4 rows per wave, 4 waves).
  if (B2D) {
#pragma unroll
    for (int k = 0; k < T::kUPT; ++k) {
      float v[8];
      unit_values<DT>(w[k], v);
      uint32_t m = max_abs_bits(v);
      m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 1, 64)));
      m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 16, 64)));
      m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 32, 64)));
      if (lane < 16 && (lane & 1) == 0) lds_m2d[wave][k][lane >> 1] = m;
    }
    __syncthreads();
    if (tid < T::kUPT * 8) {
      const int k = tid >> 3, b = tid & 7;
      const uint32_t m = max(max(lds_m2d[0][k][b], lds_m2d[1][k][b]), max(lds_m2d[2][k][b], lds_m2d[3][k][b]));
      const BlockScale br = block_scale(__uint_as_float(m), S_row);
      const BlockScale bc = block_scale(__uint_as_float(m), S_col);
      lds_s2d[0][k][b] = br.code;
      lds_e2d[0][k][b] = br.mult;
      lds_s2d[1][k][b] = bc.code;
      lds_e2d[1][k][b] = bc.mult;
    }
    __syncthreads();
  }

  // 3. row-wise orientation.
  if (do_row) {
    const uint32_t key = SR ? sr_key(p.sr_seed, 0) : 0u;
    const uint32_t half_cols = p.cols >> 1;
    const uint32_t scale_cols = p.cols >> 4;
#pragma unroll
    for (int k = 0; k < T::kUPT; ++k) {
      const uint32_t row = r0 + rsub + 16 * k;
      float v[8];
      unit_values<DT>(w[k], v);
      uint32_t code;
      float mult;
      if (B2D) {
        code = lds_s2d[0][k][ucol >> 1];
        mult = lds_e2d[0][k][ucol >> 1];
      } else {
        uint32_t m = max_abs_bits(v);
        m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), 1, 64)));
        const BlockScale bs = block_scale(__uint_as_float(m), S_row);
        code = bs.code;
        mult = bs.mult;
      }
      const bool valid = col_ok && row < p.rows;
      const uint32_t byte0 = row * half_cols + (col >> 1);
      const uint32_t word = encode8<SR>(v, mult, key, byte0);
      if (valid) *reinterpret_cast<uint32_t *>(p.row_data + byte0) = word;
      const uint32_t c1 = static_cast<uint32_t>(__shfl_down(static_cast<int>(code), 2, 64));
      const uint32_t c2 = static_cast<uint32_t>(__shfl_down(static_cast<int>(code), 4, 64));
      const uint32_t c3 = static_cast<uint32_t>(__shfl_down(static_cast<int>(code), 6, 64));
      if (valid && (ucol & 7) == 0)
        store_scale_group(p.row_scales, row, col >> 4, scale_cols, p.swizzled != 0,
                          code | (c1 << 8) | (c2 << 16) | (c3 << 24));
    }
  }

  // 4. column-wise orientation.
  if (do_col) {
    __syncthreads();
    const uint32_t key = SR ? sr_key(p.sr_seed, 1) : 0u;
    const int cq = tid % T::kNCQ;
    const int rb = tid / T::kNCQ;
    const int lc0 = cq * T::kCPT;
    const uint32_t rr = r0 + rb * 16;
    const bool rb_ok = rr < p.rows;
    const uint32_t half_rows = p.rows >> 1;
    uint2 raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      raw[i] = *reinterpret_cast<const uint2 *>(lds_tile + ((rb * 16 + i) * T::kStride + lc0) * T::kElem);
#pragma unroll
    for (int c = 0; c < T::kCPT; ++c) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (DT == kBF16) {
          const uint32_t wd = (c < 2) ? raw[i].x : raw[i].y;
          v[i] = (c & 1) ? bf16_hi(wd) : bf16_lo(wd);
        } else {
          v[i] = __uint_as_float(c == 0 ? raw[i].x : raw[i].y);
        }
      }
      if (RHT) rht16(v, p.sign_mask);
      uint32_t code;
      float mult;
      if (B2D) {
        code = lds_s2d[1][rb][(lc0 + c) >> 4];
        mult = lds_e2d[1][rb][(lc0 + c) >> 4];
      } else {
        const BlockScale bs = block_scale(__uint_as_float(max_abs_bits(v)), S_col);
        code = bs.code;
        mult = bs.mult;
      }
      const uint32_t j = c0 + lc0 + c;
      const uint32_t byte0 = j * half_rows + (rr >> 1);
      uint2 out;
      out.x = encode8<SR>(v, mult, key, byte0);
      out.y = encode8<SR>(v + 8, mult, key, byte0 + 4);
      if (j < p.cols && rb_ok) *reinterpret_cast<uint2 *>(p.col_data + byte0) = out;
      lds_cs[lc0 + c][rb] = static_cast<uint8_t>(code);
    }
    __syncthreads();
    // column-wise scales: kTC columns x kNRB codes, one 32-bit word per thread
    constexpr int kWordsPerCol = T::kNRB / 4;
    if (tid < kTC * kWordsPerCol) {
      const int lcol = tid / kWordsPerCol;
      const int h = tid % kWordsPerCol;
      const uint32_t j = c0 + lcol;
      const uint32_t sc = (r0 >> 4) + 4 * h;
      const uint32_t scale_cols = p.rows >> 4;
      if (j < p.cols && sc < scale_cols) {
        const uint32_t word = *reinterpret_cast<const uint32_t *>(&lds_cs[lcol][4 * h]);
        store_scale_group(p.col_scales, j, sc, scale_cols, p.swizzled != 0, word);
      }
    }
  }
}

template <int DT, bool B2D, bool RHT, bool SR>
hipError_t launch_one(const CastArgs &a, hipStream_t s) {
  using T = Tile<DT>;
  dim3 grid((a.cols + kTC - 1) / kTC, (a.rows + T::kTR - 1) / T::kTR);
  hipLaunchKernelGGL((k_cast<DT, B2D, RHT, SR>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const CastArgs &a, bool block_2d, bool rht, bool sr, hipStream_t s) {
  if (block_2d) return sr ? launch_one<DT, true, false, true>(a, s) : launch_one<DT, true, false, false>(a, s);
  if (rht) return sr ? launch_one<DT, false, true, true>(a, s) : launch_one<DT, false, true, false>(a, s);
  return sr ? launch_one<DT, false, false, true>(a, s) : launch_one<DT, false, false, false>(a, s);
}

}  // namespace

hipError_t launch_cast(const CastArgs &a, int dtype, bool block_2d, bool rht, bool sr, hipStream_t s) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  return dtype == kBF16 ? launch_dt<kBF16>(a, block_2d, rht, sr, s) : launch_dt<kFP32>(a, block_2d, rht, sr, s);
}

}  // namespace nvfp4
