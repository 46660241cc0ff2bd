// Fused NVFP4 cast-transpose for gfx950.
//
// One workgroup (256 threads, 4 waves of 64) owns a 128 x 128 tile of the
// input and writes, for that tile:
//   row-wise:    FP4 data [rows][cols/2] and E4M3 (or UE5M3) scales, 1x16
//                blocks along each input row (or the shared 16x16 block
//                scale);
//   column-wise: the same for the transposed tensor, 1x16 blocks along each
//                input column, optionally after a 16-point RHT of each
//                16-row column group.
// "Write both NVFP4 amax buffers" (Changes) and "Fuse NVFP4 scale swizzling
// on SM120 and SM121" (Description, Changes) describe one kernel writing
// both orientations, and scales stored directly in the GEMM layout with one
// 32-bit store per aligned group of four.
//
// Two kernels share this file:
//   k_cast_rt   1x16 / 16x16 blocks: each thread keeps an 8 x 8 sub-tile in
//               registers, so a column-wise byte (two consecutive rows of
//               one column) is one hardware FP4 conversion;
//   k_cast_rht  column-wise RHT: each thread keeps 16 rows x 4 columns, so a
//               column's 16-row transform group is whole in one thread.
// Both read the input once with non-temporal 128-bit (or 64-bit) loads, stage
// output bytes and scale codes in LDS, and leave them as wide coalesced
// stores (non-temporal, except the register-tile kernel's column-wise data
// and compact scales, which merge in L2). Grouped forms of both run the
// same tile code on the tiles of several row slices, one tensor per slice.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "codec.h"
#include "launch.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// End of the per-tensor amax reduction. With a caller workspace the amax
// pass leaves one maximum per workgroup (a multiple of four words, as float
// bit patterns of non-negative values, so unsigned max == float max); every
// cast workgroup reduces them itself, which costs a few cached 16-byte loads
// per thread instead of a zeroing launch and atomics in the amax pass.
// ---------------------------------------------------------------------------
constexpr int kPartialVecs = kMaxPartials / 4 / kThreads;  // 16-byte loads per thread

// Issued before the tile's loads, so that only these have to arrive before
// the reduction. An index past the end is clamped to the last vector, which
// cannot change a maximum.
__device__ __forceinline__ void load_partials(const uint32_t *part, uint32_t n, int tid,
                                              u32x4 (&v)[kPartialVecs]) {
  const u32x4 *p4 = reinterpret_cast<const u32x4 *>(part);
  const uint32_t last = n / 4 - 1;
#pragma unroll
  for (int i = 0; i < kPartialVecs; ++i) v[i] = p4[min(static_cast<uint32_t>(tid + i * kThreads), last)];
}

__device__ __forceinline__ uint32_t partials_max(const u32x4 (&v)[kPartialVecs]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kPartialVecs; ++i) m = max(m, max(max(v[i].x, v[i].y), max(v[i].z, v[i].w)));
  return m;
}

constexpr int kWaves = kThreads / 64;

// Workgroup maximum of N values per thread, returned to every thread.
// Contains a barrier; lds holds N words per wave.
template <int N>
__device__ __forceinline__ void workgroup_max(uint32_t (&m)[N], uint32_t *lds) {
#pragma unroll
  for (int i = 0; i < N; ++i) m[i] = wave_max(m[i]);
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) lds[i * kWaves + (threadIdx.x >> 6)] = m[i];
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    m[i] = lds[i * kWaves];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m[i] = max(m[i], lds[i * kWaves + w]);
  }
}

// The amax pair of a cast workgroup: from the workspace (reduced here, and
// stored to the amax buffers by the workgroup of tile (0, 0), `writer`) or
// read from the buffers.
// TWO_ARRAYS: the column-wise amax has its own array (the RHT pair); else
// both orientations take the one tensor amax.
template <bool TWO_ARRAYS>
__device__ __forceinline__ void amax_pair(const CastArgs &p, const u32x4 (&pr)[kPartialVecs],
                                          const u32x4 (&pc)[kPartialVecs], uint32_t *lds, bool writer,
                                          float &amax_row, float &amax_col) {
  if (p.partials != nullptr) {
    uint32_t m[TWO_ARRAYS ? 2 : 1];
    m[0] = partials_max(pr);
    if constexpr (TWO_ARRAYS) m[1] = partials_max(pc);
    workgroup_max(m, lds);
    amax_row = __uint_as_float(m[0]);
    amax_col = __uint_as_float(m[TWO_ARRAYS ? 1 : 0]);
    if (writer && threadIdx.x == 0) {
      if (p.row_amax) *p.row_amax = amax_row;
      if (p.col_amax) *p.col_amax = amax_col;
    }
  } else {
    amax_row = p.row_data != nullptr ? *p.row_amax : 0.0f;
    amax_col = p.col_data != nullptr ? *p.col_amax : 0.0f;
  }
}

// Codes of 8 consecutive values of one output row, packed little-endian
// (element 2i in the low nibble of byte i). byte0 = index of the first byte
// in the orientation's data array (stochastic-rounding counter).
template <bool SR>
__device__ __forceinline__ uint32_t encode8_scaled(const float *s, uint32_t key, uint32_t byte0) {
  if (!SR) return e2m1_rne_x8(s);
  uint32_t r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = fmix32(key ^ (byte0 + q));
  return e2m1_sr_x8(s, r);
}

template <bool SR>
__device__ __forceinline__ uint32_t encode8(const float *v, float e, uint32_t key, uint32_t byte0) {
  float s[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) s[k] = v[k] * e;
  return encode8_scaled<SR>(s, key, byte0);
}

// Four scales (c .. c+3 of scale row r, c % 4 == 0) packed in `word`.
// Compact scales take ordinary (cached) stores: a tile owns only 8 bytes of
// each scale row, and streamed 4-byte pieces reach HBM as partial writes
// (in a measurement they doubled the cast time); in L2 the pieces of
// neighbouring tiles merge into whole lines first.
__device__ __forceinline__ void store_scale_group(uint8_t *base, uint32_t r, uint32_t c, uint32_t scale_cols,
                                                  bool swizzled, uint32_t word) {
  if (swizzled) {
    __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(base + swizzled_scale_offset(r, c, scale_cols)));
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

// ---------------------------------------------------------------------------
// Register-tile cast (1x16 or 16x16 blocks, no RHT).
//
// A workgroup owns a 128 x 128 tile; thread (ucol = tid % 16, rg = tid / 16)
// owns the 8 x 8 sub-tile of rows 8rg..8rg+7 and columns 8ucol..8ucol+7, kept
// in registers. Each load instruction of a wave reads 4 rows x 256 contiguous
// bytes. With 8 consecutive rows in one thread, one conversion of the pair
// (row 2i, row 2i+1) of a column gives a whole column-wise output byte, so the
// column-wise side needs no transpose of the data through LDS:
//   row-wise 1x16 block   = lanes (ucol, ucol ^ 1): DPP exchange,
//   column-wise 1x16 block = lanes (rg, rg ^ 1) = lane ^ 16: swizzle exchange,
//   16x16 block            = the four lanes of both pairs: one scale per thread.
// The multiplier S / value(s) of every E4M3 code is computed once per
// workgroup (one correctly rounded division per code) and looked up in LDS.
// Scale codes and column-wise data words go through LDS so that they leave
// as 32-bit scale words and 64 contiguous bytes per column. The input is read
// once and the outputs are not read back, so loads and data stores are
// non-temporal (streamed past the caches), the column-wise pieces too,
// although a tile writes only half of each 128-byte line it touches and the
// tile below it the other half: cached, the caches merged the halves but the
// kernels measured slower (the dirty lines were written back at the end).
// Compact scale pieces are the exception (store_scale_group).
// ---------------------------------------------------------------------------
constexpr int kRT = 128;  // register-tile edge

// lane ^ 16 (bit-mask swizzle: and 0x1F, or 0, xor 0x10)
__device__ __forceinline__ uint32_t swz_xor16(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(x), 0x401F));
}

// lo ? a : b without letting the compiler turn a select between two array
// elements into a lane-dependent index (which would move the array to scratch)
__device__ __forceinline__ uint32_t pick(bool lo, uint32_t a, uint32_t b) {
  const uint32_t mask = 0u - static_cast<uint32_t>(lo);
  return b ^ ((a ^ b) & mask);
}

__device__ __forceinline__ uint32_t block_code(uint32_t m_bits, float S, bool ue5m3) {
  const float q = div6(__uint_as_float(m_bits));
  return scale_encode(q * S, ue5m3);
}

__device__ __forceinline__ float code_multiplier(uint32_t code, float S, bool ue5m3) {
  return code == 0 ? 0.0f : fminf(S / scale_decode(code, ue5m3), kFltMax);
}

// The multiplier of every scale code of both orientations, in LDS: E4M3
// has 127 finite non-negative codes (one division per thread), UE5M3 248
// (two per thread). Codes past the format's last one are never looked up.
__device__ __forceinline__ void fill_multipliers(float (&lds)[2][256], int tid, float S_row, float S_col,
                                                 bool ue5m3) {
  if (!ue5m3) {
    if (tid < 127) lds[0][tid] = code_multiplier(tid, S_row, false);
    else if (tid >= 128 && tid < 255) lds[1][tid - 128] = code_multiplier(tid - 128, S_col, false);
  } else if (tid < 248) {
    lds[0][tid] = code_multiplier(tid, S_row, true);
    lds[1][tid] = code_multiplier(tid, S_col, true);
  }
}

template <int DT>
struct RT {
  static constexpr int kElem = DT == kBF16 ? 2 : 4;
  static constexpr int kWords = 8 * kElem / 4;  // 32-bit words per 8-element row piece
};

// value c (0..7) of a row piece
template <int DT>
__device__ __forceinline__ float piece_value(const uint32_t (&w)[RT<DT>::kWords], int c) {
  if (DT == kBF16) return (c & 1) ? bf16_hi(w[c >> 1]) : bf16_lo(w[c >> 1]);
  return __uint_as_float(w[c]);
}

// max |x| bit pattern of a row piece
template <int DT>
__device__ __forceinline__ uint32_t piece_max(const uint32_t (&w)[RT<DT>::kWords]) {
  uint32_t m = 0;
  if (DT == kBF16) {
    ushort2_t h = {0, 0};
#pragma unroll
    for (int q = 0; q < 4; ++q) h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2_t, w[q] & 0x7FFF7FFFu));
    m = static_cast<uint32_t>(max(h.x, h.y)) << 16;
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) m = max(m, w[q] & 0x7FFFFFFFu);
  }
  return m;
}

// LDS of one register tile's encode.
struct RtLds {
  float mult[2][256];        // multiplier per scale code (row, col)
  // scale codes of the tile, row-wise [tile row][16-col block] and column-wise
  // [tile col][16-row block]; compact: line * 8 + block; swizzled: the two
  // 512-byte GEMM tiles that the 128 x 8 codes form, in memory order
  uint8_t rs[kRT * 8];
  uint8_t cs[kRT * 8];
  uint32_t cw[16][kRT + 1];  // column-wise data words [row group][tile col]
  uint32_t red[kWaves];
};

// Loads of the thread's 8 x 8 sub-tile of tile (r0, c0), issued without a
// branch: in an edge tile, pieces outside the input load from a clamped
// address (a value of the input, so the tile's maximum is unchanged) and are
// zeroed by rt_clear_outside before the block maxima are taken.
template <int DT>
__device__ __forceinline__ void rt_load(const CastArgs &p, uint32_t r0, uint32_t c0,
                                        uint32_t (&w)[8][RT<DT>::kWords]) {
  constexpr int W = RT<DT>::kWords;
  const uint32_t col = c0 + 8 * (threadIdx.x & 15);
  const uint32_t rbase = r0 + 8 * (threadIdx.x >> 4);
  const uint32_t lcol = col < p.cols ? col : 0u;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t r = min(rbase + k, p.rows - 1);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(p.x) +
                                                       (static_cast<uint64_t>(r) * p.cols + lcol) * RT<DT>::kElem);
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      const u32x4 t = __builtin_nontemporal_load(src + q);
      w[k][4 * q] = t.x;
      w[k][4 * q + 1] = t.y;
      w[k][4 * q + 2] = t.z;
      w[k][4 * q + 3] = t.w;
    }
  }
}

// A mask rather than a branch: a per-lane branch around array stores makes
// the compiler copy the whole register array through the branch.
template <int DT>
__device__ __forceinline__ void rt_clear_outside(const CastArgs &p, uint32_t r0, uint32_t c0,
                                                 uint32_t (&w)[8][RT<DT>::kWords]) {
  if (r0 + kRT <= p.rows && c0 + kRT <= p.cols) return;  // an interior tile has nothing outside (uniform)
  const uint32_t col = c0 + 8 * (threadIdx.x & 15);
  const uint32_t rbase = r0 + 8 * (threadIdx.x >> 4);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t keep = 0u - static_cast<uint32_t>(col < p.cols && rbase + k < p.rows);
#pragma unroll
    for (int q = 0; q < RT<DT>::kWords; ++q) w[k][q] &= keep;
  }
}

template <int DT, bool B2D, bool SR, bool PRE = false, bool RS = false>
__device__ __forceinline__ void rt_encode(const CastArgs &p, uint32_t tx, uint32_t ty,
                                          uint32_t (&w)[8][RT<DT>::kWords], float S_row, float S_col, bool ue,
                                          RtLds &sh, uint32_t m2d = 0);

// The 16x16 block maximum (bit pattern) of the thread's sub-tile, taken over
// the four lanes that share the block.
template <int DT>
__device__ __forceinline__ uint32_t block2d_max(const uint32_t (&w)[8][RT<DT>::kWords]) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = max(m, piece_max<DT>(w[k]));
  m = max(m, dpp_mov<kQuadXor1>(m));
  return max(m, swz_xor16(m));
}

template <int DT, bool B2D, bool SR>
__device__ __forceinline__ void cast_rt_tile(const CastArgs &p, uint32_t tx, uint32_t ty) {
  constexpr int W = RT<DT>::kWords;
  __shared__ RtLds sh;

  if (p.noop != nullptr && *p.noop == 1.0f) return;

  const int tid = threadIdx.x;
  const uint32_t r0 = ty * kRT;
  const uint32_t c0 = tx * kRT;

  u32x4 part[kPartialVecs];
  if (p.partials != nullptr) load_partials(p.partials, p.npartials, tid, part);

  // Every thread issues all its loads without a branch, so that the wait for
  // the workspace loads above does not have to wait for these too.
  uint32_t w[8][W];
  rt_load<DT>(p, r0, c0, w);

  float amax_row, amax_col;
  amax_pair<false>(p, part, part, sh.red, (tx | ty) == 0, amax_row, amax_col);
  const bool ue = p.ue5m3 != 0;
  const float S_row = p.row_data != nullptr ? global_encode_scale(amax_row, ue) : 1.0f;
  const float S_col = p.col_data != nullptr ? global_encode_scale(amax_col, ue) : 1.0f;
  fill_multipliers(sh.mult, tid, S_row, S_col, ue);
  rt_encode<DT, B2D, SR>(p, tx, ty, w, S_row, S_col, ue, sh);
}

// Block scales, codes and stores of one tile whose values are in w (zero
// outside the input) and whose multipliers are in sh.mult; sh.mult is read
// only after the barrier below, so the caller may fill it right before.
// PRE: the caller has cleared w outside the input and, with 16x16 blocks,
// passes the block maximum in m2d.
// RS (row-scaled, 1x16 blocks): every row and every column has a global
// scale of its own, which the caller has put in sh.mult[0][tile row] and
// sh.mult[1][tile column] before a barrier; S_row and S_col are unused, and
// each block's multiplier is divided out from its own scale rather than
// looked up.
template <int DT, bool B2D, bool SR, bool PRE, bool RS>
__device__ __forceinline__ void rt_encode(const CastArgs &p, uint32_t tx, uint32_t ty,
                                          uint32_t (&w)[8][RT<DT>::kWords], float S_row, float S_col, bool ue,
                                          RtLds &sh, uint32_t m2d) {
  static_assert(!(RS && B2D), "row-scaled tiles have 1x16 blocks");
  const int tid = threadIdx.x;
  const int ucol = tid & 15;
  const int rg = tid >> 4;
  const uint32_t r0 = ty * kRT;
  const uint32_t c0 = tx * kRT;
  const uint32_t col = c0 + 8 * ucol;
  const uint32_t rbase = r0 + 8 * rg;
  const bool col_ok = col < p.cols;
  const bool do_row = p.row_data != nullptr;
  const bool do_col = p.col_data != nullptr;

  if (!PRE) rt_clear_outside<DT>(p, r0, c0, w);
  // 16x16 blocks with equal row and column global scales share their codes
  // and every product (a uniform branch: the scales come from the same two
  // amax words in every lane)
  const bool share = B2D && do_row && do_col && __builtin_amdgcn_readfirstlane(S_row == S_col);

  // ---- block scale codes ----
  uint32_t rcode[8], ccode[8];
  float rmul[RS ? 8 : 1], cmul[RS ? 8 : 1];  // RS: the blocks' multipliers
  if (B2D) {
    const uint32_t m = PRE ? m2d : block2d_max<DT>(w);
    const uint32_t cr = block_code(m, S_row, ue);
    const uint32_t cc = share ? cr : block_code(m, S_col, ue);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      rcode[k] = cr;
      ccode[k] = cc;
    }
  } else {
    if (do_row) {
      // row k's block is this piece and the neighbour lane's piece; the two
      // lanes split the eight divisions and swap results.
      uint32_t mr[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        mr[k] = piece_max<DT>(w[k]);
        mr[k] = max(mr[k], dpp_mov<kQuadXor1>(mr[k]));
      }
      const bool lo = (ucol & 1) == 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float S = RS ? sh.mult[0][8 * rg + (lo ? j : j + 4)] : S_row;
        const uint32_t mine = block_code(pick(lo, mr[j], mr[j + 4]), S, ue);
        const uint32_t other = dpp_mov<kQuadXor1>(mine);
        rcode[j] = pick(lo, mine, other);
        rcode[j + 4] = pick(lo, other, mine);
        if (RS) {
          const uint32_t mm = __float_as_uint(code_multiplier(mine, S, ue));
          const uint32_t om = dpp_mov<kQuadXor1>(mm);
          rmul[j] = __uint_as_float(pick(lo, mm, om));
          rmul[j + 4] = __uint_as_float(pick(lo, om, mm));
        }
      }
    }
    if (do_col) {
      // column c's block is this thread's 8 rows and lane ^ 16's 8 rows.
      uint32_t mc[8];
      if (DT == kBF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ushort2_t h = {0, 0};
#pragma unroll
          for (int k = 0; k < 8; ++k) h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2_t, w[k][q] & 0x7FFF7FFFu));
          uint32_t both = __builtin_bit_cast(uint32_t, h);
          both = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, both),
                                                                        __builtin_bit_cast(ushort2_t, swz_xor16(both))));
          mc[2 * q] = both << 16;
          mc[2 * q + 1] = both & 0xFFFF0000u;
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          uint32_t m = 0;
#pragma unroll
          for (int k = 0; k < 8; ++k) m = max(m, w[k][c] & 0x7FFFFFFFu);
          mc[c] = max(m, swz_xor16(m));
        }
      }
      const bool lo = (rg & 1) == 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float S = RS ? sh.mult[1][8 * ucol + (lo ? j : j + 4)] : S_col;
        const uint32_t mine = block_code(pick(lo, mc[j], mc[j + 4]), S, ue);
        const uint32_t other = swz_xor16(mine);
        ccode[j] = pick(lo, mine, other);
        ccode[j + 4] = pick(lo, other, mine);
        if (RS) {
          const uint32_t mm = __float_as_uint(code_multiplier(mine, S, ue));
          const uint32_t om = swz_xor16(mm);
          cmul[j] = __uint_as_float(pick(lo, mm, om));
          cmul[j + 4] = __uint_as_float(pick(lo, om, mm));
        }
      }
    }
  }
  // codes to LDS (one writer per block and row / column)
  const bool swz = p.swizzled != 0;
  auto code_slot = [swz](int line, int blk) {
    return swz ? ((blk >> 2) << 9) + ((line & 31) << 4) + ((line >> 5) << 2) + (blk & 3) : line * 8 + blk;
  };
  // A thread's eight lines are consecutive and stay inside one group of 32,
  // so their slots are the first one's plus 16 k (swizzled) or 8 k (compact):
  // constant offsets, in a uniform branch per layout.
  auto put8 = [swz](uint8_t *dst, int first, const uint32_t (&code)[8]) {
    if (swz) {
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[first + 16 * k] = static_cast<uint8_t>(code[k]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[first + 8 * k] = static_cast<uint8_t>(code[k]);
    }
  };
  if (do_row && (ucol & 1) == 0) put8(sh.rs, code_slot(8 * rg, ucol >> 1), rcode);
  if (do_col && (rg & 1) == 0) put8(sh.cs, code_slot(8 * ucol, rg >> 1), ccode);
  lds_barrier();

  float re[8], ce[8];
  if (B2D) {  // one block per thread: one multiplier per orientation
    const float r = do_row ? sh.mult[0][rcode[0]] : 0.0f;
    const float c = do_col ? sh.mult[1][ccode[0]] : 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      re[k] = r;
      ce[k] = c;
    }
  } else if (RS) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      re[k] = do_row ? rmul[k] : 0.0f;
      ce[k] = do_col ? cmul[k] : 0.0f;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      re[k] = do_row ? sh.mult[0][rcode[k]] : 0.0f;
      ce[k] = do_col ? sh.mult[1][ccode[k]] : 0.0f;
    }
  }
  // interior tiles (uniform) store without per-lane bounds checks
  const bool interior = r0 + kRT <= p.rows && c0 + kRT <= p.cols;

  // ---- encode: row pairs (2i, 2i+1) ----
  const uint32_t krow = SR ? sr_key(p.sr_seed, 0) : 0u;
  const uint32_t kcol = SR ? sr_key(p.sr_seed, 1) : 0u;
  const uint32_t half_cols = p.cols >> 1;
  const uint32_t half_rows = p.rows >> 1;
  uint32_t colw[8];  // byte i is written in row pair i; every byte is written
  // Nearest even with shared codes and products: the column-wise codes are
  // the row-wise codes (the conversion rounds each value on its own), so the
  // column-wise bytes are the row-wise words' nibbles rearranged; masks and
  // byte permutes cost about half the second set of conversions.
  uint32_t ev[4], od[4];
  const bool from_rows = !SR && share;  // uniform
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v0[8], v1[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      v0[c] = piece_value<DT>(w[2 * i], c);
      v1[c] = piece_value<DT>(w[2 * i + 1], c);
    }
    float s0[8], s1[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      s0[c] = v0[c] * re[2 * i];
      s1[c] = v1[c] * re[2 * i + 1];
    }
    if (do_row) {
      const uint32_t row = rbase + 2 * i;
      const uint32_t byte0 = row * half_cols + (col >> 1);
      const uint32_t word0 = encode8_scaled<SR>(s0, krow, byte0);
      const uint32_t word1 = encode8_scaled<SR>(s1, krow, byte0 + half_cols);
      if (from_rows) {
        // the column-wise byte of column c in this row pair is nibble c of
        // word0 (low nibble) and of word1 (high): gather the bytes of the
        // even columns and of the odd columns
        ev[i] = (word0 & 0x0F0F0F0Fu) | ((word1 << 4) & 0xF0F0F0F0u);
        od[i] = ((word0 >> 4) & 0x0F0F0F0Fu) | (word1 & 0xF0F0F0F0u);
      }
      uint32_t *dst = reinterpret_cast<uint32_t *>(p.row_data + byte0);
      if (interior) {
        __builtin_nontemporal_store(word0, dst);
        __builtin_nontemporal_store(word1, dst + (half_cols >> 2));
      } else {
        if (col_ok && row < p.rows) __builtin_nontemporal_store(word0, dst);
        if (col_ok && row + 1 < p.rows) __builtin_nontemporal_store(word1, dst + (half_cols >> 2));
      }
    }
    if (do_col && !from_rows) {
      float t0[8], t1[8];
      if (share) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          t0[c] = s0[c];
          t1[c] = s1[c];
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          t0[c] = v0[c] * ce[c];
          t1[c] = v1[c] * ce[c];
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float a = t0[c];
        const float b = t1[c];
        if (SR) {
          const uint32_t byte = (col + c) * half_rows + (rbase >> 1) + i;
          colw[c] = e2m1_sr_pair_into(i == 0 ? __float_as_uint(a) : colw[c], a, b, fmix32(kcol ^ byte), i);
        } else {
          colw[c] = e2m1_rne_pair_into(i == 0 ? __float_as_uint(a) : colw[c], a, b, i);
        }
      }
    }
  }
  if (from_rows) {
    // 4x4 byte transposes: colw[2k] byte i = ev[i] byte k, colw[2k+1] byte i = od[i] byte k
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t (&x)[4] = h ? od : ev;
      const uint32_t lo01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);
      const uint32_t hi01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);
      const uint32_t lo23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
      const uint32_t hi23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
      colw[0 + h] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
      colw[2 + h] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
      colw[4 + h] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
      colw[6 + h] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
    }
  }
  if (do_col) {
#pragma unroll
    for (int c = 0; c < 8; ++c) sh.cw[rg][8 * ucol + c] = colw[c];
  }

  if (do_col) {
    lds_barrier();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int e = tid + kThreads * it;
      const int lc = e >> 2, h = e & 3;
      const uint32_t j = c0 + lc;
      const uint32_t rr = r0 + 32 * h;
      if (j < p.cols && rr < p.rows) {
        uint8_t *dst = p.col_data + j * half_rows + (rr >> 1);
        // streamed: with cached stores the end of the kernel still had the
        // dirty lines to write back (8192x5120 16x16 single pass: 30.8 ->
        // 29.9 us per call)
        if (rr + 32 <= p.rows)
          __builtin_nontemporal_store(
              u32x4{sh.cw[4 * h][lc], sh.cw[4 * h + 1][lc], sh.cw[4 * h + 2][lc], sh.cw[4 * h + 3][lc]},
              reinterpret_cast<u32x4 *>(dst));
        else
          *reinterpret_cast<u32x2 *>(dst) = u32x2{sh.cw[4 * h][lc], sh.cw[4 * h + 1][lc]};
      }
    }
  }
  // ---- scales: 128 rows (or columns) x 8 codes = one 32-bit word per thread ----
  if (swz) {
    // the tile's codes are two whole GEMM tiles, 1 KiB contiguous per orientation
    // (swizzled shapes are multiples of 128, so every tile is complete)
    if (do_row)
      __builtin_nontemporal_store(reinterpret_cast<const uint32_t *>(sh.rs)[tid],
                                  reinterpret_cast<uint32_t *>(p.row_scales + swizzled_scale_offset(r0, c0 >> 4, p.cols >> 4)) + tid);
    if (do_col)
      __builtin_nontemporal_store(reinterpret_cast<const uint32_t *>(sh.cs)[tid],
                                  reinterpret_cast<uint32_t *>(p.col_scales + swizzled_scale_offset(c0, r0 >> 4, p.rows >> 4)) + tid);
    return;
  }
  const int t_line = tid >> 1;
  const int t_half = tid & 1;
  if (do_row) {
    const uint32_t row = r0 + t_line;
    const uint32_t sc = (c0 >> 4) + 4 * t_half;
    const uint32_t scale_cols = p.cols >> 4;
    if (row < p.rows && sc < scale_cols)
      store_scale_group(p.row_scales, row, sc, scale_cols, false,
                        reinterpret_cast<const uint32_t *>(sh.rs)[tid]);
  }
  if (do_col) {
    const uint32_t j = c0 + t_line;
    const uint32_t sc = (r0 >> 4) + 4 * t_half;
    const uint32_t scale_cols = p.rows >> 4;
    if (j < p.cols && sc < scale_cols)
      store_scale_group(p.col_scales, j, sc, scale_cols, false,
                        reinterpret_cast<const uint32_t *>(sh.cs)[tid]);
  }
}

// ---------------------------------------------------------------------------
// Register-tile cast with the column-wise RHT.
//
// A workgroup owns a 128 x 128 tile; thread (cg = tid % 32, rq = tid / 32)
// owns rows 16rq..16rq+15 of columns 4cg..4cg+3, so each column's 16-row
// RHT group is whole in one thread: the transform, the block maximum and
// the eight output bytes of that column need no lane exchange. A wave's load
// reads 2 rows x 256 contiguous bytes. Row-wise (plain) 1x16 blocks are lane
// quads (DPP). Row-wise and column-wise data bytes are staged in LDS and
// leave as 16-byte stores (64 contiguous bytes per row / column).
// ---------------------------------------------------------------------------
template <int DT, bool SR, bool MFMA>
__device__ __forceinline__ void cast_rht_tile(const CastArgs &p, uint32_t tx, uint32_t ty) {
  static_assert(!MFMA || DT == kBF16, "the matrix-core transform takes BF16 input");
  constexpr int kElem = DT == kBF16 ? 2 : 4;
  constexpr int W = kElem;  // 32-bit words per 4-column row piece: 2 (BF16) or 4 (FP32)
  __shared__ float lds_mult[2][256];
  __shared__ __align__(4) uint8_t lds_rs[kRT * 8];
  __shared__ __align__(4) uint8_t lds_cs[kRT * 8];
  __shared__ __align__(16) uint8_t lds_rd[kRT][64 + 16];  // row-wise data bytes (padded rows)
  __shared__ __align__(16) uint8_t lds_cd[kRT][64 + 16];  // column-wise data bytes
  __shared__ uint32_t lds_red[2 * kWaves];

  if (p.noop != nullptr && *p.noop == 1.0f) return;

  const int tid = threadIdx.x;
  const int cg = tid & 31;
  const int rq = tid >> 5;
  const uint32_t r0 = ty * kRT;
  const uint32_t c0 = tx * kRT;
  const uint32_t col = c0 + 4 * cg;
  const uint32_t rbase = r0 + 16 * rq;
  const bool col_ok = col < p.cols;
  const bool do_row = p.row_data != nullptr;
  const bool do_col = p.col_data != nullptr;

  u32x4 part_row[kPartialVecs], part_col[kPartialVecs];
  if (p.partials != nullptr) {
    load_partials(p.partials, p.npartials, tid, part_row);
    load_partials(p.partials + kMaxPartials, p.npartials, tid, part_col);
  }

  // Every thread issues all its loads without a branch (see k_cast_rt); in
  // an edge tile, pieces outside the input load from a clamped address and
  // are zeroed afterwards.
  const bool interior = r0 + kRT <= p.rows && c0 + kRT <= p.cols;  // uniform
  const uint32_t lcol = col_ok ? col : 0u;
  // interior tiles: one uniform base per row of the thread's group and one
  // 32-bit lane offset for all 16 loads (scalar address arithmetic); the
  // offset stays below 2^32 while 128 rows of the input do
  const bool lane_offset = interior && p.cols <= (1u << 22);  // uniform
  const uint8_t *tile_base = static_cast<const uint8_t *>(p.x) + static_cast<uint64_t>(r0) * p.cols * kElem;
  const uint32_t lane_off = ((rbase - r0) * p.cols + col) * kElem;
  uint32_t w[16][W];
  auto load_piece = [&](int k, const uint8_t *src) {
    if constexpr (DT == kBF16) {
      const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(src));
      w[k][0] = t.x;
      w[k][1] = t.y;
    } else {
      const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
      w[k][0] = t.x;
      w[k][1] = t.y;
      w[k][2] = t.z;
      w[k][3] = t.w;
    }
  };
  if (lane_offset) {
#pragma unroll
    for (int k = 0; k < 16; ++k) load_piece(k, tile_base + static_cast<uint64_t>(k) * p.cols * kElem + lane_off);
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t r = min(rbase + k, p.rows - 1);
      load_piece(k, static_cast<const uint8_t *>(p.x) + (static_cast<uint64_t>(r) * p.cols + lcol) * kElem);
    }
  }
  auto value = [&](int k, int c) -> float {
    if constexpr (DT == kBF16) return (c & 1) ? bf16_hi(w[k][c >> 1]) : bf16_lo(w[k][c >> 1]);
    else return __uint_as_float(w[k][c]);
  };

  float amax_row, amax_col;
  amax_pair<true>(p, part_row, part_col, lds_red, (tx | ty) == 0, amax_row, amax_col);
  const bool ue = p.ue5m3 != 0;
  const float S_row = do_row ? global_encode_scale(amax_row, ue) : 1.0f;
  const float S_col = do_col ? global_encode_scale(amax_col, ue) : 1.0f;
  fill_multipliers(lds_mult, tid, S_row, S_col, ue);
  if (!interior) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (!(col_ok && rbase + k < p.rows)) {
#pragma unroll
        for (int q = 0; q < W; ++q) w[k][q] = 0;
      }
    }
  }
  const bool swz = p.swizzled != 0;
  auto code_slot = [swz](int line, int blk) {
    return swz ? ((blk >> 2) << 9) + ((line & 31) << 4) + ((line >> 5) << 2) + (blk & 3) : line * 8 + blk;
  };

  // ---- row-wise block codes: row k's block is the lane quad's 16 values ----
  uint32_t rcode[16];
  if (do_row) {
    const int q = cg & 3;
    uint32_t mine[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) mine[j] = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      // max |x| of the row piece: BF16 as a packed 16-bit max of the
      // magnitude bits (no unpacking), FP32 as a float max with abs
      // modifiers; for finite inputs both are the max of the |x| bit patterns
      uint32_t m;
      if constexpr (DT == kBF16) {
        const ushort2_t h = __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, w[k][0] & 0x7FFF7FFFu),
                                                      __builtin_bit_cast(ushort2_t, w[k][1] & 0x7FFF7FFFu));
        m = static_cast<uint32_t>(max(h.x, h.y)) << 16;
      } else {
        m = __float_as_uint(fmaxf(fmaxf(fabsf(value(k, 0)), fabsf(value(k, 1))),
                                  fmaxf(fabsf(value(k, 2)), fabsf(value(k, 3)))));
      }
      m = max(m, dpp_mov<kQuadXor1>(m));
      m = max(m, dpp_mov<kQuadXor2>(m));
      // quad lane q turns rows q, q+4, q+8, q+12 into codes
      if ((k & 3) == 0) mine[k >> 2] = m;
      else mine[k >> 2] = pick(q == (k & 3), m, mine[k >> 2]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) mine[j] = block_code(mine[j], S_row, ue);
#pragma unroll
    for (int k = 0; k < 16; ++k) rcode[k] = quad_bcast(mine[k >> 2], k & 3);
    if (q == 0) {
#pragma unroll
      for (int k = 0; k < 16; ++k) lds_rs[code_slot(16 * rq + k, cg >> 2)] = static_cast<uint8_t>(rcode[k]);
    }
  }
  __syncthreads();  // multipliers ready

  // ---- encode ----
  // Stochastic rounding: each row piece (two output bytes) and each column
  // half (four bytes) is a run of consecutive output bytes (e2m1_sr_run). Where
  // the global scales allow it (sr_fold_ok, uniform), the 2^23 of the SR
  // preparation is folded into each block's multiplier.
  const uint32_t half_cols = p.cols >> 1;
  const uint32_t half_rows = p.rows >> 1;
  auto encode_rows = [&](auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    const uint32_t kmix = SR ? sr_key_mix(sr_key(p.sr_seed, 0)) : 0u;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float e = lds_mult[0][rcode[k]];
      uint32_t h;
      if constexpr (SR) {
        float t[4];
        if constexpr (FAST) {
          const float ef = e * kSrScale;
#pragma unroll
          for (int c = 0; c < 4; ++c) t[c] = sr_prepare_folded(value(k, c), ef);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) t[c] = sr_prepare(value(k, c) * e);
        }
        // bytes b0, b0 + 1 of the row, b0 even
        h = e2m1_sr_run<2, 0>(t, sr_run_mix((rbase + k) * half_cols + (col >> 1)), kmix);
      } else {
        const float s0 = value(k, 0) * e, s1 = value(k, 1) * e, s2 = value(k, 2) * e, s3 = value(k, 3) * e;
        h = e2m1_rne_pair_into(__float_as_uint(s0), s0, s1, 0);
        h = e2m1_rne_pair_into(h, s2, s3, 1);
      }
      *reinterpret_cast<uint16_t *>(&lds_rd[16 * rq + k][2 * cg]) = static_cast<uint16_t>(h);
    }
  };

  // Column-wise: RHT of each 16-row column group, then encode. The
  // transform's sign flips go on whole input words (one sign per row; the
  // row-wise side is done with them), and its 1/4 is folded into the block
  // max (exact: rounding is monotonic) and into the multiplier (exact: a
  // power of two), so each column runs the unnormalized transform only.
  float tv[4][16];   // unnormalized transformed values of the thread's 4 columns
  uint32_t ccode[4];  // their block scale codes
  auto transform_cols = [&]() {
    // MFMA: the 4x4 matrix-core form (fwht16_mfma), signs in its operands;
    // else butterflies on the vector ALU after sign flips on whole words
    uint32_t a1[4][2];
    float a2[4];
    if constexpr (MFMA) {
      fwht16_mfma_operands(p.sign_mask, a1, a2);
    } else {
      constexpr uint32_t kSign = DT == kBF16 ? 0x80008000u : 0x80000000u;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
#pragma unroll
        for (int q = 0; q < W; ++q) w[k][q] ^= ((p.sign_mask >> k) & 1u) ? kSign : 0u;  // uniform select
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (MFMA) {
        // rows (4j, 4j+1) and (4j+2, 4j+3) of column c as BF16 pairs
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        uint32_t x2[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x2[j][0] = __builtin_amdgcn_perm(w[4 * j + 1][c >> 1], w[4 * j][c >> 1], sel);
          x2[j][1] = __builtin_amdgcn_perm(w[4 * j + 3][c >> 1], w[4 * j + 2][c >> 1], sel);
        }
        fwht16_mfma(x2, a1, a2, tv[c]);
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) tv[c][k] = value(k, c);
        fwht16(tv[c]);
      }
      // BF16 transformed values: bf16(4t) == 4 bf16(t), so the unnormalized
      // values are rounded and the folding of 1/4 below stays as it is
      if (p.sign_mask & kRhtBf16) bf16_round16(tv[c]);
      float ms = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) ms = fmaxf(ms, fabsf(tv[c][k]));
      ccode[c] = block_code(__float_as_uint(ms * 0.25f), S_col, ue);
      lds_cs[code_slot(4 * cg + c, rq)] = static_cast<uint8_t>(ccode[c]);
    }
  };
  auto encode_cols = [&](auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    const uint32_t kmix = SR ? sr_key_mix(sr_key(p.sr_seed, 1)) : 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v[16];
      uint32_t lo, hi;
      if constexpr (SR) {
        if constexpr (FAST) {
          const float ef = lds_mult[1][ccode[c]] * (kSrScale * 0.25f);
#pragma unroll
          for (int k = 0; k < 16; ++k) v[k] = sr_prepare_folded(tv[c][k], ef);
        } else {
          const float e = lds_mult[1][ccode[c]] * 0.25f;
#pragma unroll
          for (int k = 0; k < 16; ++k) v[k] = sr_prepare(tv[c][k] * e);
        }
        // bytes b0 .. b0 + 7 of column col + c, b0 a multiple of 8
        const uint32_t run = sr_run_mix((col + c) * half_rows + (rbase >> 1));
        lo = e2m1_sr_run<4, 0>(v, run, kmix);
        hi = e2m1_sr_run<4, 4>(v + 8, run, kmix);
      } else {
        const float e = lds_mult[1][ccode[c]] * 0.25f;
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = tv[c][k] * e;
        lo = e2m1_rne_x8(v);
        hi = e2m1_rne_x8(v + 8);
      }
      *reinterpret_cast<u32x2 *>(&lds_cd[4 * cg + c][8 * rq]) = u32x2{lo, hi};
    }
  };

  // one uniform choice per tile; only the stochastic encode differs
  const bool fast = SR && __builtin_amdgcn_readfirstlane((!do_row || sr_fold_ok(S_row, ue, DT == kFP32, 1)) &&
                                                         (!do_col || sr_fold_ok(S_col, ue, DT == kFP32, 4)));
  if (do_row) {
    if (fast) encode_rows(std::integral_constant<bool, SR>{});
    else encode_rows(std::false_type{});
  }
  if (do_col) {
    transform_cols();
    if (fast) encode_cols(std::integral_constant<bool, SR>{});
    else encode_cols(std::false_type{});
  }
  __syncthreads();

  // ---- data: 128 lines x 64 bytes per orientation, 16 bytes per store ----
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int e = tid + kThreads * it;
    const int line = e >> 2, part = e & 3;
    if (do_row) {
      const uint32_t row = r0 + line;
      const uint32_t cc = c0 + 32 * part;  // first column of this 16-byte piece
      if (row < p.rows && cc < p.cols) {
        uint8_t *dst = p.row_data + row * (p.cols >> 1) + (cc >> 1);
        const u32x4 val = *reinterpret_cast<const u32x4 *>(&lds_rd[line][16 * part]);
        if (cc + 32 <= p.cols)
          __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(dst));
        else
          __builtin_nontemporal_store(u32x2{val.x, val.y}, reinterpret_cast<u32x2 *>(dst));
      }
    }
    if (do_col) {
      const uint32_t j = c0 + line;
      const uint32_t rr = r0 + 32 * part;
      if (j < p.cols && rr < p.rows) {
        uint8_t *dst = p.col_data + j * (p.rows >> 1) + (rr >> 1);
        const u32x4 val = *reinterpret_cast<const u32x4 *>(&lds_cd[line][16 * part]);
        if (rr + 32 <= p.rows)
          __builtin_nontemporal_store(val, reinterpret_cast<u32x4 *>(dst));
        else
          __builtin_nontemporal_store(u32x2{val.x, val.y}, reinterpret_cast<u32x2 *>(dst));
      }
    }
  }

  // ---- scales ----
  if (swz) {
    if (do_row)
      __builtin_nontemporal_store(reinterpret_cast<const uint32_t *>(lds_rs)[tid],
                                  reinterpret_cast<uint32_t *>(p.row_scales + swizzled_scale_offset(r0, c0 >> 4, p.cols >> 4)) + tid);
    if (do_col)
      __builtin_nontemporal_store(reinterpret_cast<const uint32_t *>(lds_cs)[tid],
                                  reinterpret_cast<uint32_t *>(p.col_scales + swizzled_scale_offset(c0, r0 >> 4, p.rows >> 4)) + tid);
    return;
  }
  const int t_line = tid >> 1;
  const int t_half = tid & 1;
  if (do_row) {
    const uint32_t row = r0 + t_line;
    const uint32_t sc = (c0 >> 4) + 4 * t_half;
    if (row < p.rows && sc < (p.cols >> 4))
      store_scale_group(p.row_scales, row, sc, p.cols >> 4, false, reinterpret_cast<const uint32_t *>(lds_rs)[tid]);
  }
  if (do_col) {
    const uint32_t j = c0 + t_line;
    const uint32_t sc = (r0 >> 4) + 4 * t_half;
    if (j < p.cols && sc < (p.rows >> 4))
      store_scale_group(p.col_scales, j, sc, p.rows >> 4, false, reinterpret_cast<const uint32_t *>(lds_cs)[tid]);
  }
}

// Tile order. Workgroups go to the 8 XCDs round-robin (workgroup i to XCD
// i % 8). With compact scales a tile owns 8 bytes of each scale row, and the
// pieces of horizontally adjacent tiles share lines, so each XCD takes a
// contiguous run of the row-major tile order (i -> its position within
// the run of XCD i % 8): neighbours then run together on one XCD and L2
// merges their pieces. With swizzled scales each tile writes whole blocks,
// and the launch order measured faster.
__device__ __forceinline__ uint32_t tile_index(const CastArgs &p, uint32_t i, uint32_t n) {
  if (p.swizzled) return i;
  const uint32_t x = i & 7u, q = n >> 3, r = n & 7u;
  return x * q + min(x, r) + (i >> 3);
}

// Tile (tx, ty) at position L of a tx_n x ty_n tile grid. Swizzled scales:
// row-major. Compact scales: row-major over 8 x 8 blocks of tiles (edge
// blocks partial), row-major inside a block, so that one XCD's run covers
// tiles that are neighbours both across (row-wise scale pieces) and down
// (column-wise scale pieces): 5120x8192 2D compact 41.6 -> 38.2 us.
__device__ __forceinline__ void tile_xy(const CastArgs &p, uint32_t L, uint32_t tx_n, uint32_t ty_n, uint32_t &tx,
                                        uint32_t &ty) {
  if (p.swizzled) {
    ty = L / tx_n;
    tx = L - ty * tx_n;
    return;
  }
  constexpr uint32_t B = 8;
  const uint32_t by = L / (B * tx_n);
  const uint32_t rem = L - by * B * tx_n;
  const uint32_t h = min(B, ty_n - B * by);            // rows of this block row
  const uint32_t bx = min(rem / (B * h), (tx_n - 1) / B);  // full-width blocks come first
  const uint32_t rem2 = rem - bx * B * h;
  const uint32_t w = min(B, tx_n - B * bx);            // columns of this block
  ty = B * by + rem2 / w;
  tx = B * bx + rem2 % w;
}

template <int DT, bool B2D, bool SR>
__global__ __launch_bounds__(kThreads) void k_cast_rt(CastArgs p) {
  const uint32_t t = tile_index(p, blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  uint32_t tx, ty;
  tile_xy(p, t, gridDim.x, gridDim.y, tx, ty);
  cast_rt_tile<DT, B2D, SR>(p, tx, ty);
}

// Row-scaled quantize of one tile per workgroup: the global scales of the
// tile's 128 rows and 128 columns from the per-row and per-column amax
// arrays (p.row_amax, p.col_amax), one division per thread, then the tile
// encode with each block's multiplier divided out from its own scale
// ("Implement row-scaled NVFP4 fprop recipe", Greptile summary: block scales
// relative to a per-row amax; the column-wise side relative to a per-column
// amax as the review thread of "Write both NVFP4 amax buffers" sizes it).
template <int DT, bool SR>
__global__ __launch_bounds__(kThreads) void k_cast_rt_rowscaled(CastArgs p) {
  constexpr int W = RT<DT>::kWords;
  __shared__ RtLds sh;
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  const uint32_t t = tile_index(p, blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  uint32_t tx, ty;
  tile_xy(p, t, gridDim.x, gridDim.y, tx, ty);
  const int tid = threadIdx.x;
  const uint32_t r0 = ty * kRT, c0 = tx * kRT;
  uint32_t w[8][W];
  rt_load<DT>(p, r0, c0, w);
  const bool ue = p.ue5m3 != 0;
  if (tid < kRT) {
    const uint32_t r = r0 + tid;
    sh.mult[0][tid] = p.row_data != nullptr && r < p.rows ? global_encode_scale(p.row_amax[r], ue) : 1.0f;
  } else {
    const uint32_t c = c0 + (tid - kRT);
    sh.mult[1][tid - kRT] = p.col_data != nullptr && c < p.cols ? global_encode_scale(p.col_amax[c], ue) : 1.0f;
  }
  lds_barrier();
  rt_encode<DT, false, SR, false, true>(p, tx, ty, w, 1.0f, 1.0f, ue, sh);
}

template <int DT, bool SR, bool MFMA>
__global__ __launch_bounds__(kThreads) void k_cast_rht(CastArgs p) {
  const uint32_t t = tile_index(p, blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  uint32_t tx, ty;
  tile_xy(p, t, gridDim.x, gridDim.y, tx, ty);
  cast_rht_tile<DT, SR, MFMA>(p, tx, ty);
}

// ---------------------------------------------------------------------------
// Single-pass register-tile cast (per-tensor amax, no RHT).
//
// Every block scale depends on the amax of the whole input, so the
// two-launch form reads the input twice: in the amax pass and in the cast.
// Here each workgroup first loads its K tiles (tiles L = blockIdx.x +
// k * gridDim.x, k < K, in the launch order of k_cast_rt) into registers,
// the last one into LDS in one variant, publishes the maximum of its tiles,
// waits until the grid's maximum is known, and encodes its tiles from
// registers: the input is read once. The host sizes the grid so that all of
// it can be resident at once (at most the occupancy limit, and at most four
// workgroups, per CU times the CU count), but the kernel does not rely on
// it: while other streams' kernels hold CUs, part of the grid may start
// only after the rest has finished.
//
// Handoff (workspace words in launch.h), with relaxed agent-scope atomics
// only: ordered read-modify-write atomics and fences at agent scope write
// back or invalidate a whole L2 each, and with hundreds of workgroups they
// cost tens of microseconds. A call tags its words with t = e + 1, e being
// the epoch read at the start. Workgroup i marks its slot started
// (t << 32 | kSlotStarted) as it starts, and stores t << 32 | max once it
// has the maximum of its tiles.
//   Fast path: the first workgroup of each group of kSlotGroup waits (one
//   64-lane load per poll) until its members' slots carry maxima tagged t,
//   and stores the group's maximum, tagged, to the group slot; every
//   workgroup waits for all group slots (at most 32, one load per poll), or
//   for the done word, and reduces them.
//   Slow path, after fast_ticks of waiting, or as soon as the wait shows
//   workgroups that have not started (handoff_fast): the workgroup claims,
//   by compare-and-swap, the slots among kClaimSpan slots from a spread
//   start that no workgroup of this call has touched yet (their owners have
//   not started), takes the maximum of each such workgroup's tiles from
//   memory and stores it, tagged, to the slot. Then the first workgroup to
//   tag the reducer word claims what is left over every slot, waits until
//   every slot carries a maximum tagged t, reduces them and stores the
//   result to the done word; the others wait for the done word. Every slot
//   the reducer waits for belongs to a workgroup that is running, its owner
//   or its claimer, so the wait ends however many workgroups the hardware
//   runs at once; an owner that starts later stores the same maximum over
//   its claimer's and takes the done word. Only the chunks of workgroups
//   that had not started are read twice. The slow path is bounded all the
//   same (kLastResortTicks): past it, and in a workspace whose exit
//   counters are not in a state that a call left, a workgroup takes the
//   maximum of the whole input itself.
// No value of an earlier call can pass for this call's: the epoch advances
// once per call, when the last workgroup counts out (exit counters, which
// a workgroup passes once it holds the call's maximum, before its encode),
// so every workgroup of a call reads the same epoch, even one that starts
// after others stopped waiting.
// ---------------------------------------------------------------------------
constexpr uint32_t kDefaultFastTicks = 5000;   // 50 us of the 100 MHz counter
constexpr uint32_t kClaimSpan = 512;           // slots each workgroup of the slow path scans for claims
constexpr uint32_t kLastResortTicks = 2000000;  // 20 ms
// Tags run 1 .. 2^32 - 1, never 0. A call tags with e + 1 .. e + adv (adv:
// 1, or the grouped kernel's laps over the slots, at most kMaxLaps) and
// leaves the epoch at e + adv; once that passes kEpochLimit, every tagged
// word is cleared and the epoch restarts at 0, so the next call's tags stay
// below 2^32 and no word left 2^32 calls earlier can pass for its own.
constexpr uint32_t kMaxLaps = 256;  // above (2^32 / (128 x 128)) / kMaxPartials = 128
constexpr uint32_t kEpochLimit = 0xFFFFFFFFu - kMaxLaps;
static_assert(kMaxPartials / kSlotGroup < 63, "lane 63 of the group-slot poll reads the done word");

// workgroups of a grid of G whose exits count on line x
__device__ __forceinline__ uint32_t line_members(uint32_t G, uint32_t x) {
  return (G - x + kExitLines - 1) / kExitLines;
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent64(const uint32_t *p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent64(uint32_t *p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// a slot value that carries a maximum of the call tagged t
__device__ __forceinline__ bool holds_max(uint64_t v, uint32_t t) {
  return static_cast<uint32_t>(v >> 32) == t && static_cast<uint32_t>(v) < 0x80000000u;
}

// max |x| bit pattern over the whole input, by one workgroup (the last
// resort after the slow wait ran out)
template <int DT>
__device__ uint32_t input_max(const CastArgs &p) {
  const u32x4 *x = static_cast<const u32x4 *>(p.x);
  const uint64_t nvec = static_cast<uint64_t>(p.rows) * p.cols * RT<DT>::kElem / 16;
  uint32_t m = 0;
  for (uint64_t i = threadIdx.x; i < nvec; i += kThreads) {
    const u32x4 v = x[i];
    if (DT == kBF16) {
      ushort2_t h = {0, 0};
      h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2_t, v.x & 0x7FFF7FFFu));
      h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2_t, v.y & 0x7FFF7FFFu));
      h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2_t, v.z & 0x7FFF7FFFu));
      h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2_t, v.w & 0x7FFF7FFFu));
      m = max(m, static_cast<uint32_t>(max(h.x, h.y)) << 16);
    } else {
      m = max(m, max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu)));
    }
  }
  return m;
}

// max |x| bit pattern of the thread's pieces of tile (r0, c0) that lie in
// the input, read from memory (a claimed workgroup's tile), from clamped
// addresses as in rt_load: all eight pieces' loads in flight at once for
// BF16, four at a time for FP32 (registers: the slow path runs with the
// workgroup's own tiles held)
template <int DT>
__device__ uint32_t tile_part_max(const CastArgs &p, uint32_t r0, uint32_t c0) {
  constexpr int W = RT<DT>::kWords;
  constexpr int B = DT == kBF16 ? 8 : 4;
  const uint32_t col = c0 + 8 * (threadIdx.x & 15);
  const uint32_t rbase = r0 + 8 * (threadIdx.x >> 4);
  const uint32_t lcol = col < p.cols ? col : 0u;
  uint32_t m = 0;
#pragma unroll
  for (int h = 0; h < 8; h += B) {
    uint32_t w[B][W];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const uint32_t r = min(rbase + h + k, p.rows - 1);
      const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(p.x) +
                                                         (static_cast<uint64_t>(r) * p.cols + lcol) * RT<DT>::kElem);
#pragma unroll
      for (int q = 0; q < W / 4; ++q) {
        const u32x4 t = src[q];
        w[k][4 * q] = t.x;
        w[k][4 * q + 1] = t.y;
        w[k][4 * q + 2] = t.z;
        w[k][4 * q + 3] = t.w;
      }
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const uint32_t pm = piece_max<DT>(w[k]);
      m = max(m, col < p.cols && rbase + h + k < p.rows ? pm : 0u);
    }
  }
  return m;
}

// the thread's part of the maximum over the K tiles of workgroup c
template <int DT, int K>
__device__ uint32_t chunk_part_max(const CastArgs &p, uint32_t c, uint32_t G, uint32_t T, uint32_t tx_n,
                                   uint32_t ty_n) {
  uint32_t m = 0;
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    const uint32_t L = c + k * G;
    if (L >= T) break;
    uint32_t tx, ty;
    tile_xy(p, tile_index(p, L, T), tx_n, ty_n, tx, ty);
    m = max(m, tile_part_max<DT>(p, ty * kRT, tx * kRT));
  }
  return m;
}

// Wave 0's fast path: publish m, then wait at most fast_ticks for the group
// slots or the done word. Returns (in every lane) whether the grid's
// maximum, amax, was found. Every workgroup of the grid that is running
// marked its slot started within a few microseconds of its start, long
// before this one finished its loads; so once kGraceTicks have passed, a
// member slot without this call's tag, or a missing group slot whose
// first workgroup's slot has no tag, means workgroups that have not
// started because the grid is not all resident: then the wait stops at
// once, for the slow path.
constexpr uint32_t kGraceTicks = 1000;  // 10 us
__device__ __forceinline__ bool handoff_fast(uint32_t *ws, uint32_t m, uint32_t fast_ticks, uint32_t t, bool ok,
                                             uint32_t &amax) {
  const uint32_t G = gridDim.x, wg = blockIdx.x, lane = threadIdx.x;
  const uint64_t tagged = static_cast<uint64_t>(t) << 32;
  if (lane == 0) st_agent64(ws + kSlotWord + 2 * wg, tagged | m);
  const uint64_t t0 = wall_clock64();
  if (ok && wg % kSlotGroup == 0) {  // the group's first workgroup
    const uint32_t i = wg + lane;
    uint64_t v;
    for (;;) {
      v = i < G ? ld_agent64(ws + kSlotWord + 2 * i) : tagged;
      const uint64_t d = lane == 0 ? ld_agent64(ws + kDoneWord) : 0;
      if (__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(d >> 32)) == t) {  // the slow path's reducer is done
        amax = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(d));
        return true;
      }
      if (__all(holds_max(v, t))) break;
      const uint64_t dt = wall_clock64() - t0;
      if (dt > fast_ticks || (dt > kGraceTicks && __any(static_cast<uint32_t>(v >> 32) != t))) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    const uint32_t gm = wave_max(static_cast<uint32_t>(v));
    if (ok && lane == 0) st_agent64(ws + kGroupSlotWord + 2 * (wg / kSlotGroup), tagged | gm);
  }
  const uint32_t ngroups = (G + kSlotGroup - 1) / kSlotGroup;
  while (ok) {
    const uint64_t v = lane < ngroups ? ld_agent64(ws + kGroupSlotWord + 2 * lane)
                       : lane == 63   ? ld_agent64(ws + kDoneWord)
                                      : tagged;
    const bool mine = static_cast<uint32_t>(v >> 32) == t;
    const uint64_t b = __ballot(mine);
    if (b >> 63) {  // a workgroup of the slow path reduced every slot
      amax = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), 63));
      return true;
    }
    if ((b | (1ull << 63)) == ~0ull) {
      amax = wave_max(lane < ngroups ? static_cast<uint32_t>(v) : 0u);
      return true;
    }
    const uint64_t dt = wall_clock64() - t0;
    if (dt > fast_ticks) {
      ok = false;
    } else if (dt > kGraceTicks) {
      const bool missing = lane < ngroups && !mine;
      const uint64_t lv = missing ? ld_agent64(ws + kSlotWord + 2 * kSlotGroup * lane) : tagged;
      if (__any(static_cast<uint32_t>(lv >> 32) != t)) ok = false;
      else __builtin_amdgcn_s_sleep(2);
    } else {
      __builtin_amdgcn_s_sleep(2);
    }
  }
  return false;
}

// Wave 0: claim the next slot, from position `base` (below `limit`) of the
// scan order (start, start + 1, ... mod G), that no workgroup of this call
// has touched. Returns its workgroup, or G when none is left below limit or
// the reducer has already stored the done word. Four windows of 64 slots
// per step, their loads in flight together; base advances past the steps
// found without such a slot. Workgroups that scan the same windows would
// all try the same slot first: each tries the first candidate at or after
// its own lane `pick` of the first window at or after its own window
// pick >> 6 that has one. A compare-and-swap lost to another workgroup
// leaves the slot tagged t, so every step either claims a slot, removes a
// candidate or advances, and the scan ends.
__device__ uint32_t claim_next(uint32_t *ws, uint32_t t, uint32_t G, uint32_t limit, uint32_t start, uint32_t pick,
                               uint32_t &base) {
  const uint32_t lane = threadIdx.x;
  const uint64_t tagged = static_cast<uint64_t>(t) << 32;
  const uint32_t r = pick & 63;
  while (base < limit) {
    uint64_t v[4];
    uint32_t idx[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t pos = base + 64 * q + lane;
      idx[q] = start + pos >= G ? start + pos - G : start + pos;  // start < G and pos < G where loaded
      v[q] = pos < limit ? ld_agent64(ws + kSlotWord + 2 * idx[q]) : tagged;
    }
    const uint64_t done = lane == 0 ? ld_agent64(ws + kDoneWord) : 0;
    if (__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(done >> 32)) == t) return G;
    uint64_t cand[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) cand[q] = __ballot(static_cast<uint32_t>(v[q] >> 32) != t);
    int q = -1;
#pragma unroll
    for (int k = 3; k >= 0; --k) {  // the first window with a candidate, from window (pick >> 6) & 3 on
      const int w = (k + (pick >> 6)) & 3;
      if (cand[w] != 0) q = w;
    }
    if (q < 0) {
      base += 256;
      continue;
    }
    uint64_t c = 0;
    uint32_t i = 0, vlo = 0, vhi = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // keep the arrays in registers: no dynamic index
      if (w == q) {
        c = cand[w];
        i = idx[w];
        vlo = static_cast<uint32_t>(v[w]);
        vhi = static_cast<uint32_t>(v[w] >> 32);
      }
    }
    const uint64_t rot = r ? (c >> r) | (c << (64 - r)) : c;
    const uint32_t j = (static_cast<uint32_t>(__builtin_ctzll(rot)) + r) & 63;
    bool won = false;
    if (lane == j) {
      uint64_t expect = static_cast<uint64_t>(vhi) << 32 | vlo;
      won = __hip_atomic_compare_exchange_strong(reinterpret_cast<uint64_t *>(ws + kSlotWord + 2 * i), &expect,
                                                 tagged | kSlotClaimed, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    }
    if (__ballot(won) != 0) return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(i), j));
  }
  return G;
}

// Polls back off, up to about 2 us apart: hundreds of workgroups may poll
// one line at once.
__device__ __forceinline__ void poll_backoff(uint32_t &backoff) {
  for (uint32_t k = 0; k < backoff; ++k) __builtin_amdgcn_s_sleep(8);
  backoff = min(2 * backoff, 8u);
}

// Wave 0 of the reducer: wait at most `ticks` until every slot carries a
// maximum tagged t, and reduce them. Four windows of 64 slots per step,
// their loads in flight together; windows found complete are not read
// again.
__device__ bool wait_all_slots(const uint32_t *ws, uint32_t t, uint32_t G, uint32_t ticks, uint32_t &amax) {
  const uint32_t lane = threadIdx.x;
  const uint64_t tagged = static_cast<uint64_t>(t) << 32;
  const uint64_t t0 = wall_clock64();
  uint32_t from = 0, m = 0, backoff = 1;
  for (;;) {
    for (; from < G; from += 256) {
      uint64_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t i = from + 64 * q + lane;
        v[q] = i < G ? ld_agent64(ws + kSlotWord + 2 * i) : tagged;
      }
      bool all = true;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool h = holds_max(v[q], t);
        all = all && h;
        if (h) m = max(m, static_cast<uint32_t>(v[q]));  // max is idempotent: re-reads are harmless
      }
      if (!__all(all)) break;
    }
    if (from >= G) break;
    if (wall_clock64() - t0 > ticks) return false;
    poll_backoff(backoff);
  }
  amax = wave_max(m);
  return true;
}

// Wave 0 of every other workgroup of the slow path: wait at most `ticks`
// for the done word.
__device__ bool wait_done(const uint32_t *ws, uint32_t t, uint32_t ticks, uint32_t &amax) {
  const uint64_t t0 = wall_clock64();
  uint32_t backoff = 1;
  for (;;) {
    const uint64_t d = threadIdx.x == 0 ? ld_agent64(ws + kDoneWord) : 0;
    if (__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(d >> 32)) == t) {
      amax = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(d));
      return true;
    }
    if (wall_clock64() - t0 > ticks) return false;
    poll_backoff(backoff);
  }
}

// The count-out of a call that follows the workspace's epoch protocol
// (thread 0 of every workgroup, once it touches no tagged word any more):
// exit counters per line x = blockIdx.x mod kExitLines,
// then over the lines; the last workgroup of the grid advances the epoch
// by adv (and only it returns true). e, xb, xbt: the epoch and exit bases
// read at the start.
__device__ __forceinline__ bool epoch_exit(uint32_t *ws, uint32_t e, uint32_t adv, uint32_t xb, uint32_t xbt,
                                           uint32_t G, uint32_t x, uint32_t nx) {
  uint32_t *line = ws + kExitWord + 2 * kBarLine * x;
  const uint32_t old = __hip_atomic_fetch_add(line, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old - xb != line_members(G, x) - 1) return false;
  st_agent(line + kBarLine, old + 1);
  const uint32_t top = __hip_atomic_fetch_add(ws + kExitTopWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (top - xbt != nx - 1) return false;
  st_agent(ws + kExitTopBaseWord, top + 1);
  if (e + adv <= kEpochLimit) {
    st_agent(ws + kEpochWord, e + adv);
  } else {
    // about 4600 stores, once per 2^32 calls
    for (uint32_t i = kSlotWord; i < kEpochWord; ++i) st_agent(ws + i, 0u);
    st_agent64(ws + kDoneWord, 0u);
    st_agent64(ws + kReducerWord, 0u);
    for (uint32_t g = 0; g < kMaxGroups; ++g) st_agent64(ws + kGroupDoneWord + kBarLine * g, 0u);
    st_agent(ws + kEpochWord, 0u);
  }
  return true;
}

// The start of such a call (thread 0): the exit bases of the workgroup's
// line and over the lines, and whether the counters are in a state that
// some call left (else the workspace was not zero-filled, and only maxima
// computed by the workgroup itself are trusted).
__device__ __forceinline__ void epoch_bases(const uint32_t *ws, uint32_t G, uint32_t x, uint32_t nx, uint32_t &xb,
                                            uint32_t &xbt, bool &sane) {
  const uint32_t *line = ws + kExitWord + 2 * kBarLine * x;
  xb = ld_agent(line + kBarLine);
  xbt = ld_agent(ws + kExitTopBaseWord);
  sane = ld_agent(line) - xb < line_members(G, x) && ld_agent(ws + kExitTopWord) - xbt < nx;
}

// The thread's 8 row pieces of BF16 tile (r0, c0) loaded straight into LDS
// (no registers): piece k of thread t lands at tl[k][t], since one load of a
// wave writes its 64 lanes' 16 bytes in lane order from a wave-uniform base.
// The addresses are rt_load's, clamped in edge tiles.
__device__ __forceinline__ void rt_load_lds(const CastArgs &p, uint32_t r0, uint32_t c0, u32x4 (*tl)[kThreads]) {
  const uint32_t col = c0 + 8 * (threadIdx.x & 15);
  const uint32_t rbase = r0 + 8 * (threadIdx.x >> 4);
  const uint32_t lcol = col < p.cols ? col : 0u;
  const uint32_t wave0 = threadIdx.x & ~63u;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t r = min(rbase + k, p.rows - 1);
    const void *src = static_cast<const uint8_t *>(p.x) + (static_cast<uint64_t>(r) * p.cols + lcol) * 2;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(&tl[k][wave0]), 16, 0, 0);
  }
}

// K slots per workgroup; with KL = 1 the last one is held in LDS (32 KiB,
// BF16 only) and the others in registers, so that three workgroups fit on a
// CU where K register tiles would allow two.
template <int DT, bool B2D, bool SR, int K, int KL = 0>
__global__ __launch_bounds__(kThreads, 2) void k_cast_rt_resident(CastArgs p, uint32_t *ws, uint32_t fast_ticks) {
  constexpr int W = RT<DT>::kWords;
  constexpr int KR = K - KL;  // register tiles
  static_assert(KL == 0 || DT == kBF16, "the LDS tile holds BF16 pieces");
  __shared__ RtLds sh;
  __shared__ u32x4 tl[KL ? 8 : 1][KL ? kThreads : 1];  // the LDS tile
  __shared__ uint32_t lds_ok, lds_amax, lds_step, lds_claim;
  __shared__ uint32_t lds_start[4];  // epoch, exit base of the group, exit base over the groups, sane
  if (p.noop != nullptr && *p.noop == 1.0f) return;

  const int tid = threadIdx.x;
  const uint32_t G = gridDim.x, wg = blockIdx.x;
  const uint32_t tx_n = (p.cols + kRT - 1) / kRT, ty_n = (p.rows + kRT - 1) / kRT;
  const uint32_t T = tx_n * ty_n;
  const uint32_t xg = wg % kExitLines;
  const uint32_t nxg = min(G, kExitLines);

  // this call's epoch, and the started mark: by the second wave, before
  // its tile loads, so that the grid's running workgroups are marked
  // within microseconds of their start (the other waves' loads go first)
  if (tid == 64) {
    const uint32_t e = ld_agent(ws + kEpochWord);
    st_agent64(ws + kSlotWord + 2 * wg, static_cast<uint64_t>(e + 1) << 32 | kSlotStarted);
    lds_start[0] = e;
  }

  // ---- load every tile, maximum over them ----
  // Tile coordinates before any load, so that the loads of successive
  // tiles are not separated by integer divisions. Swizzled scales keep the
  // row-major launch order, where slot k + 1 is slot k advanced by G tiles.
  uint32_t tile_x[K], tile_y[K];
  if (p.swizzled) {  // uniform
    const uint32_t dy = G / tx_n, dx = G - dy * tx_n;
    uint32_t ty = wg / tx_n, tx = wg - ty * tx_n;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      tile_x[k] = tx;
      tile_y[k] = ty;
      tx += dx;
      ty += dy;
      if (tx >= tx_n) {
        tx -= tx_n;
        ++ty;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) tile_xy(p, tile_index(p, min(wg + k * G, T - 1), T), tx_n, ty_n, tile_x[k], tile_y[k]);
  }
  uint32_t w[KR][8][W];
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    if (wg + k * G < T) rt_load<DT>(p, tile_y[k] * kRT, tile_x[k] * kRT, w[k]);
  }
  const bool lds_tile = KL && wg + (K - 1) * G < T;  // uniform
  if constexpr (KL != 0) {
    if (lds_tile) rt_load_lds(p, tile_y[K - 1] * kRT, tile_x[K - 1] * kRT, tl);
  }
  // the exit bases (issued after the tile loads, which need not wait for
  // them); a counter that is not in a state some call left means a
  // workspace that was not zero-filled: then only the whole-input maximum
  // is trusted
  if (tid == 0) {
    uint32_t xb, xbt;
    bool sane;
    epoch_bases(ws, G, xg, nxg, xb, xbt, sane);
    lds_start[1] = xb;
    lds_start[2] = xbt;
    lds_start[3] = sane ? 1u : 0u;
  }

  // while the loads are in flight the VALU is idle: clear the pieces
  // outside the input and take the 16x16 block maxima here rather than in
  // the encode
  uint32_t m[1] = {0};
  uint32_t m2d[B2D ? K : 1];
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    if (wg + k * G < T) {
      rt_clear_outside<DT>(p, tile_y[k] * kRT, tile_x[k] * kRT, w[k]);
      if (B2D) {
        m2d[k] = block2d_max<DT>(w[k]);
        m[0] = max(m[0], m2d[k]);
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) m[0] = max(m[0], piece_max<DT>(w[k][r]));
      }
    } else if (B2D) {
      m2d[k] = 0;
    }
  }
  if constexpr (KL != 0) {
    // the LDS tile's maximum, one piece at a time (its pieces outside the
    // input are clamped copies of input values: they leave the maximum, and
    // with 16-row / 16-column blocks every block outside the input, alone)
    if (B2D) m2d[K - 1] = 0;
    if (lds_tile) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads into LDS have landed
      uint32_t ml = 0;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const u32x4 v = tl[r][tid];
        const uint32_t piece[W] = {v.x, v.y, v.z, v.w};
        ml = max(ml, piece_max<DT>(piece));
      }
      if (B2D) {
        ml = max(ml, dpp_mov<kQuadXor1>(ml));
        ml = max(ml, swz_xor16(ml));
        m2d[K - 1] = ml;
      }
      m[0] = max(m[0], ml);
    }
  }
  workgroup_max(m, sh.red);  // its barrier also publishes lds_start

  // ---- publish, then wait for the grid ----
  const uint32_t t = lds_start[0] + 1;
  const bool ws_sane = lds_start[3] != 0;  // uniform
  if (tid < 64) {
    uint32_t amax = 0;
    const bool ok = handoff_fast(ws, m[0], fast_ticks, t, ws_sane, amax);
    if (tid == 0) {
      lds_ok = ok ? 1u : 0u;
      lds_amax = amax;
    }
  }
  lds_barrier();

  uint32_t a[1] = {lds_amax};
  if (lds_ok == 0) {  // uniform: the slow path
    if (ws_sane) {
      const uint64_t tagged = static_cast<uint64_t>(t) << 32;
      const uint64_t t0 = wall_clock64();
      // claims: within kClaimSpan slots of a spread start; the reducer then
      // scans every slot for what is left
      const uint32_t h = wg * 0x9E3779B9u;
      const uint32_t start = static_cast<uint32_t>((static_cast<uint64_t>(h) * G) >> 32);
      const uint32_t pick = (h >> 8) & 255;
      bool reducer = false;  // uniform
      for (int pass = 0; pass < 2; ++pass) {
        uint32_t base = 0;  // wave 0's scan position
        const uint32_t limit = pass == 0 ? min(G, kClaimSpan) : G;
        for (;;) {
          if (tid < 64) {
            const uint32_t c = claim_next(ws, t, G, limit, start, pick, base);
            if (tid == 0) lds_claim = c;
          }
          lds_barrier();
          const uint32_t c = lds_claim;  // uniform
          if (c >= G) break;
          uint32_t cm[1] = {chunk_part_max<DT, K>(p, c, G, T, tx_n, ty_n)};
          workgroup_max(cm, sh.red);
          if (tid == 0) st_agent64(ws + kSlotWord + 2 * c, tagged | cm[0]);
        }
        if (pass == 1) break;
        // elect the reducer: the first workgroup to tag the reducer word
        if (tid == 0) {
          uint64_t r = ld_agent64(ws + kReducerWord);
          bool won = false;
          if (static_cast<uint32_t>(r >> 32) != t)
            won = __hip_atomic_compare_exchange_strong(reinterpret_cast<uint64_t *>(ws + kReducerWord), &r,
                                                       tagged | wg, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
          lds_step = won ? 1u : 0u;
        }
        lds_barrier();
        reducer = lds_step != 0;
        if (!reducer) break;
      }
      if (tid < 64) {
        const uint64_t spent = wall_clock64() - t0;
        const uint32_t left = spent < kLastResortTicks ? kLastResortTicks - static_cast<uint32_t>(spent) : 0u;
        uint32_t am = 0;
        const bool ok = reducer ? wait_all_slots(ws, t, G, left, am) : wait_done(ws, t, left, am);
        if (tid == 0) {
          if (ok && reducer) st_agent64(ws + kDoneWord, tagged | am);
          lds_amax = ok ? am : 0xFFFFFFFFu;  // no maximum: the last resort below
        }
      }
      lds_barrier();
      a[0] = lds_amax;
    }
    if (!ws_sane || a[0] == 0xFFFFFFFFu) {  // uniform: the last resort
      a[0] = input_max<DT>(p);
      workgroup_max(a, sh.red);
    }
  }
  const float amax = __uint_as_float(a[0]);
  if (wg == 0 && tid == 0) {
    if (p.row_amax) *p.row_amax = amax;
    if (p.col_amax) *p.col_amax = amax;
  }

  // ---- count out: the last workgroup of the grid advances the epoch ----
  // The workgroup holds the call's maximum and touches no tagged word from
  // here on; a workgroup that has not started has not counted, so the epoch
  // only advances once every workgroup has read it. Counting here rather
  // than after the encode takes the counters' atomics off the kernel's tail.
  if (tid == 0) epoch_exit(ws, lds_start[0], 1, lds_start[1], lds_start[2], G, xg, nxg);

  // ---- encode from registers ----
  const bool ue = p.ue5m3 != 0;
  const float S_row = p.row_data != nullptr ? global_encode_scale(amax, ue) : 1.0f;
  const float S_col = p.col_data != nullptr ? global_encode_scale(amax, ue) : 1.0f;
  fill_multipliers(sh.mult, tid, S_row, S_col, ue);
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    if (wg + k * G < T) {
      if (k > 0) lds_barrier();  // the previous tile's LDS reads are done
      rt_encode<DT, B2D, SR, true>(p, tile_x[k], tile_y[k], w[k], S_row, S_col, ue, sh, B2D ? m2d[B2D ? k : 0] : 0u);
    }
  }
  if constexpr (KL != 0) {
    if (lds_tile) {  // into the registers of the tiles just encoded
      lds_barrier();
      uint32_t wl[8][W];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const u32x4 v = tl[r][tid];
        wl[r][0] = v.x;
        wl[r][1] = v.y;
        wl[r][2] = v.z;
        wl[r][3] = v.w;
      }
      const uint32_t ty = tile_y[K - 1], tx = tile_x[K - 1];
      rt_clear_outside<DT>(p, ty * kRT, tx * kRT, wl);
      rt_encode<DT, B2D, SR, true>(p, tx, ty, wl, S_row, S_col, ue, sh, B2D ? m2d[B2D ? K - 1 : 0] : 0u);
    }
  }

}

// The arguments of group g's own tensor: its rows of the input, its blocks
// of the concatenated outputs, its amax slots.
template <int DT>
__device__ __forceinline__ CastArgs group_args(const CastArgs &p, const GroupTable &t, uint32_t g) {
  CastArgs q = p;
  const uint64_t r0 = t.row_start[g];
  q.rows = t.row_start[g + 1] - t.row_start[g];
  q.x = static_cast<const uint8_t *>(p.x) + r0 * p.cols * RT<DT>::kElem;
  if (p.row_data != nullptr) {
    q.row_data = p.row_data + r0 * (p.cols >> 1);
    q.row_scales = p.row_scales + r0 * (p.cols >> 4);
  }
  if (p.col_data != nullptr) {
    q.col_data = p.col_data + p.cols * r0 / 2;
    q.col_scales = p.col_scales + p.cols * r0 / 16;
  }
  if (p.row_amax != nullptr) q.row_amax = p.row_amax + g;
  if (p.col_amax != nullptr) q.col_amax = p.col_amax + g;
  if (p.partials != nullptr) {  // the group's own maxima (a multiple of four, 16-byte aligned)
    q.partials = p.partials + t.part_start[g];
    q.npartials = t.part_start[g + 1] - t.part_start[g];
  }
  return q;
}

// One workgroup per 128 x 128 tile of some group; the tiles of group g are
// unit_start[g] .. unit_start[g + 1] - 1 (in tile_index order), in tile_xy
// order over that group's own tile grid.
template <int DT, bool B2D, bool SR>
__global__ __launch_bounds__(kThreads) void k_cast_rt_grouped(CastArgs p, GroupTable t) {
  const uint32_t u = tile_index(p, blockIdx.x, gridDim.x);
  const uint32_t g = group_of(t, u);
  const uint32_t local = u - t.unit_start[g];
  const uint32_t tiles_x = (p.cols + kRT - 1) / kRT;
  const CastArgs q = group_args<DT>(p, t, g);
  uint32_t tx, ty;
  tile_xy(p, local, tiles_x, (q.rows + kRT - 1) / kRT, tx, ty);
  cast_rt_tile<DT, B2D, SR>(q, tx, ty);
}

template <int DT, bool SR, bool MFMA>
__global__ __launch_bounds__(kThreads) void k_cast_rht_grouped(CastArgs p, GroupTable t) {
  const uint32_t u = tile_index(p, blockIdx.x, gridDim.x);
  const uint32_t g = group_of(t, u);
  const uint32_t local = u - t.unit_start[g];
  const uint32_t tiles_x = (p.cols + kRT - 1) / kRT;
  const CastArgs q = group_args<DT>(p, t, g);
  uint32_t tx, ty;
  tile_xy(p, local, tiles_x, (q.rows + kRT - 1) / kRT, tx, ty);
  cast_rht_tile<DT, SR, MFMA>(q, tx, ty);
}

// ---------------------------------------------------------------------------
// Grouped quantize with a per-group amax in one launch. A group's cast needs
// that group's amax only, and a group's work is a run of consecutive
// workgroups, which start together: first the group's head, then one
// workgroup per tile. Each tile loads into registers and stores its
// maximum to its slot (workgroup i: slot i mod kMaxPartials, tagged with the
// call's first tag + i / kMaxPartials, its lap over the slots). The head
// gathers the group's slots, stores the group's maximum to the group's done
// slot and writes the amax; the tiles wait for that slot and encode from
// registers. The input is read once, and no two workgroups update one word
// (atomics on one line are serialized) other than the exit counters, which
// are spread over kExitLines lines. The head holds no tile, so gathering up
// to kMaxFusedGroupTiles slots at once costs the tiles no registers.
//
// Waits. The head started before its group's tiles (workgroups start in
// index order) and waits for nothing but their slots, at most lead_ticks; a
// slot still missing then, or overwritten by a workgroup of a later lap, it
// replaces by reading that tile's maximum from the input. So the head
// always publishes, and the tiles wait for it at most wait_ticks (then take
// the group's maximum from the input). With every group at most
// kMaxFusedGroupTiles tiles, a group fits on the GPU beside the groups
// before it that are still finishing. The epoch advances only when every
// workgroup has exited (the single-pass protocol), so no workgroup of a
// call can take the next call's tags.
// ---------------------------------------------------------------------------

// no maximum (a maximum is below 2^31)
constexpr uint32_t kNoMax = 0xFFFFFFFFu;

// max |x| bit pattern of the thread's share of tile (r0, c0), one 16-byte
// load at a time (few registers: the caller holds its own tile's)
template <int DT>
__device__ uint32_t tile_max_lean(const CastArgs &p, uint32_t r0, uint32_t c0) {
  constexpr uint32_t E = RT<DT>::kElem;
  const u32x4 *x = static_cast<const u32x4 *>(p.x);
  const uint32_t vpr = p.cols * E / 16;                       // 16-byte vectors per row
  const uint32_t v0 = c0 * E / 16, nv = min(kRT * E / 16, vpr - v0);  // the tile's, per row
  const uint32_t n = min(kRT, p.rows - r0) * nv;
  uint32_t m = 0;
#pragma unroll 1
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) {
    const uint32_t r = i / nv;
    const u32x4 v = x[static_cast<uint64_t>(r0 + r) * vpr + v0 + (i - r * nv)];
    if (DT == kBF16) {
      ushort2_t h = __builtin_bit_cast(ushort2_t, v.x & 0x7FFF7FFFu);
      h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2_t, v.y & 0x7FFF7FFFu));
      h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2_t, v.z & 0x7FFF7FFFu));
      h = __builtin_elementwise_max(h, __builtin_bit_cast(ushort2_t, v.w & 0x7FFF7FFFu));
      m = max(m, static_cast<uint32_t>(max(h.x, h.y)) << 16);
    } else {
      m = max(m, max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu)));
    }
  }
  return m;
}

// The head of group g: the group's maximum from the slots of its tiles,
// workgroups first + 1 .. first + ntiles (or, for slots missing after
// lead_ticks or taken by a later lap, from the tiles themselves).
template <int DT>
__device__ uint32_t gather_group(const CastArgs &q, const uint32_t *ws, uint32_t b, uint32_t laps, bool sane,
                                 uint32_t first, uint32_t ntiles, uint32_t lead_ticks, uint32_t *lds_direct,
                                 uint32_t &lds_ndirect, uint32_t &lds_m, uint32_t *red) {
  constexpr uint32_t kPolls = kMaxFusedGroupTiles / 64;  // slots per lane
  const int tid = threadIdx.x;
  if (tid < 64) {
    // lane l: the tiles l + 64 k (workgroups first + 1 + l + 64 k)
    uint32_t pending = 0, direct = 0, m = 0;
#pragma unroll
    for (uint32_t k = 0; k < kPolls; ++k)
      if (tid + 64 * k < ntiles) (sane ? pending : direct) |= 1u << k;  // no tag can be trusted: read every tile
    const uint64_t t0 = wall_clock64();
    while (__any(pending != 0)) {
      uint64_t v[kPolls];
#pragma unroll
      for (uint32_t k = 0; k < kPolls; ++k) {
        const uint32_t i = first + 1 + tid + 64 * k;
        v[k] = (pending >> k & 1u) ? ld_agent64(ws + kSlotWord + 2 * (i % kMaxPartials)) : 0;
      }
#pragma unroll
      for (uint32_t k = 0; k < kPolls; ++k) {
        if (!(pending >> k & 1u)) continue;
        const uint32_t i = first + 1 + tid + 64 * k;
        const uint32_t want = b + i / kMaxPartials, tag = static_cast<uint32_t>(v[k] >> 32);
        if (tag == want && static_cast<uint32_t>(v[k]) < 0x80000000u) {
          m = max(m, static_cast<uint32_t>(v[k]));
          pending &= ~(1u << k);
        } else if (tag > want && tag < b + laps) {  // a later lap's workgroup took the slot
          pending &= ~(1u << k);
          direct |= 1u << k;
        }
      }
      if (__any(pending != 0)) {
        if (wall_clock64() - t0 > lead_ticks) {
          direct |= pending;
          pending = 0;
        } else {
          __builtin_amdgcn_s_sleep(2);
        }
      }
    }
#pragma unroll
    for (uint32_t k = 0; k < kPolls; ++k) {
      if (direct >> k & 1u) lds_direct[atomicAdd(&lds_ndirect, 1u)] = tid + 64 * k;
    }
    m = wave_max(m);
    if (tid == 0) lds_m = m;
  }
  lds_barrier();
  uint32_t a[1] = {lds_m};
  const uint32_t nd = lds_ndirect;
  if (nd != 0) {  // uniform: the missing tiles' maxima from the input
    const uint32_t tiles_x = (q.cols + kRT - 1) / kRT, tiles_y = (q.rows + kRT - 1) / kRT;
    uint32_t dm = 0;
    for (uint32_t d = 0; d < nd; ++d) {
      uint32_t dx, dy;
      tile_xy(q, tile_index(q, lds_direct[d], ntiles), tiles_x, tiles_y, dx, dy);
      dm = max(dm, tile_max_lean<DT>(q, dy * kRT, dx * kRT));
    }
    uint32_t r[1] = {dm};
    workgroup_max(r, red);
    a[0] = max(a[0], r[0]);
  }
  return a[0];
}

template <int DT, bool B2D, bool SR>
__global__ __launch_bounds__(kThreads) void k_grouped_fused(CastArgs p, GroupTable t, uint32_t *ws,
                                                            uint32_t lead_ticks, uint32_t wait_ticks) {
  constexpr int W = RT<DT>::kWords;
  __shared__ RtLds sh;
  __shared__ uint32_t lds_start[4];  // epoch, exit base of the line, exit base over the lines, sane
  __shared__ uint32_t lds_amax, lds_ndirect;
  __shared__ uint32_t lds_direct[kMaxFusedGroupTiles];  // tiles whose maxima the head reads itself
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  const int tid = threadIdx.x;
  const uint32_t G = gridDim.x, wg = blockIdx.x;
  const uint32_t x = wg % kExitLines, nx = min(G, kExitLines);
  const uint32_t laps = (G + kMaxPartials - 1) / kMaxPartials;
  if (tid == 0) {
    uint32_t xb, xbt;
    bool sane;
    lds_start[0] = ld_agent(ws + kEpochWord);
    epoch_bases(ws, G, x, nx, xb, xbt, sane);
    lds_start[1] = xb;
    lds_start[2] = xbt;
    lds_start[3] = sane ? 1u : 0u;
    lds_ndirect = 0;
  }
  if (wg == 0) {  // empty groups: amax 0 and nothing else
    for (uint32_t g = tid; g < t.ngroups; g += kThreads) {
      if (t.row_start[g + 1] == t.row_start[g]) {
        if (p.row_amax) p.row_amax[g] = 0.0f;
        if (p.col_amax) p.col_amax[g] = 0.0f;
      }
    }
  }
  const uint32_t g = group_of(t, wg);
  const uint32_t first = t.unit_start[g];  // the group's head
  const uint32_t ntiles = t.unit_start[g + 1] - first - 1;
  const CastArgs q = group_args<DT>(p, t, g);
  uint32_t *done = ws + kGroupDoneWord + kBarLine * g;

  if (wg == first) {  // the head (uniform)
    lds_barrier();    // lds_start
    const uint32_t m = gather_group<DT>(q, ws, lds_start[0] + 1, laps, lds_start[3] != 0, first, ntiles, lead_ticks,
                                        lds_direct, lds_ndirect, lds_amax, sh.red);
    if (tid == 0) {
      st_agent64(done, static_cast<uint64_t>(lds_start[0] + 1) << 32 | m);
      if (q.row_amax) *q.row_amax = __uint_as_float(m);
      if (q.col_amax) *q.col_amax = __uint_as_float(m);
      epoch_exit(ws, lds_start[0], laps, lds_start[1], lds_start[2], G, x, nx);
    }
    return;
  }

  // a tile: inside a group tile_index gives each XCD a contiguous run of its
  // tiles (workgroup i runs on XCD i % 8, and local indices keep that map
  // one to one), so that neighbouring tiles' scale pieces merge in one L2
  const uint32_t tiles_x = (p.cols + kRT - 1) / kRT, tiles_y = (q.rows + kRT - 1) / kRT;
  uint32_t tx, ty;
  tile_xy(p, tile_index(p, wg - first - 1, ntiles), tiles_x, tiles_y, tx, ty);
  uint32_t w[8][W];
  rt_load<DT>(q, ty * kRT, tx * kRT, w);
  uint32_t a[1] = {0};
#pragma unroll
  for (int k = 0; k < 8; ++k) a[0] = max(a[0], piece_max<DT>(w[k]));
  workgroup_max(a, sh.red);  // its barrier also publishes lds_start
  const uint32_t b = lds_start[0] + 1;  // the call's first tag
  if (tid == 0) {
    st_agent64(ws + kSlotWord + 2 * (wg % kMaxPartials), static_cast<uint64_t>(b + wg / kMaxPartials) << 32 | a[0]);
    uint32_t am = kNoMax;
    if (lds_start[3] != 0) {
      const uint64_t t0 = wall_clock64();
      for (;;) {
        const uint64_t v = ld_agent64(done);
        if (static_cast<uint32_t>(v >> 32) == b && static_cast<uint32_t>(v) < 0x80000000u) {
          am = static_cast<uint32_t>(v);
          break;
        }
        if (wall_clock64() - t0 > wait_ticks) break;
        __builtin_amdgcn_s_sleep(4);
      }
    }
    lds_amax = am;
  }
  lds_barrier();
  a[0] = lds_amax;
  if (a[0] == kNoMax) {  // uniform: the group's maximum from its input
    a[0] = input_max<DT>(q);
    workgroup_max(a, sh.red);
  }
  // count out before the encode: no tagged word is touched from here on
  if (tid == 0) epoch_exit(ws, lds_start[0], laps, lds_start[1], lds_start[2], G, x, nx);
  const float amax = __uint_as_float(a[0]);
  const bool ue = q.ue5m3 != 0;
  const float S_row = q.row_data != nullptr ? global_encode_scale(amax, ue) : 1.0f;
  const float S_col = q.col_data != nullptr ? global_encode_scale(amax, ue) : 1.0f;
  fill_multipliers(sh.mult, tid, S_row, S_col, ue);
  rt_encode<DT, B2D, SR>(q, tx, ty, w, S_row, S_col, ue, sh);
}

template <int DT, bool B2D, bool SR>
hipError_t launch_rt(const CastArgs &a, hipStream_t s) {
  dim3 grid((a.cols + kRT - 1) / kRT, (a.rows + kRT - 1) / kRT);
  hipLaunchKernelGGL((k_cast_rt<DT, B2D, SR>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT, bool SR>
hipError_t launch_rht(const CastArgs &a, hipStream_t s) {
  dim3 grid((a.cols + kRT - 1) / kRT, (a.rows + kRT - 1) / kRT);
  if (DT == kBF16 && rht_cast_on_matrix_cores())
    hipLaunchKernelGGL((k_cast_rht<DT, SR, DT == kBF16>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_cast_rht<DT, SR, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const CastArgs &a, bool block_2d, bool rht, bool sr, hipStream_t s) {
  if (rht) return sr ? launch_rht<DT, true>(a, s) : launch_rht<DT, false>(a, s);
  if (block_2d) return sr ? launch_rt<DT, true, true>(a, s) : launch_rt<DT, true, false>(a, s);
  return sr ? launch_rt<DT, false, true>(a, s) : launch_rt<DT, false, false>(a, s);
}

template <int DT>
hipError_t launch_grouped_dt(const CastArgs &a, const GroupTable &t, bool block_2d, bool rht, bool sr, hipStream_t s) {
  const dim3 grid(t.unit_start[t.ngroups]), block(kThreads);
  if (rht) {
    const bool mfma = DT == kBF16 && rht_cast_on_matrix_cores();
    if (sr && mfma)
      hipLaunchKernelGGL((k_cast_rht_grouped<DT, true, DT == kBF16>), grid, block, 0, s, a, t);
    else if (sr)
      hipLaunchKernelGGL((k_cast_rht_grouped<DT, true, false>), grid, block, 0, s, a, t);
    else if (mfma)
      hipLaunchKernelGGL((k_cast_rht_grouped<DT, false, DT == kBF16>), grid, block, 0, s, a, t);
    else
      hipLaunchKernelGGL((k_cast_rht_grouped<DT, false, false>), grid, block, 0, s, a, t);
  } else if (block_2d) {
    if (sr)
      hipLaunchKernelGGL((k_cast_rt_grouped<DT, true, true>), grid, block, 0, s, a, t);
    else
      hipLaunchKernelGGL((k_cast_rt_grouped<DT, true, false>), grid, block, 0, s, a, t);
  } else {
    if (sr)
      hipLaunchKernelGGL((k_cast_rt_grouped<DT, false, true>), grid, block, 0, s, a, t);
    else
      hipLaunchKernelGGL((k_cast_rt_grouped<DT, false, false>), grid, block, 0, s, a, t);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cast_grouped(const CastArgs &a, const uint32_t *row_start, const uint32_t *part_start,
                               uint32_t ngroups, int dtype, bool block_2d, bool rht, bool sr, hipStream_t s) {
  GroupTable t{};
  t.ngroups = ngroups;
  const uint32_t tiles_x = (a.cols + kRT - 1) / kRT;
  for (uint32_t g = 0; g <= ngroups; ++g) {
    t.row_start[g] = row_start[g];
    t.part_start[g] = part_start ? part_start[g] : 0;
  }
  t.unit_start[0] = 0;
  for (uint32_t g = 0; g < ngroups; ++g)
    t.unit_start[g + 1] = t.unit_start[g] + (row_start[g + 1] - row_start[g] + kRT - 1) / kRT * tiles_x;
  if (t.unit_start[ngroups] == 0) return hipSuccess;
  return dtype == kBF16 ? launch_grouped_dt<kBF16>(a, t, block_2d, rht, sr, s)
                        : launch_grouped_dt<kFP32>(a, t, block_2d, rht, sr, s);
}

hipError_t launch_cast_rowscaled(const CastArgs &a, int dtype, bool sr, hipStream_t s) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  const dim3 grid((a.cols + kRT - 1) / kRT, (a.rows + kRT - 1) / kRT), block(kThreads);
  if (dtype == kBF16) {
    if (sr) hipLaunchKernelGGL((k_cast_rt_rowscaled<kBF16, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_cast_rt_rowscaled<kBF16, false>), grid, block, 0, s, a);
  } else {
    if (sr) hipLaunchKernelGGL((k_cast_rt_rowscaled<kFP32, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_cast_rt_rowscaled<kFP32, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_cast(const CastArgs &a, int dtype, bool block_2d, bool rht, bool sr, hipStream_t s) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  return dtype == kBF16 ? launch_dt<kBF16>(a, block_2d, rht, sr, s) : launch_dt<kFP32>(a, block_2d, rht, sr, s);
}

// ---- single-pass cast: plan and launch ----
namespace {

// Kernel variants: v = 1 .. 5 is K = v register tiles (32 VGPRs each for
// BF16; five take 217-227 VGPRs in all, no spills); kLdsVariant is four
// slots, three in registers (156-166 VGPRs) and one in LDS. BF16 only
// beyond one tile: an FP32 tile takes 64 VGPRs, and two per workgroup leave
// room for only two workgroups per CU, which holds no more tiles than one
// per workgroup at four per CU.
constexpr int kLdsVariant = 6;
constexpr int kVariants = 7;
constexpr int kMaxDevices = 64;
std::atomic<uint32_t> g_wait_ticks{0};
std::atomic<uint32_t> g_forced_variant{0};

template <int DT, bool B2D, bool SR>
const void *resident_kernel_v(int v) {
  switch (v) {
    case 1: return reinterpret_cast<const void *>(&k_cast_rt_resident<DT, B2D, SR, 1>);
  }
  if constexpr (DT == kBF16) {
    switch (v) {
      case 2: return reinterpret_cast<const void *>(&k_cast_rt_resident<DT, B2D, SR, 2>);
      case 3: return reinterpret_cast<const void *>(&k_cast_rt_resident<DT, B2D, SR, 3>);
      case 4: return reinterpret_cast<const void *>(&k_cast_rt_resident<DT, B2D, SR, 4>);
      case 5: return reinterpret_cast<const void *>(&k_cast_rt_resident<DT, B2D, SR, 5>);
      case kLdsVariant: return reinterpret_cast<const void *>(&k_cast_rt_resident<DT, B2D, SR, 4, 1>);
    }
  }
  return nullptr;
}

const void *resident_kernel_for(int dtype, bool b2d, bool sr, int v) {
  if (dtype == kBF16) {
    if (b2d) return sr ? resident_kernel_v<kBF16, true, true>(v) : resident_kernel_v<kBF16, true, false>(v);
    return sr ? resident_kernel_v<kBF16, false, true>(v) : resident_kernel_v<kBF16, false, false>(v);
  }
  if (b2d) return sr ? resident_kernel_v<kFP32, true, true>(v) : resident_kernel_v<kFP32, true, false>(v);
  return sr ? resident_kernel_v<kFP32, false, true>(v) : resident_kernel_v<kFP32, false, false>(v);
}

// Workgroups of one kernel that may run at once: the occupancy limit per CU,
// but at most kMaxResidentPerCu, times the CU count; cached per device, 0
// when the runtime cannot tell. Grids at the full occupancy limit (6
// workgroups per CU for the 1x16 kernel with one tile) were measured not to
// be resident all at once, so that the waits ran out; grids of 2 to 4 per CU
// were.
constexpr int kMaxResidentPerCu = 4;

// The device the stream's work runs on (the current device for the null
// stream), or -1.
int stream_device(hipStream_t s) {
  hipDevice_t dev = -1;
  if (hipStreamGetDevice(s, &dev) != hipSuccess) return -1;
  return dev >= 0 && dev < kMaxDevices ? static_cast<int>(dev) : -1;
}

// The occupancy limit comes from the runtime for the current device; the
// library's devices are assumed to be of one kind (they are on an MI355X
// node), and the CU count is the stream's device's own.
uint32_t resident_capacity(int dev, int dtype, bool b2d, bool sr, int v) {
  static std::atomic<int32_t> cache[kMaxDevices][2][2][2][kVariants];
  if (dev < 0 || dev >= kMaxDevices) return 0;
  std::atomic<int32_t> &slot = cache[dev][dtype][b2d][sr][v];
  int32_t c = slot.load(std::memory_order_relaxed);
  if (c == 0) {
    int per_cu = 0, cus = 0;
    const void *f = resident_kernel_for(dtype, b2d, sr, v);
    if (f == nullptr || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      per_cu = cus = 0;
    c = per_cu > 0 && cus > 0 ? std::min(per_cu, kMaxResidentPerCu) * cus : -1;
    slot.store(c, std::memory_order_relaxed);
  }
  return c > 0 ? static_cast<uint32_t>(c) : 0u;
}

// CU count of a device (0 when the runtime cannot tell)
uint32_t device_cus(int dev) {
  int cus = 0;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus > 0 ? static_cast<uint32_t>(cus) : 0u;
}

uint32_t round8(uint32_t g) { return (g + kGridGrain - 1) / kGridGrain * kGridGrain; }

template <int DT, bool B2D, bool SR>
hipError_t launch_resident_v(const CastArgs &a, uint32_t *ws, uint32_t G, int v, uint32_t ticks, hipStream_t s) {
  const dim3 grid(G), block(kThreads);
  if (v == 1) {
    hipLaunchKernelGGL((k_cast_rt_resident<DT, B2D, SR, 1>), grid, block, 0, s, a, ws, ticks);
    return hipGetLastError();
  }
  if constexpr (DT == kBF16) {
    switch (v) {
      case 2: hipLaunchKernelGGL((k_cast_rt_resident<DT, B2D, SR, 2>), grid, block, 0, s, a, ws, ticks); break;
      case 3: hipLaunchKernelGGL((k_cast_rt_resident<DT, B2D, SR, 3>), grid, block, 0, s, a, ws, ticks); break;
      case 4: hipLaunchKernelGGL((k_cast_rt_resident<DT, B2D, SR, 4>), grid, block, 0, s, a, ws, ticks); break;
      case 5: hipLaunchKernelGGL((k_cast_rt_resident<DT, B2D, SR, 5>), grid, block, 0, s, a, ws, ticks); break;
      case kLdsVariant:
        hipLaunchKernelGGL((k_cast_rt_resident<DT, B2D, SR, 4, 1>), grid, block, 0, s, a, ws, ticks);
        break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace

ResidentPlan resident_plan(int dtype, bool block_2d, bool sr, uint32_t rows, uint32_t cols, bool when_faster,
                           hipStream_t stream) {
  ResidentPlan none{0, 0};
  if (rows == 0 || cols == 0) return none;
  const int dev = stream_device(stream);
  if (dev < 0) return none;
  const uint32_t tiles = ((rows + kRT - 1) / kRT) * ((cols + kRT - 1) / kRT);
  // Stochastic rounding hashes every output byte; beyond two tiles per CU
  // the two-launch form measured faster with it (8192x5120 16x16: 56.4 vs
  // 58.3 us; 1x16: 61.7 vs 64.9 us), below it slower (2048x4096 16x16: 19.6
  // vs 17.6 us).
  if (when_faster && sr && tiles > 2 * device_cus(dev)) return none;
  // Variants in order of tiles per workgroup: one to three register tiles,
  // three plus one LDS tile (three workgroups per CU), four or five register
  // tiles (two per CU). Each takes as many workgroups as can be resident,
  // up to one per tile: with fewer, some CUs hold more tiles than others
  // (8192x4096 1x16 with 688 workgroups of three slots: 35.5 us; 768: the
  // CUs even).
  static constexpr int kOrder[] = {1, 2, 3, kLdsVariant, 4, 5};
  // A forced variant takes one workgroup per `slots` tiles, however many
  // that is (it may be more than can be resident at once).
  const int forced = static_cast<int>(g_forced_variant.load(std::memory_order_relaxed));
  if (forced != 0 && (dtype == kBF16 || forced == 1)) {
    const uint64_t slots = forced == kLdsVariant ? 4 : forced;
    const uint64_t G = round8(static_cast<uint32_t>((tiles + slots - 1) / slots));
    if (G <= kMaxPartials) return ResidentPlan{forced, static_cast<uint32_t>(G)};
  }
  for (int v : kOrder) {
    const int slots = v == kLdsVariant ? 4 : v;
    if (v > 1 && dtype != kBF16) break;
    const uint32_t cap = resident_capacity(dev, dtype, block_2d, sr, v) / kGridGrain * kGridGrain;
    const uint32_t G = std::min(cap, round8(tiles));
    if (G > 0 && G <= kMaxPartials && static_cast<uint64_t>(G) * slots >= tiles) return ResidentPlan{v, G};
  }
  return none;
}

hipError_t launch_cast_resident(const CastArgs &a, uint32_t *ws, int dtype, bool block_2d, bool sr,
                                const ResidentPlan &plan, hipStream_t s) {
  const uint32_t t = g_wait_ticks.load(std::memory_order_relaxed);
  const uint32_t ticks = t != 0 ? t : kDefaultFastTicks;
  const uint32_t G = plan.grid;
  const int v = plan.variant;
  if (dtype == kBF16) {
    if (block_2d) return sr ? launch_resident_v<kBF16, true, true>(a, ws, G, v, ticks, s)
                            : launch_resident_v<kBF16, true, false>(a, ws, G, v, ticks, s);
    return sr ? launch_resident_v<kBF16, false, true>(a, ws, G, v, ticks, s)
              : launch_resident_v<kBF16, false, false>(a, ws, G, v, ticks, s);
  }
  if (block_2d) return sr ? launch_resident_v<kFP32, true, true>(a, ws, G, v, ticks, s)
                          : launch_resident_v<kFP32, true, false>(a, ws, G, v, ticks, s);
  return sr ? launch_resident_v<kFP32, false, true>(a, ws, G, v, ticks, s)
            : launch_resident_v<kFP32, false, false>(a, ws, G, v, ticks, s);
}

hipError_t launch_grouped_fused(const CastArgs &a, const uint32_t *row_start, uint32_t ngroups, int dtype,
                                bool block_2d, bool sr, uint32_t *ws, hipStream_t s) {
  GroupTable t{};
  t.ngroups = ngroups;
  const uint32_t tiles_x = (a.cols + kRT - 1) / kRT;
  t.unit_start[0] = 0;
  for (uint32_t g = 0; g <= ngroups; ++g) t.row_start[g] = row_start[g];
  for (uint32_t g = 0; g < ngroups; ++g) {  // a head and the tiles of each non-empty group
    const uint32_t n = (row_start[g + 1] - row_start[g] + kRT - 1) / kRT * tiles_x;
    t.unit_start[g + 1] = t.unit_start[g] + (n != 0 ? 1 + n : 0);
  }
  if (t.unit_start[ngroups] == 0) return hipSuccess;
  // The head waits at most the fast bound for its group's slots (then
  // reads the missing tiles itself); the tiles wait for the head, which
  // always publishes, at most the last-resort time. The test hook sets both.
  const uint32_t tw = g_wait_ticks.load(std::memory_order_relaxed);
  const uint32_t lead = tw != 0 ? tw : kDefaultFastTicks, wait = tw != 0 ? tw : kLastResortTicks;
  const dim3 grid(t.unit_start[ngroups]), block(kThreads);
#define NVFP4_FUSED(D, B, R) hipLaunchKernelGGL((k_grouped_fused<D, B, R>), grid, block, 0, s, a, t, ws, lead, wait)
  if (dtype == kBF16) {
    if (block_2d) { if (sr) NVFP4_FUSED(kBF16, true, true); else NVFP4_FUSED(kBF16, true, false); }
    else { if (sr) NVFP4_FUSED(kBF16, false, true); else NVFP4_FUSED(kBF16, false, false); }
  } else {
    if (block_2d) { if (sr) NVFP4_FUSED(kFP32, true, true); else NVFP4_FUSED(kFP32, true, false); }
    else { if (sr) NVFP4_FUSED(kFP32, false, true); else NVFP4_FUSED(kFP32, false, false); }
  }
#undef NVFP4_FUSED
  return hipGetLastError();
}

void set_resident_wait_ticks(uint32_t ticks) { g_wait_ticks.store(ticks, std::memory_order_relaxed); }

bool set_resident_variant(uint32_t v) {
  if (v >= static_cast<uint32_t>(kVariants)) return false;
  g_forced_variant.store(v, std::memory_order_relaxed);
  return true;
}

}  // namespace nvfp4
