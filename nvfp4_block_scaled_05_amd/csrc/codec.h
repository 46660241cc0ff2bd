// Device-side NVFP4 codec helpers for gfx950 (wave64).
//
// Every floating-point step is one correctly rounded FP32 operation, in the
// order the NVFP4 two-level scaling defines it (global encode scale from
// the amax, E4M3 block scale relative to it, per-block multiplier, E2M1
// code), so that the results are reproducible bit for bit. The library is
// built with -ffp-contract=off, so no multiply-add is fused.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr float kFltMax = 3.40282346638528859812e+38f;
// Largest E2M1 magnitude times the largest block-scale magnitude: 6 * 448
// with E4M3 scales, 6 * 61440 with UE5M3 scales.
constexpr float kGlobalScaleNumerator = 2688.0f;
constexpr float kGlobalScaleNumeratorUe5m3 = 368640.0f;

// ---------------------------------------------------------------------------
// Two-level scaling ("Implement row-scaled NVFP4 fprop recipe", Greptile
// summary: FP8 block scales relative to a per-tensor or per-row FP32 amax,
// with a zero guard).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float global_encode_scale(float amax, bool ue5m3) {
  if (amax == 0.0f) return 1.0f;
  float s = (ue5m3 ? kGlobalScaleNumeratorUe5m3 : kGlobalScaleNumerator) / amax;  // IEEE division
  return fminf(s, kFltMax);  // an overflow to +inf clamps
}

// E4M3 (bias 7, max 448) of a non-negative value, nearest even, saturating.
// Branch-free: at and above 2^-6 the code is the binary32 pattern rounded
// to 3 mantissa bits (ties to even, by an integer add of 0x7FFFF plus the
// kept low bit; a carry bumps the exponent) and rebiased from 127 to 7;
// below 2^-6 it is the nearest-even multiple of 2^-9 (8 is the smallest
// normal, code 0x08); codes past 0x7E (448), +inf included, saturate.
__device__ __forceinline__ uint32_t e4m3_encode(float sd) {
  const uint32_t u = __float_as_uint(sd);
  const uint32_t normal = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
  const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(sd * 512.0f));
  return min(sd < 0.015625f ? sub : normal, 0x7Eu);
}

__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  uint32_t e = (code >> 3) & 0xFu;
  uint32_t m = code & 7u;
  if (e == 0) return static_cast<float>(m) * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// UE5M3 block scales: unsigned, 5 exponent bits (bias 15), 3 mantissa
// bits, subnormals m * 2^-17, exponent 31 reserved, so the largest value is
// 61440 (code 0xF7); nearest even, saturating. The format is named but not
// defined in "Fuse NVFP4 scale swizzling on SM120 and SM121" (Changes); this
// is the reading the library takes.
__device__ __forceinline__ uint32_t ue5m3_encode(float sd) {
  // as e4m3_encode: rounded binary32 pattern rebiased from 127 to 15 at and
  // above 2^-14, nearest-even multiples of 2^-17 below, saturation at 0xF7
  const uint32_t u = __float_as_uint(sd);
  const uint32_t normal = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (112u << 3);
  const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(sd * 131072.0f));
  return min(sd < 6.103515625e-05f ? sub : normal, 0xF7u);
}

__device__ __forceinline__ float ue5m3_decode(uint32_t code) {
  uint32_t e = (code >> 3) & 0x1Fu;
  uint32_t m = code & 7u;
  if (e == 0) return static_cast<float>(m) * 7.62939453125e-06f;  // m * 2^-17
  return __uint_as_float(((e + 112u) << 23) | (m << 20));
}

// The block-scale format of a call: E4M3 (default) or UE5M3 (uniform flag).
__device__ __forceinline__ uint32_t scale_encode(float sd, bool ue5m3) {
  return ue5m3 ? ue5m3_encode(sd) : e4m3_encode(sd);
}

__device__ __forceinline__ float scale_decode(uint32_t code, bool ue5m3) {
  return ue5m3 ? ue5m3_decode(code) : e4m3_decode(code);
}

struct BlockScale {
  uint32_t code;  // scale byte
  float mult;     // encode multiplier e
};

// fl(m / 6) for m >= 0 without a division: q0 = fl(m * fl(1/6)), then one
// Newton correction with the exact residual fma(-q0, 6, m). Compared with
// the correctly rounded quotient on every non-negative binary32 value, it
// differs only where the quotient is subnormal (m < 2^-122) and at +inf;
// those take the division.
__device__ __forceinline__ float div6(float m) {
  constexpr float r = 1.0f / 6.0f;
  const float q0 = m * r;
  float q = __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, m), r, q0);
  if (!(m >= 0x1p-122f && m <= kFltMax)) q = m / 6.0f;
  return q;
}

// sd = fl(fl(m / 6) * S); e = fl(S / value(s)), 0 when s == 0.
__device__ __forceinline__ BlockScale block_scale(float block_amax, float S, bool ue5m3) {
  float q = div6(block_amax);
  float sd = q * S;
  BlockScale b;
  b.code = scale_encode(sd, ue5m3);
  b.mult = b.code == 0 ? 0.0f : fminf(S / scale_decode(b.code, ue5m3), kFltMax);
  return b;
}

// ---------------------------------------------------------------------------
// E2M1 encoding of already scaled values v' (finite). Magnitudes
// {0, .5, 1, 1.5, 2, 3, 4, 6} are codes 0..7; bit 3 is the sign bit of v'.
// ---------------------------------------------------------------------------

// Nearest-even E2M1 codes of four pairs (a[2q], a[2q+1]) packed into one
// 32-bit word, pair q in byte q, first element in the low nibble, with the
// gfx950 conversion instruction at scale 1.0 (an exact no-op scale). The
// instruction rounds to nearest even, saturates beyond 6 and keeps the sign
// of zero and of values that round to zero (ties go to the code with a zero
// low bit); the GPU tests compare it with the CPU definition on every BF16
// value and on FP32 values around every decision point.
__device__ __forceinline__ uint32_t e2m1_rne_x8(const float *a) {
  // all four bytes are written, so any starting value will do; a[0]'s own
  // register saves an initialising move
  uint32_t w = __float_as_uint(a[0]);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a[0], a[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a[2], a[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a[4], a[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a[6], a[7], 1.0f, 3);
  return w;
}

// Nearest-even codes of the pair (a, b) written into byte `sel` (0..3) of w,
// a in the low nibble; the other bytes of w are kept. `sel` must fold to a
// constant (call it from unrolled loops).
__device__ __forceinline__ uint32_t e2m1_rne_pair_into(uint32_t w, float a, float b, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 3);
  }
}

// Stochastic rounding with 16 random bits r16: between grid neighbours
// lo <= |v| < hi (|v| < 6), round up iff r16 < 65536 * f, f = (|v| - lo) /
// (hi - lo); |v| >= 6 gives 6; the sign is kept. One random word r per byte:
// the even element takes r & 0xFFFF, the odd one r >> 16.
//
// This runs on the gfx950 SR conversion, whose rule was measured on this
// hardware (every binade from denormals up, zeros, infinities, signs,
// saturation, both slots, values at and next to every threshold): it divides
// its input by the scale operand (exactly, for a power of two), and with
// random operand R it rounds the pair's first element up iff
// floor(f * 2^22) + R >= 2^32, the second with R << 1 in place of R;
// |v| >= 6 (and +-inf) gives 6; signs are kept. Two exact adjustments turn
// that into the rule above:
//   1. The value is handed over as t = ceil(|v| * 2^23) with v's sign, and
//      scale 2^23, i.e. |v| rounded up to a multiple of 2^-23. Grid values
//      are multiples of 1/2, so this never passes hi (reaching hi exactly is
//      right too: then f > 1 - 2^-22 and every r16 rounds up). For |v| >= 1
//      it changes nothing, and below 1 it makes floor(f' * 2^22) equal to
//      ceil(f * 2^22). Above 2, f * 2^22 is an integer already.
//   2. R = (65535 - r16) * 2^16 + 65535 (first slot), and R such that R << 1
//      = (65535 - r16) * 2^16 + 65534 (second slot). Only R's top 22 bits
//      count, so both read ceil(f * 2^22) >= 64 * r16 + 1, which for an
//      integer r16 is f * 2^22 > 64 * r16, i.e. r16 < 65536 * f.
// The conversion runs twice per pair (one random operand per element) and
// only byte 0 of its result is used: its other bytes are left undefined.
// The GPU tests compare this with the CPU definition on every BF16 value and
// on values at every threshold.
constexpr float kSrScale = 8388608.0f;  // 2^23

__device__ __forceinline__ float sr_prepare(float v) {
  return __builtin_copysignf(__builtin_ceilf(fabsf(v) * kSrScale), v);
}

typedef float sr_float2 __attribute__((ext_vector_type(2)));

// Byte 0: the codes of (a, b) (prepared values) for random operand rnd.
__device__ __forceinline__ uint32_t cvt_sr(float a, float b, uint32_t rnd) {
  return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, sr_float2{a, b}, rnd, kSrScale, 0);
}

// Byte 0: stochastic codes of the pair (a, b) with random word r.
__device__ __forceinline__ uint32_t e2m1_sr_byte(float a, float b, uint32_t r) {
  const float pa = sr_prepare(a), pb = sr_prepare(b);
  const uint32_t nr = ~r;
  const uint32_t even = cvt_sr(pa, pb, (nr << 16) | 0xFFFFu);  // low nibble: a's code
  const uint32_t odd = cvt_sr(pa, pb, (nr >> 1) | 0x7FFFu);     // high nibble: b's code
  return (even & 0x0Fu) | (odd & ~0x0Fu);  // one v_bfi; bytes 1..3 are don't-care
}

// byte `sel` of w <- stochastic codes of the pair (a, b) with random word r;
// the other bytes of w are kept. `sel` must fold to a constant.
__device__ __forceinline__ uint32_t e2m1_sr_pair_into(uint32_t w, float a, float b, uint32_t r, int sel) {
  const uint32_t byte = e2m1_sr_byte(a, b, r);
  // v_perm: result byte k = w's byte k, or byte 0 of `byte` (selector 4) at k = sel
  const uint32_t selector = (0x03020100u & ~(0xFFu << (8 * sel))) | (0x04u << (8 * sel));
  return __builtin_amdgcn_perm(byte, w, selector);
}

// Stochastic codes of four pairs (a[2q], a[2q+1]) into byte q, with random
// word r[q] for pair q.
__device__ __forceinline__ uint32_t e2m1_sr_x8(const float *a, const uint32_t *r) {
  uint32_t b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) b[q] = e2m1_sr_byte(a[2 * q], a[2 * q + 1], r[q]);
  // bytes 0 of b0, b1 into bytes 0, 1; of b2, b3 into bytes 2, 3 (0x0C: zero)
  return __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u) | __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
}

// ---------------------------------------------------------------------------
// Counter-based random words: fmix32, the 32-bit finalizer of MurmurHash3
// (A. Appleby, public domain).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

__device__ __forceinline__ uint32_t sr_key(uint32_t seed, uint32_t orientation) {
  return fmix32(fmix32(seed) ^ (orientation + 1u));
}

// ---------------------------------------------------------------------------
// 16-point random Hadamard transform in registers: sign flips from the mask,
// an in-place fast Walsh-Hadamard transform (natural = Sylvester order), and
// the orthonormal factor 1/4 (exact).
// ---------------------------------------------------------------------------
// Unnormalized 16-point fast Walsh-Hadamard transform, in place.
__device__ __forceinline__ void fwht16(float (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// Two binary32 values rounded to BF16 (nearest, ties to even) and widened
// back; the pair becomes one v_cvt_pk_bf16_f32.
__device__ __forceinline__ void bf16_round_pair(float &a, float &b) {
  a = static_cast<float>(static_cast<__bf16>(a));
  b = static_cast<float>(static_cast<__bf16>(b));
}

__device__ __forceinline__ void bf16_round16(float (&v)[16]) {
#pragma unroll
  for (int k = 0; k < 16; k += 2) bf16_round_pair(v[k], v[k + 1]);
}

__device__ __forceinline__ void rht16(float (&v)[16], uint32_t sign_mask) {
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = __uint_as_float(__float_as_uint(v[k]) ^ (((sign_mask >> k) & 1u) << 31));
  fwht16(v);
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] *= 0.25f;
}

// ---------------------------------------------------------------------------
// GEMM-swizzled scale offset of scale (r, c) in an [n][k/16] scale matrix with
// scale_cols = k/16 (n % 128 == 0, scale_cols % 4 == 0): 128 x 4 tiles of 512
// bytes in row-major tile order; inside a tile (r%32)*16 + (r%128)/32*4 + c%4.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t swizzled_scale_offset(uint64_t r, uint64_t c, uint64_t scale_cols) {
  uint64_t tile = (r >> 7) * (scale_cols >> 2) + (c >> 2);
  return (tile << 9) + ((r & 31u) << 4) + (((r & 127u) >> 5) << 2) + (c & 3u);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), CTRL, 0xF, 0xF, false));
}

// quad_perm controls: lane ^ 1 and lane ^ 2 within each group of four
constexpr int kQuadXor1 = 0xB1;  // [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // [2,3,0,1]

// Lane s (0..3) of each group of four, broadcast to the group; s constant.
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x, int s) {
  switch (s) {
    case 0: return dpp_mov<0x00>(x);
    case 1: return dpp_mov<0x55>(x);
    case 2: return dpp_mov<0xAA>(x);
    default: return dpp_mov<0xFF>(x);
  }
}

// Maximum over the wave, uniform: DPP steps leave each row of 16 lanes with
// its maximum (quad xor 1, quad xor 2, half-row mirror, row mirror), then the
// four rows are read out as scalars.
// Workgroup barrier that orders LDS accesses only. __syncthreads() is also a
// workgroup-scope fence on global memory, which makes every wave wait until
// all of its global stores have completed: a barrier that follows output
// stores would then stall for their whole round trip to memory.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, dpp_mov<kQuadXor1>(v));
  v = max(v, dpp_mov<kQuadXor2>(v));
  v = max(v, dpp_mov<0x141>(v));
  v = max(v, dpp_mov<0x140>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace nvfp4
