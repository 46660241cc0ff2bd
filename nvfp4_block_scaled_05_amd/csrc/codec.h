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
// Stochastic rounding of runs of consecutive output bytes, the same rule as
// e2m1_sr_byte with fewer instructions per byte.
//
// Random words. For a byte b = b0 + i of a run whose first index b0 is a
// multiple of a power of two above i (so b = b0 ^ i and b >> 16 == b0 >> 16),
// fmix32's first step x ^ (x >> 16) of x = K ^ b splits into
//   (K ^ (K >> 16)) ^ (b0 ^ (b0 >> 16)) ^ i:
// a per-orientation part (sr_key_mix, uniform), a per-run part (sr_run_mix)
// and the constant i, one xor per byte.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t sr_key_mix(uint32_t key) { return key ^ (key >> 16); }
__device__ __forceinline__ uint32_t sr_run_mix(uint32_t b0) { return b0 ^ (b0 >> 16); }

// fmix32 after its first step (x already x ^ (x >> 16)), without the final
// xor-shift: fmix32 = h ^ (h >> 16) for the h returned.
__device__ __forceinline__ uint32_t fmix32_after_first(uint32_t x) {
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  return x * 0xC2B2AE35u;
}

// Both SR conversions of one pair (a, b), the even one into byte SEL of
// `even` and the odd one into byte SEL of `odd`, each keeping its other three
// bytes (checked on gfx950 with an in-bounds probe). The builtin does not tie
// its destination to the value it preserves, so the instructions are written
// out here, and with them the wait states the compiler would otherwise add:
// it never lets a VALU write a register that a byte-selecting conversion
// reads next, nor a VALU read a conversion's result right after it, so one
// s_nop stands on each side. Both outputs are early-clobber: the first
// conversion writes `even` while the second still reads the pair, so neither
// may share a register with an input (`even` starts as a copy of a[0]'s bits,
// which the allocator would otherwise merge with the pair).
#define NVFP4_CVT_SR_PAIR(OPSEL)                                                                   \
  asm("s_nop 0\n\t"                                                                               \
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %2, %3, %5" OPSEL "\n\t"                                  \
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %2, %4, %5" OPSEL "\n\t"                                  \
      "s_nop 0"                                                                                    \
      : "+&v"(even), "+&v"(odd)                                                                    \
      : "v"(pair), "v"(re), "v"(ro), "s"(scale))

template <int SEL>
__device__ __forceinline__ void cvt_sr_pair_into(uint32_t &even, uint32_t &odd, float a, float b, uint32_t re,
                                                 uint32_t ro) {
  const sr_float2 pair{a, b};
  const float scale = kSrScale;
  if constexpr (SEL == 0)
    NVFP4_CVT_SR_PAIR("");
  else if constexpr (SEL == 1)
    NVFP4_CVT_SR_PAIR(" op_sel:[0,0,1,0]");
  else if constexpr (SEL == 2)
    NVFP4_CVT_SR_PAIR(" op_sel:[0,0,0,1]");
  else
    NVFP4_CVT_SR_PAIR(" op_sel:[0,0,1,1]");
}
#undef NVFP4_CVT_SR_PAIR

// Stochastic codes of the N pairs (t[2i], t[2i+1]) of prepared values (as
// sr_prepare gives them), pair i into byte i of the result (N <= 4; higher
// bytes are undefined). Pair i is output byte b0 + I0 + i of its orientation;
// run_mix = sr_run_mix(b0), key_mix = sr_key_mix(K), and b0 must be a
// multiple of a power of two above I0 + N - 1. The even conversions of all
// pairs go into one word and the odd ones into another, each conversion
// filling one byte, and one bit-field merge takes the low nibbles from the
// first and the high nibbles from the second (see e2m1_sr_byte for the two
// random operands).
template <int N, int I0>
__device__ __forceinline__ uint32_t e2m1_sr_run(const float *t, uint32_t run_mix, uint32_t key_mix) {
  static_assert(N >= 1 && N <= 4, "a run fills at most one word");
  uint32_t even = 0, odd = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t h = fmix32_after_first(run_mix ^ key_mix ^ static_cast<uint32_t>(I0 + i));
    const uint32_t nr = ~(h ^ (h >> 16));  // 65535 - r16 in each half
    const uint32_t re = (nr << 16) | 0xFFFFu, ro = (nr >> 1) | 0x7FFFu;
    if (i == 0) {
      // the words start as values that die here (any start will do: every
      // used byte is written), which saves copying into them
      even = h;
      odd = nr;
    }
    if (i == 0)
      cvt_sr_pair_into<0>(even, odd, t[0], t[1], re, ro);
    else if (i == 1)
      cvt_sr_pair_into<1>(even, odd, t[2], t[3], re, ro);
    else if (i == 2)
      cvt_sr_pair_into<2>(even, odd, t[4], t[5], re, ro);
    else
      cvt_sr_pair_into<3>(even, odd, t[6], t[7], re, ro);
  }
  return odd ^ ((odd ^ even) & 0x0F0F0F0Fu);  // one v_bfi: even's low nibbles, odd's high ones
}

// sr_prepare(v * e) with one multiply fewer: ceil(|v| * e_fold) with v's sign,
// where e_fold = e * 2^23 (exact). Equal to sr_prepare(fl(v * e)) wherever
// neither product under- or overflows, which sr_fold_ok guarantees for every
// block of a tensor from its global encode scale S alone (pinned on the CPU
// by tests/test_sr_fold_cpu.py). The sign of fl(v * e) is v's (e >= 0).
__device__ __forceinline__ float sr_prepare_folded(float v, float e_fold) {
  return __builtin_copysignf(__builtin_ceilf(fabsf(v) * e_fold), v);
}

// Where the fold above is exact: log2 bounds lo <= log2(S) <= hi by scale
// format, input type and the factor c folded into the multiplier (4 on the
// RHT column side, 1 elsewhere). lo keeps every non-zero |v| * e above
// 2^-149 for the smallest non-zero input of the type (2^-133 BF16, 2^-149
// FP32; the RHT sums are multiples of it) and the largest scale; hi keeps
// e * 2^23 / c at most 2^126 for the smallest non-zero scale.
struct FoldRange {
  int ue5m3, fp32, c, lo, hi;
};
constexpr FoldRange kFoldRanges[] = {
    {0, 0, 1, -7, 94}, {0, 0, 4, -5, 94}, {0, 1, 1, 9, 94},  {0, 1, 4, 11, 94},
    {1, 0, 1, 0, 86},  {1, 0, 4, 2, 86},  {1, 1, 1, 16, 86}, {1, 1, 4, 18, 86},
};

__device__ __forceinline__ bool sr_fold_ok(float S, bool ue5m3, bool fp32, int c) {
  const FoldRange &r = kFoldRanges[(ue5m3 ? 4 : 0) + (fp32 ? 2 : 0) + (c == 4 ? 1 : 0)];
  return S >= __builtin_ldexpf(1.0f, r.lo) && S <= __builtin_ldexpf(1.0f, r.hi);
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

// The same unnormalized transform of one column of 16 BF16 values with the
// sign flips, on the matrix cores. H16 = H4 (x) H4 in Sylvester order:
// t[4r + m] = sum_j H4[r][j] * y_j[m], y_j[m] = sum_k H4[m][k] * s_{4j+k} x_{4j+k}.
// The 4x4 MFMAs work on 16 blocks of four lanes: lane (b, n) gives column n
// of B and gets column n of D, lane (b, m) gives row m of A (checked with an
// in-bounds probe). So with every lane giving its own column as B, each lane
// transforms its own vector:
//   stage 1, bf16 4x4x4: A = H4 diag(s_{4j..4j+3}) (exact in BF16), B = the
//     lane's rows 4j..4j+3 -> y_j (products exact, summed in FP32);
//   stage 2, f32 4x4x1, four accumulating steps j: A = column j of H4,
//     B = y_j[m] -> t[4r + m] in register r.
// Operands: x2[j] holds rows (4j, 4j+1) and (4j+2, 4j+3) of the column as
// BF16 pairs; a1[j] is the lane's row (lane % 4) of H4 diag(s) for group j as
// BF16 pairs, a2[j] = H4[lane % 4][j]. Both units keep denormals (probed).
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void fwht16_mfma(const uint32_t (&x2)[4][2], const uint32_t (&a1)[4][2],
                                            const float (&a2)[4], float (&t)[16]) {
  f32x4_t y[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x4_t a = __builtin_bit_cast(bf16x4_t, u32x2_t{a1[j][0], a1[j][1]});
    const bf16x4_t b = __builtin_bit_cast(bf16x4_t, u32x2_t{x2[j][0], x2[j][1]});
    y[j] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_4x4x1f32(a2[j], y[j][m], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) t[4 * r + m] = acc[r];
  }
}

// The lane's A operands of fwht16_mfma for a 16-bit sign mask.
__device__ __forceinline__ void fwht16_mfma_operands(uint32_t sign_mask, uint32_t (&a1)[4][2], float (&a2)[4]) {
  const uint32_t m = threadIdx.x & 3u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t h[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t neg = (__builtin_popcount(m & static_cast<uint32_t>(k)) & 1u) ^ ((sign_mask >> (4 * j + k)) & 1u);
      h[k] = neg ? 0xBF80u : 0x3F80u;  // BF16 -1 / +1
    }
    a1[j][0] = h[0] | (h[1] << 16);
    a1[j][1] = h[2] | (h[3] << 16);
    a2[j] = (__builtin_popcount(m & static_cast<uint32_t>(j)) & 1u) ? -1.0f : 1.0f;
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
// Every pattern used here (quad permutations, row mirrors) reads a valid lane
// for every lane, so bound_ctrl changes nothing; set, it lets the compiler
// fold the move into the instruction that consumes it.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, true));
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
