/*
 * NVFP4 quantization oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU definition of what the NVFP4 quantize
 * path computes. It exists to check the GPU library; nothing in the product
 * path may load it. Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it. It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * Sources (three TransformerEngine pull-request pages):
 *   [P1] "Write both NVFP4 amax buffers" (PR #3750)
 *   [P2] "Fuse NVFP4 scale swizzling on SM120 and SM121" (PR #3749)
 *   [P3] "Implement row-scaled NVFP4 fprop recipe" (PR #2931)
 * The pages describe the method in prose only; where they leave a step open
 * the reading used here is stated at the step and listed in the design notes.
 *
 * Arithmetic: every float operation below is one correctly rounded IEEE
 * binary32 operation (built with -O2 -ffp-contract=off, no fast-math, SSE
 * float on x86-64). Exceptions, stated where they occur: grid searches
 * compare in binary64 against exactly representable midpoints, and the
 * Hadamard sums are taken in binary64 and rounded once to binary32.
 *
 * Every function here has a pin in tests/ (library routine, closed form,
 * hand-worked example, invariant or brute force); none is "parity unpinned"
 * except where a function's comment says so.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BF16 0
#define ORACLE_FP32 1

/* The checker is built without OpenMP and runs single-threaded. For the
 * CPU-baseline timing the same source is also built with -fopenmp: then the
 * outer loops over rows, columns and blocks run in parallel. Each element's
 * arithmetic is the same either way; only the max reductions combine
 * partial maxima, and a maximum does not depend on that order. */
#ifdef _OPENMP
#include <omp.h>
#define ORACLE_PARALLEL_FOR _Pragma("omp parallel for schedule(static)")
#define ORACLE_PARALLEL_MAX_A _Pragma("omp parallel for schedule(static) reduction(max : a)")
#define ORACLE_PARALLEL_MAX_B _Pragma("omp parallel for schedule(static) reduction(max : b)")
#define ORACLE_PARALLEL_FOR_OR_NAN _Pragma("omp parallel for schedule(static) reduction(| : any_nan)")
#define ORACLE_PARALLEL_FOR_OR_TNAN _Pragma("omp parallel for schedule(static) reduction(| : t_nan)")
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
#define ORACLE_PARALLEL_FOR
#define ORACLE_PARALLEL_MAX_A
#define ORACLE_PARALLEL_MAX_B
#define ORACLE_PARALLEL_FOR_OR_NAN
#define ORACLE_PARALLEL_FOR_OR_TNAN
int oracle_num_threads(void) { return 1; }
#endif

/* ------------------------------------------------------------------ */
/* Input decoding.                                                     */
/* BF16 is the high half of a binary32 word, so widening is exact.     */
/* [P1] Changes: the quantizer takes BF16 and FP32 input.              */
/* ------------------------------------------------------------------ */
static float bits_to_float(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t float_to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

float oracle_load(const void *x, int dtype, int64_t index) {
  if (dtype == ORACLE_BF16) {
    const uint16_t *h = (const uint16_t *)x;
    return bits_to_float((uint32_t)h[index] << 16);
  }
  return ((const float *)x)[index];
}

/* ------------------------------------------------------------------ */
/* FP4 E2M1 (1 sign bit, 2 exponent bits, 1 mantissa bit).            */
/* Non-negative codes 0..7 have the magnitudes below; bit 3 is sign.   */
/* ------------------------------------------------------------------ */
static const double E2M1_MAGNITUDE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_value(uint8_t code) {
  double m = E2M1_MAGNITUDE[code & 7];
  return (code & 8) ? -m : m;
}

/* Round-to-nearest-even to E2M1 with saturation.
 * Nearest grid magnitude; on an exact midpoint the code with a zero
 * mantissa bit (an even code) wins; magnitudes beyond 6 become 6.
 * The sign bit copies the sign of the input, so -0 and negative values
 * that round to zero encode as 0x8. Inputs are finite. */
uint8_t oracle_e2m1_rne(float v) {
  double a = fabs((double)v);
  uint8_t code = 7; /* saturation when no midpoint is reached */
  for (int k = 0; k < 7; ++k) {
    /* midpoint of two grid values; exact in binary64 */
    double mid = 0.5 * (E2M1_MAGNITUDE[k] + E2M1_MAGNITUDE[k + 1]);
    if (a < mid) {
      code = (uint8_t)k;
      break;
    }
    if (a == mid) {
      code = (uint8_t)((k % 2 == 0) ? k : k + 1);
      break;
    }
  }
  return (uint8_t)(code | (signbit(v) ? 8 : 0));
}

/* Stochastic rounding to E2M1.
 * With A = |v|: A >= 6 gives 6. Otherwise lo is the largest grid value
 * <= A and hi the next one; the result is hi when r16 < frac * 65536 with
 * frac = (A - lo) / (hi - lo), else lo. So the probability of rounding up
 * is ceil(frac * 65536) / 65536, and grid values never move. The sign is
 * handled as in oracle_e2m1_rne. r16 is 16 random bits.
 * [P2] Changes and Validation list stochastic rounding as a quantizer
 * option without stating its rule; this rule is the reading used here. */
uint8_t oracle_e2m1_sr(float v, uint16_t r16) {
  double a = fabs((double)v);
  uint8_t code;
  if (a >= 6.0) {
    code = 7;
  } else {
    int k = 0;
    while (E2M1_MAGNITUDE[k + 1] <= a) ++k; /* grid[k] <= a < grid[k+1] */
    double frac = (a - E2M1_MAGNITUDE[k]) / (E2M1_MAGNITUDE[k + 1] - E2M1_MAGNITUDE[k]);
    code = ((double)r16 < frac * 65536.0) ? (uint8_t)(k + 1) : (uint8_t)k;
  }
  return (uint8_t)(code | (signbit(v) ? 8 : 0));
}

/* ------------------------------------------------------------------ */
/* FP8 E4M3 (OCP "E4M3FN": bias 7, no infinities, 0x7F is NaN).        */
/* [P2] Changes names E4M3 block scales; [P3] Greptile summary calls    */
/* them FP8 block scales.                                              */
/* ------------------------------------------------------------------ */
double oracle_e4m3_value(uint8_t code) {
  int e = (code >> 3) & 0xF;
  int m = code & 7;
  double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return (code & 0x80) ? -mag : mag;
}

/* Round-to-nearest-even to E4M3 with saturation to the largest finite
 * value 448 (code 0x7E); the argument is a non-negative block scale, so the
 * sign bit is always 0 and NaN is never produced. */
static double e4m3_table[0x7F];
static int e4m3_table_ready = 0;

uint8_t oracle_e4m3_rne_satfinite(float sd) {
  if (!e4m3_table_ready) { /* the decoded values of codes 0x00..0x7E, once */
    for (int k = 0; k < 0x7F; ++k) e4m3_table[k] = oracle_e4m3_value((uint8_t)k);
    e4m3_table_ready = 1;
  }
  double a = (double)sd;
  for (int k = 0; k < 0x7E; ++k) {
    double lo = e4m3_table[k];
    double hi = e4m3_table[k + 1];
    double mid = 0.5 * (lo + hi); /* exact in binary64 */
    if (a < mid) return (uint8_t)k;
    if (a == mid) return (uint8_t)((k % 2 == 0) ? k : k + 1);
  }
  return 0x7E;
}

/* ------------------------------------------------------------------ */
/* UE5M3 block scales (opt-in; "parity unpinned" against the pages).   */
/* [P2] Changes and Validation test "E4M3/UE5M3" block scales but do   */
/* not define UE5M3. Reading: an unsigned float, 5 exponent bits with  */
/* bias 15 and 3 mantissa bits; exponent 0 holds the subnormals        */
/* m * 2^-17; exponent 31 (codes 0xF8..0xFF) is reserved, as in the    */
/* IEEE-style 5-bit-exponent formats, so the largest finite value is   */
/* 1.875 * 2^15 = 61440 (code 0xF7). Encoding: nearest value, ties to  */
/* the even code, saturating to 61440.                                 */
/* ------------------------------------------------------------------ */
double oracle_ue5m3_value(uint8_t code) {
  int e = code >> 3;
  int m = code & 7;
  return (e == 0) ? ldexp((double)m, -17) : ldexp(1.0 + m / 8.0, e - 15);
}

static double ue5m3_table[0xF8];
static int ue5m3_table_ready = 0;

uint8_t oracle_ue5m3_rne_satfinite(float sd) {
  if (!ue5m3_table_ready) { /* the decoded values of codes 0x00..0xF7, once */
    for (int k = 0; k < 0xF8; ++k) ue5m3_table[k] = oracle_ue5m3_value((uint8_t)k);
    ue5m3_table_ready = 1;
  }
  double a = (double)sd;
  for (int k = 0; k < 0xF7; ++k) {
    double lo = ue5m3_table[k];
    double hi = ue5m3_table[k + 1];
    double mid = 0.5 * (lo + hi); /* exact in binary64 */
    if (a < mid) return (uint8_t)k;
    if (a == mid) return (uint8_t)((k % 2 == 0) ? k : k + 1);
  }
  return 0xF7;
}

/* Decoded value and nearest-even encoding of a block scale in format fmt
 * (0: E4M3, 1: UE5M3), and the largest finite value of that format. */
static double scale_value(uint8_t code, int fmt) {
  return fmt ? oracle_ue5m3_value(code) : oracle_e4m3_value(code);
}

static uint8_t scale_encode(float sd, int fmt) {
  return fmt ? oracle_ue5m3_rne_satfinite(sd) : oracle_e4m3_rne_satfinite(sd);
}

/* ------------------------------------------------------------------ */
/* Two-level scaling.                                                  */
/* [P3] Greptile summary: block-level FP8 scales are computed relative */
/* to a tensor-level (or row-level) FP32 amax, with zero-guard handling */
/* in the reference quantizer. The formula is not printed on the pages; */
/* the reading used: the global encode scale maps amax onto the largest */
/* product of the two formats, 6 (E2M1) * 448 (E4M3) = 2688; with      */
/* UE5M3 block scales 6 * 61440 = 368640.                              */
/* ------------------------------------------------------------------ */
float oracle_global_encode_scale_fmt(float amax, int fmt) {
  if (amax == 0.0f) return 1.0f; /* zero guard */
  float s = (fmt ? 368640.0f : 2688.0f) / amax;
  if (s > FLT_MAX) s = FLT_MAX; /* amax so small that the quotient overflows */
  return s;
}

float oracle_global_encode_scale(float amax) { return oracle_global_encode_scale_fmt(amax, 0); }

/* Block decode scale: sd = (m / 6) * S, stored in the scale format. */
uint8_t oracle_block_scale_fmt(float block_amax, float S, int fmt) {
  float q = block_amax / 6.0f;
  float sd = q * S;
  return scale_encode(sd, fmt);
}

uint8_t oracle_block_scale(float block_amax, float S) { return oracle_block_scale_fmt(block_amax, S, 0); }

/* Block encode multiplier: e = S / value(s), or 0 when the stored scale is
 * zero (every value of the block then encodes as a signed zero). */
float oracle_block_encode_multiplier_fmt(uint8_t s, float S, int fmt) {
  if (s == 0) return 0.0f;
  float sf = (float)scale_value(s, fmt);
  float e = S / sf;
  if (e > FLT_MAX) e = FLT_MAX;
  return e;
}

float oracle_block_encode_multiplier(uint8_t s, float S) { return oracle_block_encode_multiplier_fmt(s, S, 0); }

/* ------------------------------------------------------------------ */
/* Counter-based random bits for stochastic rounding.                  */
/* fmix32 is the 32-bit finalizer of MurmurHash3 (Austin Appleby,      */
/* public domain): two odd-constant multiplies between xor-shifts.     */
/* Key per direction: K_dir = fmix32(fmix32(seed) ^ (dir + 1)); the    */
/* word for output byte b of that direction is fmix32(K_dir ^ b); the  */
/* even element of the byte takes its low 16 bits, the odd element the */
/* high 16 bits. dir 0 = row-wise, 1 = column-wise.                    */
/* ------------------------------------------------------------------ */
uint32_t oracle_fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

uint32_t oracle_sr_word(uint32_t seed, int dir, uint32_t byte_index) {
  uint32_t key = oracle_fmix32(oracle_fmix32(seed) ^ (uint32_t)(dir + 1));
  return oracle_fmix32(key ^ byte_index);
}

/* ------------------------------------------------------------------ */
/* 16-point random Hadamard transform of one column group.             */
/* [P1] GPU-work table and review thread: the RHT quantizer applies a  */
/* random-sign Hadamard transform on the column-wise side and takes the */
/* column-wise amax after the transform. Reading: w_k = sigma_k * x_k  */
/* with sigma_k = -1 where bit k of the mask is set, then              */
/* t_r = (1/4) * sum_k H[r][k] w_k with the Sylvester Hadamard matrix   */
/* H[r][k] = (-1)^popcount(r & k); the sum is exact-ish in binary64 and */
/* rounded once to binary32.                                           */
/* ------------------------------------------------------------------ */
static int popcount4(unsigned v) {
  int c = 0;
  for (int i = 0; i < 4; ++i) c += (v >> i) & 1;
  return c;
}

void oracle_rht16(const float w_in[16], uint32_t sign_mask, float t_out[16]) {
  for (int r = 0; r < 16; ++r) {
    double acc = 0.0;
    for (int k = 0; k < 16; ++k) {
      double sigma = ((sign_mask >> k) & 1) ? -1.0 : 1.0;
      double h = (popcount4((unsigned)(r & k)) % 2) ? -1.0 : 1.0;
      acc += h * sigma * (double)w_in[k];
    }
    t_out[r] = (float)(0.25 * acc);
  }
}

/* ------------------------------------------------------------------ */
/* BF16 rounding of a binary32 value (round to nearest, ties to the     */
/* even significand), for the variant whose transformed values are      */
/* BF16. [P1] review thread: the post-RHT amaxes printed there (5.03125, */
/* 16.875) are BF16 values, which suggests BF16 transformed values; the */
/* page does not say so, so this is an opt-in reading. A BF16 value is  */
/* a binary32 value whose low 16 bits are zero; x lies between the two  */
/* such values lo (x's bits with the low half cleared) and the next one */
/* away from zero, and the low half of x's bits says which is nearer.   */
/* ------------------------------------------------------------------ */
float oracle_round_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint32_t lo = u & 0xFFFF0000u, rest = u & 0xFFFFu;
  uint32_t r;
  if (rest < 0x8000u) r = lo;
  else if (rest > 0x8000u) r = lo + 0x10000u;
  else r = (lo & 0x10000u) ? lo + 0x10000u : lo; /* tie: the even significand */
  float y;
  memcpy(&y, &r, 4);
  return y;
}

/* Column-wise RHT image of x: t[j][i] for column j, row i (rows % 16 == 0);
 * bf16 != 0 rounds every transformed value to BF16. */
void oracle_rht_colwise_ex(const void *x, int dtype, int64_t rows, int64_t cols, uint32_t sign_mask, int bf16,
                           float *t /* [cols][rows] */) {
  ORACLE_PARALLEL_FOR
  for (int64_t j = 0; j < cols; ++j) {
    float w[16], out[16];
    for (int64_t g = 0; g < rows / 16; ++g) {
      for (int k = 0; k < 16; ++k) w[k] = oracle_load(x, dtype, (g * 16 + k) * cols + j);
      oracle_rht16(w, sign_mask, out);
      for (int r = 0; r < 16; ++r) t[j * rows + g * 16 + r] = bf16 ? oracle_round_bf16(out[r]) : out[r];
    }
  }
}

void oracle_rht_colwise(const void *x, int dtype, int64_t rows, int64_t cols, uint32_t sign_mask,
                        float *t /* [cols][rows] */) {
  oracle_rht_colwise_ex(x, dtype, rows, cols, sign_mask, 0, t);
}

/* ------------------------------------------------------------------ */
/* Amax.                                                               */
/* [P1] Description/Changes: one reduction fills both the row-wise and  */
/* column-wise amax buffers with max|x|. [P3] Changes: the row-scaled   */
/* recipe keeps one amax per row. [P1] GPU-work table / review table:   */
/* the RHT path reduces max|x| for the row-wise side and max|RHT(x)|    */
/* for the column-wise side in one op.                                 */
/* mode 0: per tensor, mode 1: per row (and per column for the         */
/* column-wise side), mode 2: RHT pair, mode 3: RHT pair with BF16     */
/* transformed values.                                                 */
/* amax_row / amax_col may be NULL (that buffer is not requested).     */
/* ------------------------------------------------------------------ */
/* Non-finite inputs (the pages assume finite data; this is the library's
 * stated policy): an amax over values that include a NaN is NaN, and one
 * over values that include an infinity but no NaN is +inf. Written out here
 * rather than left to fmaxf, which would drop a NaN. */
static float amax_step(float a, float v) {
  const float m = fabsf(v);
  if (isnan(a) || isnan(m)) return NAN;
  return m > a ? m : a;
}

void oracle_compute_amax(const void *x, int dtype, int64_t rows, int64_t cols, int mode,
                         uint32_t sign_mask, float *amax_row, float *amax_col) {
  if (mode == 1) {
    ORACLE_PARALLEL_FOR
    for (int64_t i = 0; i < rows; ++i) {
      float a = 0.0f;
      for (int64_t j = 0; j < cols; ++j) a = amax_step(a, oracle_load(x, dtype, i * cols + j));
      if (amax_row) amax_row[i] = a;
    }
    /* the column-wise tensor's rows are the input's columns */
    if (amax_col) {
      ORACLE_PARALLEL_FOR
      for (int64_t j = 0; j < cols; ++j) {
        float a = 0.0f;
        for (int64_t i = 0; i < rows; ++i) a = amax_step(a, oracle_load(x, dtype, i * cols + j));
        amax_col[j] = a;
      }
    }
    return;
  }
  float a = 0.0f;
  int any_nan = 0;
  ORACLE_PARALLEL_MAX_A
  for (int64_t n = 0; n < rows * cols; ++n) a = fmaxf(a, fabsf(oracle_load(x, dtype, n)));
  ORACLE_PARALLEL_FOR_OR_NAN
  for (int64_t n = 0; n < rows * cols; ++n) any_nan |= isnan(oracle_load(x, dtype, n)) ? 1 : 0;
  if (any_nan) a = NAN;
  if (mode == 0) {
    if (amax_row) amax_row[0] = a;
    if (amax_col) amax_col[0] = a;
    return;
  }
  /* modes 2 and 3: RHT pair */
  if (amax_row) amax_row[0] = a;
  if (amax_col) {
    float *t = (float *)malloc(sizeof(float) * (size_t)(rows * cols));
    oracle_rht_colwise_ex(x, dtype, rows, cols, sign_mask, mode == 3, t);
    float b = 0.0f;
    int t_nan = 0;
    ORACLE_PARALLEL_MAX_B
    for (int64_t n = 0; n < rows * cols; ++n) b = fmaxf(b, fabsf(t[n]));
    ORACLE_PARALLEL_FOR_OR_TNAN
    for (int64_t n = 0; n < rows * cols; ++n) t_nan |= isnan(t[n]) ? 1 : 0;
    free(t);
    amax_col[0] = t_nan ? NAN : b;
  }
}

/* ------------------------------------------------------------------ */
/* Encoding one value with a block's multiplier: v' = v * e, then      */
/* E2M1 (RNE, or SR with the given 16 random bits).                    */
/* ------------------------------------------------------------------ */
static uint8_t encode_value(float v, float e, int stochastic, uint16_t r16) {
  float scaled = v * e;
  return stochastic ? oracle_e2m1_sr(scaled, r16) : oracle_e2m1_rne(scaled);
}

/* Encode one direction's 16-element block list into packed bytes.
 * vals: the n values of one output row of that direction (n % 16 == 0,
 * already with their block multipliers in e_per_block[n/16]).
 * Packing: element 2k in the low nibble of byte k, element 2k+1 in the
 * high nibble. byte_base is the index of the row's first byte in that
 * direction's data array (for the stochastic-rounding counter). */
static void encode_row(const float *vals, const float *e_per_block, int64_t n, int stochastic,
                       uint32_t seed, int dir, int64_t byte_base, uint8_t *out) {
  for (int64_t k = 0; k < n / 2; ++k) {
    uint32_t r = stochastic ? oracle_sr_word(seed, dir, (uint32_t)(byte_base + k)) : 0u;
    uint8_t lo = encode_value(vals[2 * k], e_per_block[(2 * k) / 16], stochastic, (uint16_t)(r & 0xFFFF));
    uint8_t hi = encode_value(vals[2 * k + 1], e_per_block[(2 * k + 1) / 16], stochastic, (uint16_t)(r >> 16));
    out[k] = (uint8_t)(lo | (hi << 4));
  }
}

/* ------------------------------------------------------------------ */
/* Quantize.                                                           */
/* Outputs (compact layouts; any direction may be NULL = not wanted):  */
/*   row_data   [rows][cols/2]   row_scales [rows][cols/16]            */
/*   col_data   [cols][rows/2]   col_scales [cols][rows/16]            */
/* The column-wise tensor is the transpose: its row j holds column j of */
/* x ([P1] Changes: one call writes both orientations).                */
/* Amax inputs: amax_row[0] (or amax_row[i] when row_scaled), and       */
/* amax_col[0] (or amax_col[j], one per input column, when row_scaled: */
/* the column-wise tensor is row-scaled along its own rows); each       */
/* direction's global scale comes from its own amax.                   */
/* block_2d: one scale per 16x16 block shared by both directions        */
/* ([P2] Changes: the 2D path); otherwise 1x16 blocks along each        */
/* direction's rows. rht: column-wise values are the RHT image (rht == */
/* 2: the image rounded to BF16).                                      */
/* Returns 0, or -1 on an unsupported combination.                     */
/* ------------------------------------------------------------------ */
int oracle_quantize_fmt(const void *x, int dtype, int64_t rows, int64_t cols, int block_2d, int row_scaled,
                        int rht, uint32_t sign_mask, int stochastic, uint32_t sr_seed, const float *amax_row,
                        const float *amax_col, uint8_t *row_data, uint8_t *row_scales, uint8_t *col_data,
                        uint8_t *col_scales, int scale_fmt) {
  int want_row = row_data != NULL;
  int want_col = col_data != NULL;
  if (cols % 16 != 0) return -1;
  if ((want_col || block_2d) && rows % 16 != 0) return -1;
  if (row_scaled && (block_2d || rht)) return -1;
  if (rht && block_2d) return -1;

  float *xv = (float *)malloc(sizeof(float) * (size_t)(rows * cols));
  ORACLE_PARALLEL_FOR
  for (int64_t n = 0; n < rows * cols; ++n) xv[n] = oracle_load(x, dtype, n);

  /* 2D: the amax of every 16x16 block; each direction turns it into a
   * scale with its own global encode scale (the two amaxes are equal when
   * they come from one reduction, so the scales are then shared). */
  float *m2d = NULL;
  if (block_2d) {
    int64_t br = rows / 16, bc = cols / 16;
    m2d = (float *)malloc(sizeof(float) * (size_t)(br * bc));
    ORACLE_PARALLEL_FOR
    for (int64_t bi = 0; bi < br; ++bi)
      for (int64_t bj = 0; bj < bc; ++bj) {
        float m = 0.0f;
        for (int di = 0; di < 16; ++di)
          for (int dj = 0; dj < 16; ++dj) m = fmaxf(m, fabsf(xv[(bi * 16 + di) * cols + bj * 16 + dj]));
        m2d[bi * bc + bj] = m;
      }
  }

  /* Row-wise direction: output row i is x[i][:]. */
  if (want_row) {
    ORACLE_PARALLEL_FOR
    for (int64_t i = 0; i < rows; ++i) {
      float *e = (float *)malloc(sizeof(float) * (size_t)(cols / 16));
      const float *v = xv + i * cols;
      float S = oracle_global_encode_scale_fmt(row_scaled ? amax_row[i] : amax_row[0], scale_fmt);
      for (int64_t b = 0; b < cols / 16; ++b) {
        float m = 0.0f;
        if (block_2d) {
          m = m2d[(i / 16) * (cols / 16) + b];
        } else {
          for (int k = 0; k < 16; ++k) m = fmaxf(m, fabsf(v[b * 16 + k]));
        }
        uint8_t s = oracle_block_scale_fmt(m, S, scale_fmt);
        e[b] = oracle_block_encode_multiplier_fmt(s, S, scale_fmt);
        row_scales[i * (cols / 16) + b] = s;
      }
      encode_row(v, e, cols, stochastic, sr_seed, 0, i * (cols / 2), row_data + i * (cols / 2));
      free(e);
    }
  }

  /* Column-wise direction: output row j is column j of x, or its RHT image. */
  if (want_col) {
    float *t = NULL;
    if (rht) {
      t = (float *)malloc(sizeof(float) * (size_t)(rows * cols));
      oracle_rht_colwise_ex(x, dtype, rows, cols, sign_mask, rht == 2, t);
    }
    ORACLE_PARALLEL_FOR
    for (int64_t j = 0; j < cols; ++j) {
      float *v = (float *)malloc(sizeof(float) * (size_t)rows);
      float *e = (float *)malloc(sizeof(float) * (size_t)(rows / 16));
      float S = oracle_global_encode_scale_fmt(row_scaled ? amax_col[j] : amax_col[0], scale_fmt);
      for (int64_t i = 0; i < rows; ++i) v[i] = rht ? t[j * rows + i] : xv[i * cols + j];
      for (int64_t b = 0; b < rows / 16; ++b) {
        float m = 0.0f;
        if (block_2d) {
          m = m2d[b * (cols / 16) + j / 16];
        } else {
          for (int k = 0; k < 16; ++k) m = fmaxf(m, fabsf(v[b * 16 + k]));
        }
        uint8_t s = oracle_block_scale_fmt(m, S, scale_fmt);
        e[b] = oracle_block_encode_multiplier_fmt(s, S, scale_fmt);
        col_scales[j * (rows / 16) + b] = s;
      }
      encode_row(v, e, rows, stochastic, sr_seed, 1, j * (rows / 2), col_data + j * (rows / 2));
      free(v);
      free(e);
    }
    free(t);
  }

  free(xv);
  free(m2d);
  return 0;
}

int oracle_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int block_2d, int row_scaled,
                    int rht, uint32_t sign_mask, int stochastic, uint32_t sr_seed, const float *amax_row,
                    const float *amax_col, uint8_t *row_data, uint8_t *row_scales, uint8_t *col_data,
                    uint8_t *col_scales) {
  return oracle_quantize_fmt(x, dtype, rows, cols, block_2d, row_scaled, rht, sign_mask, stochastic, sr_seed,
                             amax_row, amax_col, row_data, row_scales, col_data, col_scales, 0);
}

/* ------------------------------------------------------------------ */
/* GEMM-swizzled scale layout.                                         */
/* [P2] Description/Changes: scales may be written directly in the      */
/* cuBLAS GEMM layout when both dimensions are 128-aligned; four       */
/* aligned scales of one row then form one 32-bit word. Reading: the    */
/* cuBLAS block-scaling layout of 128-row x 4-scale tiles, 512 bytes    */
/* each, tiles in row-major order over the scale matrix, and inside a   */
/* tile row r, scale column c at (r%32)*16 + ((r%128)/32)*4 + c%4.      */
/* ------------------------------------------------------------------ */
int64_t oracle_swizzle_offset(int64_t r, int64_t c, int64_t scale_cols) {
  int64_t tile = (r / 128) * (scale_cols / 4) + c / 4;
  return tile * 512 + (r % 32) * 16 + ((r % 128) / 32) * 4 + (c % 4);
}

/* compact [rows][scale_cols] -> swizzled (rows % 128 == 0, scale_cols % 4 == 0). */
int oracle_swizzle_scales(const uint8_t *compact, int64_t rows, int64_t scale_cols, uint8_t *swizzled) {
  if (rows % 128 != 0 || scale_cols % 4 != 0) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < scale_cols; ++c)
      swizzled[oracle_swizzle_offset(r, c, scale_cols)] = compact[r * scale_cols + c];
  return 0;
}

/* [P2] Description: shapes whose scales do not fill whole tiles stay compact
 * from the quantize call, and a separate pass after it produces the GEMM
 * layout. Reading: that pass pads the scale matrix with zeros to whole
 * 128 x 4 tiles, [ceil(rows/128)*128][ceil(scale_cols/4)*4], and lays the
 * padded matrix out as above. swizzled holds that many bytes. */
void oracle_swizzle_scales_padded(const uint8_t *compact, int64_t rows, int64_t scale_cols, uint8_t *swizzled) {
  const int64_t prows = (rows + 127) / 128 * 128;
  const int64_t pcols = (scale_cols + 3) / 4 * 4;
  for (int64_t r = 0; r < prows; ++r)
    for (int64_t c = 0; c < pcols; ++c)
      swizzled[oracle_swizzle_offset(r, c, pcols)] = (r < rows && c < scale_cols) ? compact[r * scale_cols + c] : 0;
}

/* ------------------------------------------------------------------ */
/* Dequantize one direction (its own orientation, compact scales):      */
/* y = (value(code) * value(s)) / S, the product being exact; S is the  */
/* global encode scale of amax[0], or of amax[i] for row i when         */
/* row_scaled ([P3] Changes: dequantization picks the row's amax for    */
/* row-scaled tensors).                                                */
/* ------------------------------------------------------------------ */
void oracle_dequantize_fmt(const uint8_t *data, const uint8_t *scales, const float *amax, int row_scaled,
                           int64_t rows, int64_t cols, float *y, int scale_fmt) {
  for (int64_t i = 0; i < rows; ++i) {
    float S = oracle_global_encode_scale_fmt(row_scaled ? amax[i] : amax[0], scale_fmt);
    for (int64_t j = 0; j < cols; ++j) {
      uint8_t byte = data[i * (cols / 2) + j / 2];
      uint8_t code = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);
      float sf = (float)scale_value(scales[i * (cols / 16) + j / 16], scale_fmt);
      float p = (float)oracle_e2m1_value(code) * sf;
      y[i * cols + j] = p / S;
    }
  }
}

void oracle_dequantize(const uint8_t *data, const uint8_t *scales, const float *amax, int row_scaled,
                       int64_t rows, int64_t cols, float *y) {
  oracle_dequantize_fmt(data, scales, amax, row_scaled, rows, cols, y, 0);
}

/* Bit helpers exported for the tests' hand-worked checks. */
uint32_t oracle_float_bits(float f) { return float_to_bits(f); }

/* ------------------------------------------------------------------ */
/* Array forms of the scalar steps, so the tests can sweep many inputs  */
/* in one call. Each applies the scalar definition above elementwise.   */
/* ------------------------------------------------------------------ */
void oracle_e2m1_rne_array(const float *v, int64_t n, uint8_t *codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = oracle_e2m1_rne(v[i]);
}

void oracle_e2m1_sr_array(const float *v, const uint16_t *r16, int64_t n, uint8_t *codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = oracle_e2m1_sr(v[i], r16[i]);
}

void oracle_e4m3_array(const float *v, int64_t n, uint8_t *codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = oracle_e4m3_rne_satfinite(v[i]);
}

void oracle_ue5m3_array(const float *v, int64_t n, uint8_t *codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = oracle_ue5m3_rne_satfinite(v[i]);
}

void oracle_fmix32_array(const uint32_t *h, int64_t n, uint32_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_fmix32(h[i]);
}
