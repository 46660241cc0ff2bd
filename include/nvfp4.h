/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 quantize library.
 *
 * NVFP4 stores a tensor as 4-bit E2M1 values, packed two per byte, with one
 * FP8 E4M3 decode scale per 16 values and one FP32 amax per tensor (or per
 * row) from which a global encode scale is derived. One quantize call can
 * write both orientations of the tensor: the row-wise one (the tensor as
 * stored) and the column-wise one (its transpose), each with its own data,
 * scales and amax buffer.
 *
 * The operations follow three TransformerEngine pull-request pages:
 *   "Write both NVFP4 amax buffers" (PR #3750): one reduction fills both
 *     amax buffers after a zeroing pass clears both (Description, Changes);
 *   "Fuse NVFP4 scale swizzling on SM120 and SM121" (PR #3749): scales are
 *     written directly in the GEMM-swizzled layout when both dimensions
 *     are 128-aligned (Description, Changes);
 *   "Implement row-scaled NVFP4 fprop recipe" (PR #2931): one amax per row,
 *     row-wise output only, compact scales (Description, Changes, summary).
 *
 * Conventions for every call:
 *   - Tensors are row-major. Device buffers are owned by the caller; the
 *     library allocates no device memory and never synchronizes: work is
 *     queued on `stream` (a hipStream_t; NULL means the null stream) and
 *     runs asynchronously. Pointers are never stored, so calls can be
 *     captured in a HIP graph.
 *   - State kept between calls: on the device, only what a caller's
 *     workspace holds (nvfp4_config_t.workspace). On the host, process-wide
 *     caches of per-device launch facts (occupancy limits and compute-unit
 *     counts, read once from the runtime), the settings of the nvfp4_debug_set_*
 *     test hooks, and the per-thread text of
 *     nvfp4_last_error. None of it changes what a call computes.
 *   - Arguments are validated on the host before anything is queued. On a
 *     bad argument the call returns a non-zero status, queues nothing and
 *     writes nothing; nvfp4_last_error() then describes the problem.
 *   - A failure reported by the HIP runtime at launch returns NVFP4_ERR_HIP.
 *     Errors inside kernels are not detected.
 *   - Non-finite inputs (the method assumes finite data): every amax the
 *     library computes (per tensor, per row, per column, either of the RHT
 *     pair) is NaN when the values it covers include a NaN, and +inf when
 *     they include an infinity and no NaN (on the RHT column side, an
 *     infinity that meets another one of the opposite sign in a 16-point
 *     group gives NaN). FP4 data and scales derived from non-finite values
 *     are unspecified; every access stays inside the caller's buffers.
 *   - No call throws across the ABI.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,       /* rows/cols not supported by the requested layout */
  NVFP4_ERR_ALIGN = 3,       /* a pointer is not aligned as required */
  NVFP4_ERR_UNSUPPORTED = 4, /* an option or a combination of options is not supported */
  NVFP4_ERR_HIP = 5          /* the HIP runtime reported an error */
} nvfp4_status_t;

typedef enum {
  NVFP4_IN_BF16 = 0, /* input elements are bfloat16 */
  NVFP4_IN_FP32 = 1  /* input elements are float */
} nvfp4_dtype_t;

typedef enum {
  /* scales of one orientation [n][k] stored row-major as [n][k/16] bytes */
  NVFP4_SCALES_COMPACT = 0,
  /* the GEMM layout: the [n][k/16] scale matrix cut into tiles of 128 rows
   * by 4 scale columns, tiles in row-major order, 512 bytes each; inside a
   * tile, scale (r, c) sits at byte (r % 32) * 16 + (r % 128) / 32 * 4 + c % 4.
   * Needs n % 128 == 0 and k % 128 == 0 ("Fuse NVFP4 scale swizzling ...",
   * Description and Changes: the 128x128 alignment, and four aligned
   * scales written as one 32-bit word). */
  NVFP4_SCALES_GEMM_SWIZZLED = 1
} nvfp4_scale_layout_t;

typedef enum {
  NVFP4_SCALE_E4M3 = 0, /* OCP E4M3 (bias 7, max 448), round to nearest even, saturating */
  NVFP4_SCALE_UE5M3 = 1 /* named on "Fuse NVFP4 scale swizzling ..." (Changes, Validation)
                           but not defined there. Reading: unsigned, 5 exponent bits
                           (bias 15), 3 mantissa bits, subnormals m * 2^-17, exponent 31
                           reserved, max 61440 (code 0xF7); round to nearest even,
                           saturating. The global scale numerator becomes 6 * 61440. */
} nvfp4_scale_fmt_t;

typedef enum {
  /* the single-pass form where it fits and measured faster (nearest even;
   * stochastic rounding up to 2 x 128 x 128 elements per CU), else the
   * two-pass form */
  NVFP4_AMAX_PATH_AUTO = 0,
  /* always the amax pass and the cast kernel (two launches) */
  NVFP4_AMAX_PATH_TWO_PASS = 1,
  /* the single-pass form whenever every 128x128 tile fits in the
   * workgroups that can be resident at once (BF16: up to 3 tiles in
   * registers and one in LDS per workgroup, or 5 in registers; FP32: one;
   * at most 4 workgroups per CU), else the two-pass form */
  NVFP4_AMAX_PATH_SINGLE_PASS = 2
} nvfp4_amax_path_t;
/* The single-pass form is fastest with its whole grid on the GPU at once.
 * While kernels of other streams hold CUs, part of the grid may have to wait
 * for them; the workgroups already running then wait 50 us, take over the
 * amax of the tiles of the workgroups that have not started (reading those
 * tiles twice) and go on: the bytes are the same, the call slower. The
 * one-launch grouped form waits the same way, per group: after 50 us a
 * group's head reads the maxima of the group's tiles that have not started
 * from the input itself. Callers that overlap the quantize with
 * long-running kernels on other streams may prefer
 * NVFP4_AMAX_PATH_TWO_PASS. */

/* One orientation of an NVFP4 tensor. For the row-wise orientation of an
 * R x C input, n = R and k = C; for the column-wise one, n = C and k = R
 * (row j of the column-wise tensor is column j of the input).
 *   data   [n][k/2] bytes: element 2i in the low nibble of byte i, element
 *          2i+1 in the high nibble; E2M1 code = sign bit 3, magnitude
 *          index 0..7 for {0, 0.5, 1, 1.5, 2, 3, 4, 6}. 16-byte aligned.
 *   scales E4M3 bytes, compact [n][k/16] or GEMM-swizzled (n*k/16 bytes).
 *          4-byte aligned.
 *   amax   FP32: [1] per tensor, or [n] with row scaling. 4-byte aligned. */
typedef struct {
  uint8_t *data;
  uint8_t *scales;
  float *amax;
} nvfp4_out_t;

/* Options of a call. A NULL config means all fields zero except
 * compute_amax = 1. */
typedef struct {
  /* 0: 1x16 blocks along each orientation's rows. 1: 16x16 blocks with one
   * scale shared by both orientations ("Write both NVFP4 amax buffers",
   * Changes: 1D and 2D quantization). Needs R % 16 == 0. */
  uint32_t block_2d;
  /* nvfp4_scale_layout_t, for every orientation the call writes. */
  uint32_t scale_layout;
  /* nvfp4_scale_fmt_t. */
  uint32_t scale_fmt;
  /* 0: E2M1 round to nearest even. 1: stochastic rounding: value |v| between
   * grid neighbours lo < hi rounds up when r16 < 65536 * (|v| - lo) / (hi - lo),
   * with r16 = 16 bits of w = fmix32(K ^ b) (low half for the byte's even
   * element, high half for the odd one), b the byte's index in that
   * orientation's data array, K = fmix32(fmix32(sr_seed) ^ (1 + orientation)),
   * orientation 0 = row-wise, 1 = column-wise, and fmix32 the MurmurHash3
   * 32-bit finalizer. Scales always use nearest even. */
  uint32_t stochastic;
  uint32_t sr_seed;
  /* 1: one amax per row of the input ("Implement row-scaled NVFP4 fprop
   * recipe", Changes): 1x16 blocks, compact scales, no RHT; row->amax
   * holds R floats. The column-wise orientation, whose rows are the input's
   * columns, is scaled along its own rows the same way: col->amax holds C
   * floats, col->amax[j] = max_i |x[i][j]| (the quantizer prototype in the
   * review thread of "Write both NVFP4 amax buffers" sizes the column-wise
   * amax of a row-scaled tensor by the input's last dimension; how the
   * column-wise side uses it is on no page, so this reading is the plainest
   * one), and row->amax and col->amax must be distinct buffers. */
  uint32_t row_scaled;
  /* 1: the column-wise orientation encodes the 16-point random Hadamard
   * transform of each group of 16 consecutive rows of a column: with
   * w_k = sigma_k * x[16g + k][j], sigma_k = -1 where bit k of rht_sign_mask
   * is set, t_r = 1/4 * sum_k (-1)^popcount(r & k) * w_k takes position
   * 16g + r, and col->amax = max|t| ("Write both NVFP4 amax buffers", GPU
   * work per quantize call and review thread). The row-wise orientation and
   * row->amax stay plain. Needs block_2d == 0. */
  uint32_t rht;
  uint32_t rht_sign_mask; /* bits 0..15; higher bits are ignored */
  /* With rht == 1 only (else NVFP4_ERR_UNSUPPORTED). 1: every transformed
   * value t is rounded to BF16 (nearest, ties to even) before col->amax,
   * the column-wise block scales and the codes are taken from it. The
   * post-RHT amaxes printed in the review thread of "Write both NVFP4 amax
   * buffers" are BF16 values, which suggests BF16 transformed values; the
   * page does not say so, so this is an option and 0 (binary32 t) the
   * default. */
  uint32_t rht_bf16;
  /* nvfp4_quantize only. 1: zero the amax buffers and reduce them inside the
   * call. 0: use the amax buffers as they are (for instance after a MAX
   * all-reduce across devices). */
  uint32_t compute_amax;
  /* Device pointer or NULL. When *noop == 1.0f the call writes nothing, amax
   * buffers included ("Write both NVFP4 amax buffers", Changes). */
  const float *noop;
  /* nvfp4_quantize (and nvfp4_quantize_grouped) with compute_amax == 1 and
   * a per-tensor (per-group) amax only (not row_scaled): NULL, or device
   * memory of at least NVFP4_WORKSPACE_BYTES
   * bytes, 16-byte aligned, owned by the caller, zero-filled before its
   * first use. With a workspace the call takes one of two forms:
   *   single pass (one launch; not with the RHT; see amax_path): each
   *     workgroup loads its tiles into registers (one of them into LDS in
   *     one variant), publishes its maximum in the workspace, waits
   *     (bounded) until every workgroup has published, and encodes from
   *     registers, so the input is read once;
   *   two pass: the amax pass stores one maximum per workgroup there and
   *     the cast kernel finishes the reduction and writes the amax buffers
   *     (two launches, no zeroing pass, no atomics).
   * With NULL the amax buffers are zeroed and reduced with atomics (three
   * launches). The first 16 KiB of the workspace are scratch (contents on
   * entry do not matter). The rest holds the single-pass handoff: one
   * tagged slot per workgroup, one per group of a grouped call, an epoch
   * and exit counters, which every call leaves ready for the next; it must
   * be zero on first use and must not be
   * written by anything else. A workspace that breaks this is detected
   * (barring a chance of about one in 2^32) and every call on it then takes
   * a slow fallback that still gives the same bytes. Calls that share a
   * workspace must not run concurrently (queue them on one stream). Ignored
   * by the other calls and paths. */
  void *workspace;
  /* nvfp4_quantize only: NULL, or the address of two hipEvent_t handles
   * that the call records on its stream just before and just after the
   * launch of its cast kernel (on the row-scaled path: before its first
   * and after its last kernel, per-column amax pass included), so that
   * the kernel can be timed inside a whole call. Not recorded when the call
   * is rejected or the input is empty. */
  void *const *cast_events;
  /* nvfp4_amax_path_t; nvfp4_quantize or nvfp4_quantize_grouped with a
   * workspace, compute_amax == 1, a per-tensor (per-group) amax and no RHT
   * (ignored otherwise). Every path gives the same bytes. */
  uint32_t amax_path;
} nvfp4_config_t;

/* Bytes of the optional quantize workspace (nvfp4_config_t.workspace). */
#define NVFP4_WORKSPACE_BYTES 98304u

/* NVFP4_WORKSPACE_BYTES, for bindings that cannot read the macro. */
uint64_t nvfp4_workspace_bytes(void);

/*
 * Amax reduction ("Write both NVFP4 amax buffers", Description and Changes).
 * x: device, R x C elements of `dtype`, 16-byte aligned, C % 16 == 0,
 * R * C < 2^32.
 *   default:   both buffers are set to +0 and then to max|x| by one
 *              reduction; either pointer may be NULL; equal pointers are
 *              written once.
 *   row_scaled: row_amax[i] = max_j |x[i][j]| for each of R rows and
 *              col_amax[j] = max_i |x[i][j]| for each of C columns; either
 *              pointer may be NULL; equal pointers are rejected.
 *   rht:       row_amax = max|x|, col_amax = max|t| over the column-wise
 *              RHT image (needs R % 16 == 0), both from one read of x.
 * An empty input (R == 0 or C == 0) writes +0.
 */
nvfp4_status_t nvfp4_compute_amax(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t cols,
                                  float *row_amax, float *col_amax, const nvfp4_config_t *cfg,
                                  void *stream);

/*
 * Quantize x (R x C, device, 16-byte aligned, C % 16 == 0, R * C < 2^32)
 * into the requested orientations; row or col may be NULL, not both. The
 * column-wise orientation needs R % 16 == 0.
 *
 * Sources: "Write both NVFP4 amax buffers" (Description, Changes: one
 * quantize call writes the row-wise and the column-wise orientation, 1D and
 * 2D blocks, each from its own amax buffer filled by one reduction; GPU work
 * per quantize call: zeroing, amax, cast); "Fuse NVFP4 scale swizzling on
 * SM120 and SM121" (Description, Changes: E4M3 or UE5M3 block scales,
 * stochastic rounding, the RHT column-wise side, scales written in the GEMM
 * layout by the quantize kernel); "Implement row-scaled NVFP4 fprop recipe"
 * (Changes, Greptile summary: FP8 block scales relative to a per-tensor or
 * per-row amax, with a zero guard). The formula below is the reading taken
 * of that two-level scaling; the pages state no operation order.
 *
 * Per orientation: S = 2688 / amax (368640 / amax with UE5M3 scales; 1
 * when amax == 0, at most FLT_MAX); per block of 16 (or 16x16): m = max|v|,
 * scale s = E4M3(fl(m / 6) * S) (or UE5M3),
 * multiplier e = S / s (0 when s == 0, at most FLT_MAX), code =
 * E2M1(fl(v * e)), each step one correctly rounded FP32 operation.
 *
 * With compute_amax == 1 this queues the zeroing pass, the amax reduction
 * and the cast, or with a workspace the amax pass and the cast, which
 * finishes the reduction (row-scaled: one fused kernel for the row-wise
 * side; the column-wise side zeroes, reduces and encodes in three); with
 * compute_amax == 0 only the cast, which reads the amax buffers as given.
 * Either way the amax buffers hold the same values afterwards.
 */
nvfp4_status_t nvfp4_quantize(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t cols,
                              const nvfp4_out_t *row, const nvfp4_out_t *col,
                              const nvfp4_config_t *cfg, void *stream);

/*
 * Allocation-free nvfp4_quantize, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Same arguments, validation, results and errors as
 * nvfp4_quantize, except that config.workspace must be NULL
 * (NVFP4_ERR_UNSUPPORTED otherwise): the call uses a workspace of the
 * library's own instead, a static device array of NVFP4_WORKSPACE_BYTES
 * (96 KiB) that each GPU holds from its first such call until the process
 * ends. That size serves every input nvfp4_quantize accepts, so no input is
 * rejected for its size beyond nvfp4_quantize's own limits.
 *   - No device memory is allocated or freed, by the library or by any
 *     library it calls.
 *   - The first call on a device also queues, on `stream`, one small kernel
 *     that zero-fills that device's array (the workspace's first-use rule);
 *     later calls find it as the previous call left it.
 *   - Every call on one GPU shares that GPU's array: calls that may overlap
 *     on one GPU (different streams, or different host threads without
 *     ordering) race on it and can produce wrong results. Queue them on one
 *     stream.
 */
nvfp4_status_t nvfp4_quantize_noalloc(const void *x, nvfp4_dtype_t dtype, int64_t rows, int64_t cols,
                                      const nvfp4_out_t *row, const nvfp4_out_t *col,
                                      const nvfp4_config_t *cfg, void *stream);

/* Most groups of one nvfp4_quantize_grouped call. */
#define NVFP4_MAX_GROUPS 256

/*
 * Grouped quantize (the row-scaled page's grouped tensor storage: one tensor
 * per group with its own amax, "Implement row-scaled NVFP4 fprop recipe",
 * changed files). x is R x C with R = group_rows[0] + ... +
 * group_rows[G-1] (1 <= G <= NVFP4_MAX_GROUPS; group_rows is a host array;
 * a group may be empty). Group g is the slice of group_rows[g] rows starting
 * at row s_g = group_rows[0] + ... + group_rows[g-1]. Each group is
 * quantized exactly as nvfp4_quantize would quantize that slice on its own
 * with the same config (stochastic-rounding byte indices counted within
 * the group's own arrays), in at most three launches for all groups:
 *   row  data [R][C/2] and scales (compact [R][C/16], or each group's
 *        swizzled block at byte s_g * C/16), amax [G];
 *   col  group g's column-wise tensor [C][group_rows[g]]: data at byte
 *        C * s_g / 2, scales at byte C * s_g / 16 (compact or swizzled
 *        block), amax [G].
 * Each group_rows[g] must be a multiple of 16 for column-wise output, 16x16
 * blocks or the RHT, and of 128 for swizzled scales (C too). Row-scaled
 * configs (row-wise only here, 1x16, compact, no RHT) run as one fused launch:
 * row->amax then holds one entry per row, [R] (the same page's grouped
 * storage sizes it as the sum of the groups' rows), and nearest-even
 * results equal a single nvfp4_quantize over all rows; stochastic rounding
 * counts its byte indices within each group. Otherwise a computed amax
 * with a workspace takes one launch when no group has more than 512
 * 128x128 tiles, there is no RHT and amax_path is not
 * NVFP4_AMAX_PATH_TWO_PASS: each group's tiles load into registers, hand
 * their maxima to a head workgroup of the group through the workspace and
 * encode once it has published the group's amax (the input is read once).
 * Else it takes two launches (amax pass, cast), each group's workgroup
 * maxima in a range of the workspace that the group's cast tiles reduce
 * (the slots of empty groups are written +0); without a workspace the amax
 * is zeroed and reduced by atomic max (three launches). The same workspace
 * rule holds as for nvfp4_quantize: one call at a time per workspace, in
 * stream order.
 */
nvfp4_status_t nvfp4_quantize_grouped(const void *x, nvfp4_dtype_t dtype, int64_t num_groups,
                                      const int64_t *group_rows, int64_t cols, const nvfp4_out_t *row,
                                      const nvfp4_out_t *col, const nvfp4_config_t *cfg, void *stream);

/*
 * Dequantize one orientation q (n = rows, k = cols in q's own orientation,
 * k % 16 == 0) into y [rows][cols] FP32 (device, 4-byte aligned):
 * y = (value(code) * value(s)) / S, S from q->amax[0], or q->amax[i] for
 * row i when row_scaled ("Implement row-scaled NVFP4 fprop recipe",
 * Changes: the dequantize kernel selects the row's amax; a row-scaled
 * column-wise tensor passes its per-column amax, which is per row in its
 * own orientation). scale_layout and
 * scale_fmt (nvfp4_scale_fmt_t) are those the tensor was quantized with.
 */
nvfp4_status_t nvfp4_dequantize(const nvfp4_out_t *q, int64_t rows, int64_t cols, uint32_t scale_layout,
                                uint32_t scale_fmt, uint32_t row_scaled, float *y, void *stream);

/*
 * Compact -> GEMM-swizzled scales, for shapes with partial scale tiles
 * ("Fuse NVFP4 scale swizzling ...", Description: such shapes keep compact
 * scales from the quantize call and a separate pass lays them out for the
 * GEMM). compact: device, [rows][scale_cols] bytes (scale_cols = k/16 of the
 * orientation), 4-byte aligned. swizzled: device, 4-byte aligned,
 * nvfp4_swizzled_scales_bytes(rows, scale_cols) bytes: the scale matrix
 * padded with zeros to [ceil(rows/128)*128][ceil(scale_cols/4)*4] in the
 * layout of NVFP4_SCALES_GEMM_SWIZZLED. Every byte of it is written. For
 * rows % 128 == 0 and scale_cols % 4 == 0 the result equals the swizzled
 * scales that nvfp4_quantize writes directly. rows * scale_cols < 2^32.
 */
nvfp4_status_t nvfp4_swizzle_scales(const uint8_t *compact, int64_t rows, int64_t scale_cols, uint8_t *swizzled,
                                    void *stream);

/* Size in bytes of the zero-padded swizzled scales of nvfp4_swizzle_scales
 * (0 for a negative or empty shape, or 2^32 or more rows or scale columns). */
uint64_t nvfp4_swizzled_scales_bytes(int64_t rows, int64_t scale_cols);

/* Text for the last non-OK status returned on the calling thread ("" when
 * none). The pointer stays valid until the next call on that thread. */
const char *nvfp4_last_error(void);

/*
 * Test hook: the column-wise RHT image t [cols][rows] FP32 (device) of x,
 * computed by the same device code as the quantize kernels. R % 16 == 0.
 * sign_mask bits 0..15 are the signs; bit 16 set rounds every value to
 * BF16 as rht_bf16 does; higher bits are ignored.
 */
nvfp4_status_t nvfp4_debug_rht_colwise(const void *x, nvfp4_dtype_t dtype, int64_t rows,
                                       int64_t cols, uint32_t sign_mask, float *t, void *stream);

/* Flags of nvfp4_debug_e2m1_pack. */
#define NVFP4_DEBUG_SR 1u       /* stochastic rounding (else nearest even) */
#define NVFP4_DEBUG_PAIRWISE 2u /* the one-pair encoder (else the four-pair one) */

/*
 * Test hook: E2M1 codes of n pairs (v[2i], v[2i+1]) of already scaled FP32
 * values, packed into out[i] (first value in the low nibble), by the same
 * device encoders as the quantize kernels. With NVFP4_DEBUG_SR, r[i] is the
 * pair's random word as in nvfp4_config_t.stochastic (low half for v[2i],
 * high half for v[2i+1]); r may be NULL otherwise. v, r and out are device
 * buffers; v and r 4-byte aligned. Values must be finite.
 */
nvfp4_status_t nvfp4_debug_e2m1_pack(const float *v, const uint32_t *r, uint8_t *out, int64_t n, uint32_t flags,
                                     void *stream);

/*
 * Test hook: the bound, in ticks of the GPU's 100 MHz real-time counter, on
 * how long a workgroup of the single-pass quantize waits for the others to
 * publish their maxima before it takes the slow path: it claims the tiles of
 * workgroups that have not started, takes their maxima from memory, and
 * reduces every workgroup's maximum itself (same result, the claimed tiles
 * read twice). 0 restores the default (5,000 ticks, 50 us); 1 sends nearly
 * every workgroup down the slow path, so that tests can check it.
 * Process-wide; takes effect for launches queued afterwards.
 */
nvfp4_status_t nvfp4_debug_set_wait_ticks(uint32_t ticks);

/*
 * Test hook: the tiles of 128 x 128 elements that each workgroup of the
 * single-pass quantize holds. 0 (the default): the library's choice, which
 * keeps the whole grid resident. 1 .. 5: that many tiles in registers (BF16
 * input; FP32 takes 1 only); 6: three in registers and one in LDS (BF16).
 * A forced choice launches one workgroup per that many tiles, up to 2048
 * workgroups, even where they cannot all be resident at once (the handoff's
 * slow path then completes the call), so that tests can check that case;
 * beyond 2048 workgroups, or for a choice the input type does not have, the
 * library's choice stands. Process-wide; takes effect for calls made
 * afterwards. Other values: NVFP4_ERR_UNSUPPORTED.
 */
nvfp4_status_t nvfp4_debug_set_resident_variant(uint32_t tiles_per_workgroup);

/*
 * Test hook: which unit runs the 16-point transform of BF16 input in the RHT
 * amax pass and cast (nvfp4_quantize, nvfp4_quantize_grouped,
 * nvfp4_compute_amax): on the matrix cores, two stages of 4x4 MFMAs per
 * column; on the vector ALU, butterflies. 0 (the default): the matrix cores
 * in the cast and the vector ALU in the amax pass, each the faster there on
 * MI355X; 1: the vector ALU in both; 2: the matrix cores in both. Every form
 * sums in binary32 and stays within the RHT tolerances of the oracle; they
 * may differ from each other in the last bits. FP32 input always takes the
 * vector ALU. Process-wide; takes effect for launches queued afterwards.
 * Other values: NVFP4_ERR_UNSUPPORTED.
 */
nvfp4_status_t nvfp4_debug_set_rht_unit(uint32_t unit);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
