// Internal launch interface between the C ABI (validation, dispatch) and the
// gfx950 kernels. Every launcher assumes its arguments were validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "group.h"

namespace nvfp4 {

enum InType : int { kBF16 = 0, kFP32 = 1 };

// Per-workgroup maxima of the amax pass in the caller's workspace: two arrays
// of kMaxPartials words (the plain max|x|, then max|RHT(x)|), each holding a
// non-negative float's bit pattern. The amax pass writes a multiple of
// kPartialsGrain entries (workgroups without work write +0).
constexpr uint32_t kMaxPartials = 2048;

// Bit of the internal sign-mask word (above the 16 sign bits) that asks the
// RHT kernels to round the transformed values to BF16.
constexpr uint32_t kRhtBf16 = 1u << 16;
constexpr uint32_t kPartialsGrain = 4;

// Grid-wide handoff of the single-pass kernels, in the workspace after the
// two partials arrays (word offsets; a line is 128 bytes):
//   kSlotWord       one 64-bit slot per workgroup (at most kMaxPartials):
//                   tag << 32 | the maximum of the workgroup's tiles, or
//                   tag << 32 | kSlotStarted (the workgroup runs and will
//                   store its maximum) or kSlotClaimed (another workgroup
//                   took over the maximum of those tiles). The grouped
//                   kernel's workgroup i uses slot i mod kMaxPartials, tagged
//                   with the call's first tag + i / kMaxPartials;
//   kGroupSlotWord  one 64-bit slot per group of kSlotGroup workgroups, with
//                   the group's maximum, written by its first workgroup;
//   kEpochWord      the epoch e: a call tags its slots e + 1 (the grouped
//                   kernel e + 1 .. e + its laps over the slots) and its last
//                   workgroup to exit advances e past them;
//   kDoneWord       tag << 32 | the grid's maximum, stored by the reducer
//                   of the slow path;
//   kReducerWord    tag << 32 | the workgroup elected to reduce every slot
//                   in the slow path;
//   kExitTopWord, kExitTopBaseWord
//                   the exit counter over the kExitLines lines below and its
//                   value when the call began;
//   kExitWord       per line x (workgroups blockIdx.x mod kExitLines): the
//                   exit counter at kExitWord + 2 kBarLine x and its value
//                   when the call began one line later. Exits spread over
//                   many lines: atomics on one line are serialized;
//   kGroupDoneWord  per group g of the grouped kernel, one line each:
//                   tag << 32 | the group's maximum, stored by its leader.
// All of it must be zero before a workspace is first used; every call
// leaves the counters equal to their bases, ready for the next call.
constexpr uint32_t kBarLine = 32;  // words per line
constexpr uint32_t kExitLines = 64;
constexpr uint32_t kSlotGroup = 64;
constexpr uint32_t kSlotWord = 2 * kMaxPartials;
constexpr uint32_t kGroupSlotWord = kSlotWord + 2 * kMaxPartials;
constexpr uint32_t kEpochWord = kGroupSlotWord + 2 * (kMaxPartials / kSlotGroup);
constexpr uint32_t kDoneWord = kEpochWord + kBarLine;
constexpr uint32_t kReducerWord = kDoneWord + kBarLine;
constexpr uint32_t kExitTopWord = kReducerWord + kBarLine;
constexpr uint32_t kExitTopBaseWord = kExitTopWord + kBarLine;
constexpr uint32_t kExitWord = kExitTopBaseWord + kBarLine;
constexpr uint32_t kGroupDoneWord = kExitWord + 2 * kBarLine * kExitLines;
constexpr uint32_t kWorkspaceWords = 24576;
static_assert(kGroupDoneWord + kBarLine * kMaxGroups <= kWorkspaceWords, "handoff words fit the workspace");
// Low words of a slot that carry no maximum (a maximum is a non-negative
// float's bit pattern, below 2^31).
constexpr uint32_t kSlotStarted = 0xFFFFFFFEu;
constexpr uint32_t kSlotClaimed = 0xFFFFFFFFu;
static_assert(kWorkspaceWords * 4 == 98304, "workspace size is part of the ABI");
// Grids of the single-pass kernel are a multiple of the 8 XCDs.
constexpr uint32_t kGridGrain = 8;

// Arguments of the fused cast(-transpose) kernels. A direction whose data
// pointer is NULL is not written.
struct CastArgs {
  const void *x;
  uint32_t rows, cols;
  uint8_t *row_data, *row_scales;
  float *row_amax;
  uint8_t *col_data, *col_scales;
  float *col_amax;
  uint32_t swizzled;
  uint32_t sr_seed;
  uint32_t sign_mask;
  const float *noop;
  // NULL: the amax buffers hold the amax. Otherwise the workspace of the
  // amax pass with npartials (a multiple of kPartialsGrain) entries per
  // array: every workgroup reduces them and workgroup (0, 0) stores the
  // result to the amax buffers.
  const uint32_t *partials;
  uint32_t npartials;
  uint32_t ue5m3;  // block scales in UE5M3 rather than E4M3
};

// Arguments of the row-scaled kernels: the row-wise side (one amax per row)
// or the column-wise side (one amax per input column; data and scales are
// the transposed [cols][rows / 2] and [cols][rows / 16] arrays).
struct RowScaledArgs {
  const void *x;
  uint32_t rows, cols;
  uint8_t *data, *scales;  // NULL data: only compute the amax
  float *amax;             // [rows] (row-wise side) or [cols] (column-wise side)
  uint32_t sr_seed;
  const float *noop;
  uint32_t ue5m3;  // block scales in UE5M3 rather than E4M3
};

hipError_t launch_zero_amax(float *a, float *b, const float *noop, hipStream_t s);
// partials == NULL: atomic max into a and b (zeroed beforehand). Otherwise
// store per-workgroup maxima to partials (a workspace as described above) and
// their count to *npartials; a and b are not touched.
hipError_t launch_amax(const void *x, int dtype, uint64_t n, float *a, float *b, uint32_t *partials,
                       uint32_t *npartials, const float *noop, hipStream_t s);
hipError_t launch_rht_amax(const void *x, int dtype, uint32_t rows, uint32_t cols, uint32_t mask,
                           float *row_amax, float *col_amax, uint32_t *partials, uint32_t *npartials,
                           const float *noop, hipStream_t s);
hipError_t launch_cast(const CastArgs &a, int dtype, bool block_2d, bool rht, bool sr, hipStream_t s);
// Single-pass quantize with a per-tensor amax: one launch that loads every
// tile into registers, reduces the amax through the workspace's barrier words
// and encodes from registers (one tile per workgroup may be held in LDS).
// resident_plan gives the kernel variant and grid, or variant 0 when the
// tiles of this shape do not fit in the workgroups that can be resident at
// once, or (when_faster) where the two-launch form measured faster (the
// caller then takes the amax pass and launch_cast); launch_cast_resident
// launches that plan.
struct ResidentPlan {
  int variant;    // 0: the two-pass form; else the kernel variant
  uint32_t grid;  // workgroups
};
ResidentPlan resident_plan(int dtype, bool block_2d, bool sr, uint32_t rows, uint32_t cols, bool when_faster,
                           hipStream_t stream);
hipError_t launch_cast_resident(const CastArgs &a, uint32_t *workspace, int dtype, bool block_2d, bool sr,
                                const ResidentPlan &plan, hipStream_t s);
// Which unit runs the 16-point transform of BF16 input in the RHT kernels,
// process-wide: 0 (default) the matrix cores in the cast and the vector ALU
// in the amax pass (each measured faster there), 1 the vector ALU in both,
// 2 the matrix cores in both.
void set_rht_unit(uint32_t unit);
bool rht_cast_on_matrix_cores();
bool rht_amax_on_matrix_cores();
// Bound on the fast handoff wait, in ticks of the 100 MHz real-time counter;
// after it a workgroup claims the tiles of workgroups that have not started.
// 0 restores the default.
void set_resident_wait_ticks(uint32_t ticks);
// Test hook: 0 lets resident_plan choose; 1 .. 6 forces that variant (tiles
// per workgroup; 6: three register tiles and one LDS tile) with one
// workgroup per that many tiles, even beyond what can be resident at once.
// Returns false for other values.
bool set_resident_variant(uint32_t v);

// Grouped forms. row_start: host array of ngroups + 1 prefix sums of the
// groups' row counts (validated by the caller). `a` describes the whole
// input and the base pointers of the concatenated outputs; amax buffers hold
// one float per group.
// Amax with partials == NULL: atomic max into the zeroed slots. Otherwise
// per-workgroup maxima in the workspace, group g's at part_start[g] ..
// part_start[g + 1] - 1 (filled in here, host array of ngroups + 1), and the
// slots of empty groups set to +0; the cast then takes a->partials and
// part_start.
hipError_t launch_zero_amax_n(float *a, float *b, uint32_t n, const float *noop, hipStream_t s);
hipError_t launch_amax_grouped(const void *x, int dtype, uint32_t cols, const uint32_t *row_start, uint32_t ngroups,
                               float *a, float *b, uint32_t *partials, uint32_t *part_start, const float *noop,
                               hipStream_t s);
hipError_t launch_rht_amax_grouped(const void *x, int dtype, uint32_t cols, const uint32_t *row_start,
                                   uint32_t ngroups, uint32_t mask, float *row_amax, float *col_amax,
                                   uint32_t *partials, uint32_t *part_start, const float *noop, hipStream_t s);
hipError_t launch_cast_grouped(const CastArgs &a, const uint32_t *row_start, const uint32_t *part_start,
                               uint32_t ngroups, int dtype, bool block_2d, bool rht, bool sr, hipStream_t s);
// Grouped quantize with a per-group amax in one launch: each group's tiles
// hand their maxima over through the workspace (a slot per workgroup, a
// done slot per group) and encode from registers. Every group has at most
// kMaxFusedGroupTiles 128x128 tiles; a.partials is unused; the amax buffers
// are written.
constexpr uint32_t kMaxFusedGroupTiles = 512;
hipError_t launch_grouped_fused(const CastArgs &a, const uint32_t *row_start, uint32_t ngroups, int dtype,
                                bool block_2d, bool sr, uint32_t *ws, hipStream_t s);
// compute_amax: reduce each row's amax in the kernel (else read a.amax).
hipError_t launch_rowscaled(const RowScaledArgs &a, int dtype, bool sr, bool compute_amax, hipStream_t s);
// Per-row ([rows]) and per-column ([cols]) amax of the input, either may be
// NULL: one zeroing launch and one reduction that reads the input once.
hipError_t launch_dual_amax(const void *x, int dtype, uint32_t rows, uint32_t cols, float *row_amax, float *col_amax,
                            const float *noop, hipStream_t s);
// Row-scaled quantize by 128x128 register tiles: the row-wise side (if
// a.row_data) with 1x16 blocks scaled by a.row_amax[row], the column-wise side
// (if a.col_data) with 1x16 blocks down each column scaled by
// a.col_amax[column]; the amax arrays are read, compact scales only.
hipError_t launch_cast_rowscaled(const CastArgs &a, int dtype, bool sr, hipStream_t s);
// grouped form: row_start[0..ngroups] are the groups' first rows (stochastic
// rounding counts byte indices per group)
hipError_t launch_rowscaled_grouped(const RowScaledArgs &a, const uint32_t *row_start, uint32_t ngroups, int dtype,
                                    bool sr, bool compute_amax, hipStream_t s);
hipError_t launch_dequant(const uint8_t *data, const uint8_t *scales, const float *amax, uint32_t rows,
                          uint32_t cols, bool swizzled, bool row_scaled, bool ue5m3, float *y, hipStream_t s);
// zero-padded compact -> GEMM-swizzled scales; out holds swizzled_scales_bytes()
uint64_t swizzled_scales_bytes(uint64_t rows, uint64_t scale_cols);
hipError_t launch_swizzle(const uint8_t *compact, uint32_t rows, uint32_t scale_cols, uint8_t *out, hipStream_t s);
hipError_t launch_debug_e2m1(const float *v, const uint32_t *r, uint8_t *out, uint64_t n, bool sr, bool pairwise,
                             hipStream_t s);
hipError_t launch_debug_rht(const void *x, int dtype, uint32_t rows, uint32_t cols, uint32_t mask, float *t,
                            hipStream_t s);

}  // namespace nvfp4
