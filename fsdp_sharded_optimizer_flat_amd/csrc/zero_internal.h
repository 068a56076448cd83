// zero_internal.h -- declarations shared by the library's translation units
// (host plan builder, launchers, error state).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "zero.h"

namespace zero {

// The vector kernels give each lane one quad of 4 consecutive elements (8
// bytes of bf16, 16 bytes of fp32) and each wave64 one tile of 64 quads, so
// every wave-wide load or store covers one contiguous span.
constexpr int kQuad = 4;
constexpr int kWave = 64;
constexpr int kTile = kQuad * kWave;       // 256 elements per wave
constexpr int kBlock = 256;                // threads of the grid-stride / final kernels
constexpr int kOct = 8;                    // norm: 8 consecutive elements per lane
constexpr int kNormSpan = kOct * kWave;    // norm: one partial per 512-element tile
constexpr int kNormFanIn = 1024;           // partials one reduction workgroup combines
constexpr int64_t kMaxQuadsPerLaunch = int64_t(1) << 30;  // 32-bit dispatch grid size
// The staged step: from this many gradients on, reduce chunks of at most
// kStageMaxChunk elements (128 MB of fp32, half the memory-side cache) into
// a workspace and step each chunk from it.  Measured on MI355X: with bf16
// gradients the fused step is 0.6 points faster at N = 32, the staged one 5
// points faster at 64; with fp32 gradients (twice the bytes per rank) the
// fused step is 2 points faster at 24, the staged one 4-5 points faster at
// 28 and 32.
constexpr int32_t kStageMinRanks = 33;     // bf16 gradients
constexpr int32_t kStageMinRanksF32 = 25;  // fp32 gradients
inline int32_t stage_min_ranks(int32_t grad_dtype)
{
    return grad_dtype == ZERO_F32 ? kStageMinRanksF32 : kStageMinRanks;
}
constexpr int64_t kStageMaxChunk = int64_t(1) << 25;
constexpr int64_t kStageSlack = 4;  // elements to place a chunk at the state's 16-byte phase

// One contiguous run of elements whose gradient, state and output indices all
// advance together.  Offsets are element offsets into the respective buffers.
struct Segment {
    int64_t g_off, s_off, o_off, len;
};

// A piece of a segment handed to the kernels: either a vector body (len is a
// multiple of kQuad and every buffer is aligned for quad accesses at its
// start: 16 bytes for fp32, 8 bytes for bf16) or a scalar piece (any
// alignment).
struct Piece {
    int64_t g_off, s_off, o_off, len;
    bool vec;
    // Vector pieces: how many quads (0..15) before the piece the wave grid
    // starts, chosen so that the most streamed bytes begin each wave's span
    // at a 128-byte cache line (line_phase in layout.cpp).
    int32_t phase = 0;
};

// Validated step / norm request, pointers already checked.
struct Request {
    const zero_layout *layout;
    int32_t rank;
    const void *const *grads;
    int32_t n_grads;
    int32_t grad_dtype, grad_index;
    float divisor;
    int32_t state_index;  // for the norm: the g_out index space
    int32_t out_index;
    // base pointers used for alignment decisions (may be null)
    const void *state_ptrs[3];
    int n_state_ptrs;
    const void *out_ptr;
};

// Segments of the elements a (layout, rank, index spaces) selection touches,
// with contiguous neighbours merged.  Units [u0, u1) only (u1 < 0: to the
// last unit); with grads_from_range the gradient offsets count from the
// range's first element in the gradient's index space (offset[u0] for
// GLOBAL, local_offset[u0] for LOCAL): gradient buckets that hold only the
// range's units.
std::vector<Segment> build_segments(const zero_layout *L, int32_t rank, int32_t grad_index,
                                    int32_t state_index, int32_t out_index, int32_t u0 = 0,
                                    int32_t u1 = -1, bool grads_from_range = false);

// Start of unit u (u == n_units: the end) in an index space: offset_u for
// GLOBAL, local_offset_u for LOCAL.
int64_t unit_start(const zero_layout *L, int32_t u, int32_t index);

// Split segments into vector bodies and scalar heads / tails, given the
// actual buffer addresses (every gradient, every fp32 state buffer, output).
std::vector<Piece> build_pieces(const std::vector<Segment> &segs, const Request &rq);

// Number of elements the selection processes.
int64_t selected_elements(const zero_layout *L, int32_t rank);

// Upper bound on the norm's first-stage partial count for a selection.
int64_t norm_partials_bound(const zero_layout *L, int32_t rank);

// Layout sanity (magic, counts, internal consistency of the totals).
bool layout_ok(const zero_layout *L);

// One run of a reshard's copy plan: `len` elements from local index src_k of
// source rank src_rank's shard to local index dst_k of the destination shard;
// src_rank < 0 marks padding to zero-fill.
struct ReshardRun {
    int32_t src_rank;
    int64_t src_k, dst_k, len;
};

// Both layouts valid and holding the same number of parameter elements.
bool layouts_match(const zero_layout *from, const zero_layout *to);

// The copy plan that fills rank dst_rank's local shard of `to` from the local
// shards of `from`, in destination order, contiguous runs merged.
std::vector<ReshardRun> build_reshard_runs(const zero_layout *from, const zero_layout *to,
                                           int32_t dst_rank);

// Compute units of the current device (cached per device).  <= 0 on error.
int device_cu_count();

// Dynamic LDS bytes to reserve per one-wave workgroup whose kernel declares
// `static_lds` bytes of its own, so that at most `waves_per_cu` such
// workgroups are resident on a compute unit of the current device (0 = no
// cap).  The kernels never touch this reservation: it only bounds how many
// waves stream at once.  Cached per device.
size_t occupancy_cap_lds(int waves_per_cu, size_t static_lds);

// Target resident waves per CU of the streaming kernels (0 = no cap):
// zero_set_waves_per_cu, else ZERO_STEP_WAVES_PER_CU / ZERO_STEP1_WAVES_PER_CU
// / ZERO_NORM_WAVES_PER_CU, else the defaults measured on MI355X.
// runtime_kernel: the kernel takes the rank count as an argument (loads in
// batches of 128 bytes per lane) instead of having it compiled in.
int step_waves_per_cu(int n_grads, bool runtime_kernel, int grad_bytes);  // the fused step
int step1_waves_per_cu(bool staged_chunk);  // the step on one fp32 gradient
int norm_waves_per_cu(int n_grads, bool runtime_kernel,
                      int grad_bytes);  // the norm pass and the staged reduction

// Rank counts with a kernel of their own for bf16 gradients (fused step and
// norm pass): every N up to kMaxCompiledRanks, and 64.
constexpr int kMaxCompiledRanks = 32;
constexpr bool compiled_ranks(int n) { return (n >= 1 && n <= kMaxCompiledRanks) || n == 64; }

// Record a HIP error code for zero_last_hip_error(); returns ZERO_EHIP.
zero_status hip_fail(int hip_error, const char *where);

// Uniform per-launch constants of the fused step.
struct StepConsts {
    float b1, b2, omb1, omb2, bc2, eps, step_size, decay, clip;
    float divisor, inv_divisor;
    int32_t div_pow2;        // 1: multiply by inv_divisor (exactly the same value)
    const float *clip_dev;   // if set, the clip multiplier is read from device memory
};

bool is_pow2_float(float x, float *inv);

// The step's constants from the host scalars (sc may be null: divisor only).
StepConsts make_step_consts(const zero_adamw_scalars *sc, float divisor);

// Every check zero_step makes before device work (selection, enums, NULLs,
// alignment, aliasing of written buffers); shared by the host step.
zero_status validate_step(const zero_layout *L, int32_t rank, const void *const *grads,
                          int32_t n_grads, int32_t grad_dtype, int32_t grad_index, float divisor,
                          const float *master, const float *exp_avg, const float *exp_avg_sq,
                          int32_t state_index, const uint16_t *out, int32_t out_index,
                          const zero_adamw_scalars *sc);
// The same with the gradient buffers' extent given (elements): a step over a
// unit range reads gradient buckets that hold only the range.
zero_status validate_step_ext(const zero_layout *L, int32_t rank, const void *const *grads,
                              int32_t n_grads, int32_t grad_dtype, int32_t grad_index,
                              float divisor, const float *master, const float *exp_avg,
                              const float *exp_avg_sq, int32_t state_index, const uint16_t *out,
                              int32_t out_index, const zero_adamw_scalars *sc,
                              int64_t grad_extent);

// Launchers (defined in the .hip files).  Pointers are already offset to the
// piece's first element.  Return a hipError_t value.
// waves_per_cu (one fp32 gradient only): resident waves per CU; < 0 takes
// step1_waves_per_cu(false).
int launch_step_piece(const Piece &pc, const void *const *grads, int n_grads, int grad_dtype,
                      float *w, float *m, float *v, uint16_t *out, const StepConsts &c,
                      void *stream, int waves_per_cu = -1);
// The vector pieces pcs[0..count) in as few launches as possible (several
// pieces per launch).  Every base pointer must be quad-aligned (then every
// vector piece's offsets are whole quads).  hipErrorNotSupported when the
// rank count has no compiled kernel (the caller launches piece by piece).
int launch_step_batch(const Piece *pcs, int count, const void *const *grads, int n_grads,
                      int grad_dtype, float *w, float *m, float *v, uint16_t *out,
                      const StepConsts &c, void *stream, int waves_per_cu = -1);
// One aligned segment of a norm pass: gradient elements from g_off (a
// multiple of 8) past every gradient base, g at g_out_off past g_out, its
// tiles' partials from `partial`, its first tile starting `phase` elements
// before it (norm_segment_phase).
struct NormSegment {
    int64_t g_off, g_out_off, len, partial;
    int phase;
};
// The segments in as few launches as possible, each tile's partial where a
// launch per segment puts it.  Every gradient base 16-byte aligned (g_out's
// too).  hipErrorNotSupported without a compiled bf16 kernel for n_grads.
int launch_norm_batch(const NormSegment *segs, int count, const void *const *grads, int n_grads,
                      int grad_dtype, float *g_out, const StepConsts &c, double *partials,
                      void *stream);
// One segment of `len` elements: grads and g_out already point at its first
// element, which lies at least `phase` elements into every gradient buffer.
int launch_norm_segment(int64_t len, int phase, bool vec, const void *const *grads, int n_grads,
                        int grad_dtype, float *g_out, const StepConsts &c, double *partials,
                        void *stream);
// The tiles (partials) of a segment of `len` elements whose first tile starts
// `phase` elements before it.
int64_t norm_segment_blocks(int64_t len, int phase);
// The phase of a segment whose gradients start g_off elements into their
// buffers: g_off modulo a 128-byte line of gradients, rounded down to whole
// octs.  A function of the layout, rank and index spaces only, so the
// partition (and the sum's bits) never depends on the pointers.
int norm_segment_phase(int64_t g_off, int grad_bytes);
// The staged step's first half over len elements: g = (rank-ordered sum) /
// divisor written to g_out (fp32), 16-byte gradient loads when vec.
int launch_stage_reduce(int64_t len, bool vec, const void *const *grads, int n_grads,
                        int grad_dtype, float *g_out, const StepConsts &c, void *stream);

// True if every gradient (at element g_off) and g_out (at s_off, if given)
// is 16-byte aligned, so the norm can load whole octs (8 bf16 in one access,
// 8 fp32 in two) and store g as quads on a segment.
bool segment_vec_aligned(const Segment &s, const Request &rq);
// Reduce n_partials partials to one value at *result (fixed order, several
// levels of kNormFanIn-way workgroups); scratch holds the intermediate
// levels (norm_tree_scratch(n_partials) doubles).
// coef (and *total unless null) from the rank-ordered binary64 sum of n sums.
int launch_clip_coef(const double *sums, int n, double max_norm, float *coef, double *total,
                     void *stream);
int launch_norm_tree(const double *partials, int64_t n_partials, double *scratch, double *result,
                     void *stream);
// Device address, on the current device, of the library-owned partials array
// of zero_gradnorm_async_noalloc (ZERO_NOALLOC_SCRATCH_BYTES); looked up once
// per device.  Returns a hipError_t value.
int noalloc_scratch(void **ptr);
int64_t norm_tree_scratch(int64_t n_partials);
int launch_convert(const void *src, int src_dtype, void *dst, int dst_dtype, int64_t n,
                   void *stream);
int launch_fill_zero(void *dst, int dtype, int64_t n, void *stream);

// Device copies of a reshard plan (src[r] + src_k -> dst + dst_k, zero runs
// filled), `elem` bytes per element; batched into few launches.
int launch_reshard(const std::vector<ReshardRun> &runs, const void *const *src, void *dst,
                   int elem, void *stream);

}  // namespace zero
