// capi.cpp -- the exported entry points: argument validation, aliasing
// checks, the per-piece launch loop of the step and the norm, the packer's
// copies, and diagnostics.  Every check runs before any device work.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "zero_internal.h"

namespace zero {

namespace {
thread_local std::string t_last_hip_error;

bool dtype_ok(int32_t d) { return d == ZERO_F32 || d == ZERO_BF16; }
bool index_ok(int32_t x) { return x == ZERO_GLOBAL || x == ZERO_LOCAL; }
int dsize(int32_t d) { return d == ZERO_BF16 ? 2 : 4; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t extent(const zero_layout *L, int32_t index)
{
    return index == ZERO_GLOBAL ? L->padded : L->shard;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void *p, int64_t elems, int elem_size)
{
    const uintptr_t lo = (uintptr_t)p;
    return {lo, lo + (uintptr_t)elems * (uintptr_t)elem_size};
}
bool overlap(Range a, Range b)
{
    if (a.lo == a.hi || b.lo == b.hi)
        return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// The checks zero_step and zero_gradnorm share: selection, gradients and
// divisor.  empty_grads: the gradient buffers hold no element (an empty unit
// range), so their pointers may be NULL.
zero_status check_grads(const zero_layout *L, int32_t rank, const void *const *grads,
                        int32_t n_grads, int32_t grad_dtype, int32_t grad_index, float divisor,
                        bool empty_grads = false)
{
    if (!layout_ok(L) || rank >= L->n_ranks || !dtype_ok(grad_dtype) || !index_ok(grad_index))
        return ZERO_EINVAL;
    if (!grads)
        return ZERO_EINVAL;
    if (n_grads < 1 || n_grads > ZERO_MAX_RANKS)
        return ZERO_ERANGE;
    if (!(divisor > 0.0f) || !std::isfinite(divisor))
        return ZERO_EINVAL;
    for (int q = 0; q < n_grads; ++q) {
        if (!grads[q] && !empty_grads)
            return ZERO_EINVAL;
        if (!aligned(grads[q], (size_t)dsize(grad_dtype)))
            return ZERO_EALIGN;
    }
    return ZERO_OK;
}

std::vector<const void *> offset_grads(const void *const *grads, int n, int64_t off, int gsize)
{
    std::vector<const void *> v((size_t)n);
    for (int q = 0; q < n; ++q)
        v[(size_t)q] = (const char *)grads[q] + off * gsize;
    return v;
}

}  // namespace

StepConsts make_step_consts(const zero_adamw_scalars *sc, float divisor)
{
    StepConsts c{};
    if (sc) {
        c.b1 = sc->b1;
        c.b2 = sc->b2;
        c.omb1 = sc->one_minus_b1;
        c.omb2 = sc->one_minus_b2;
        c.bc2 = sc->bc2;
        c.eps = sc->eps;
        c.step_size = sc->step_size;
        c.decay = sc->decay;
        c.clip = sc->clip_coef;
    }
    c.divisor = divisor;
    float inv = 0.0f;
    c.div_pow2 = is_pow2_float(divisor, &inv) ? 1 : 0;
    c.inv_divisor = inv;
    return c;
}

bool is_pow2_float(float x, float *inv)
{
    // Powers of two in [2^-126, 2^126], whose reciprocal is exact and normal.
    if (!(x >= 0x1p-126f && x <= 0x1p126f))
        return false;
    int e = 0;
    const float mant = std::frexp(x, &e);
    if (mant != 0.5f)
        return false;
    *inv = std::ldexp(1.0f, 1 - e);
    return true;
}

int device_cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return -1;
    static std::mutex mu;
    static std::vector<int> cache;
    std::lock_guard<std::mutex> lock(mu);
    if ((size_t)dev >= cache.size())
        cache.resize((size_t)dev + 1, 0);
    if (cache[(size_t)dev] == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return -1;
        cache[(size_t)dev] = cu;
    }
    return cache[(size_t)dev];
}

namespace {
struct DeviceLds {
    int per_cu = 0, per_block = 0;
};
DeviceLds device_lds()
{
    static std::mutex mu;
    static std::vector<DeviceLds> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return {};
    std::lock_guard<std::mutex> lock(mu);
    if ((size_t)dev >= cache.size())
        cache.resize((size_t)dev + 1);
    DeviceLds &d = cache[(size_t)dev];
    if (d.per_cu == 0) {
        int cu = 0, blk = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess ||
            hipDeviceGetAttribute(&blk, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess)
            return {};
        d.per_cu = cu;
        d.per_block = blk;
    }
    return d;
}

int env_int(const char *name, int dflt, int lo, int hi)
{
    if (const char *e = std::getenv(name)) {
        const int x = std::atoi(e);
        if (x >= lo && x <= hi)
            return x;
    }
    return dflt;
}
}  // namespace

size_t occupancy_cap_lds(int waves_per_cu, size_t static_lds)
{
    if (waves_per_cu <= 0)
        return 0;
    const DeviceLds d = device_lds();
    if (d.per_cu <= 0 || d.per_block <= 0)
        return 0;
    // LDS per workgroup in total, in whole allocation granules (rounding
    // the cap up), of which the kernel's own static LDS is part.
    size_t lds = (size_t)d.per_cu / (size_t)waves_per_cu;
    lds = lds / 512 * 512;
    if (lds > (size_t)d.per_block)
        lds = (size_t)d.per_block;
    return lds > static_lds ? lds - static_lds : 0;
}

namespace {
// Occupancy caps set at run time (zero_set_waves_per_cu); -1 = not set.
std::atomic<int> g_cap_override[3] = {{-1}, {-1}, {-1}};

// The cap of one kernel family: the run-time setting, else the environment
// variable (read once), else the built-in default.
int cap_for(int kind, const char *env, int dflt)
{
    const int o = g_cap_override[kind].load(std::memory_order_relaxed);
    if (o >= 0)
        return o;
    static const int e[3] = {env_int("ZERO_STEP_WAVES_PER_CU", -1, 0, 64),
                             env_int("ZERO_STEP1_WAVES_PER_CU", -1, 0, 64),
                             env_int("ZERO_NORM_WAVES_PER_CU", -1, 0, 64)};
    (void)env;
    return e[kind] >= 0 ? e[kind] : dflt;
}

}  // namespace

int step_waves_per_cu(int n_grads, bool runtime_kernel, int grad_bytes)
{
    // Resident one-wave workgroups per CU of the fused step.  A compiled
    // rank count keeps all N gradient quads of a lane in flight beside
    // master, m and v (4 * grad_bytes * N + 48 bytes per lane), and its best
    // cap falls as those bytes grow: fewer tiles in flight keep fewer DRAM
    // rows competing per bank, too few starve the memory pipeline.  Measured
    // on MI355X with interleaved sweeps in one process (bench.py
    // --sweep-waves step:..., the 8B shard at N ranks), % of 8 TB/s:
    //   bf16 N = 2   (64 B):  5: 53.0  6: 62.8  7: 78.0  8: 82.9  10: 84.1
    //   bf16 N = 3   (72 B):  6: 65.5  7: 79.0  8: 81.7  10: 82.0  12: 81.5
    //   bf16 N = 4   (80 B):  5: 58.8  6: 68.4  7: 80.8  8: 82.1  10: 82.4
    //   fp32 N = 2   (80 B):  6: 69.8  7: 83.0  8: 84.0  10: 82.4
    //   bf16 N = 5   (88 B):  6: 69.2  7: 82.2  8: 83.8  10: 82.3
    //   bf16 N = 6   (96 B):  6: 71.4  7: 83.8  8: 83.8  10: 82.4
    //   bf16 N = 7  (104 B):  6: 73.4  7: 83.6  8: 82.4  10: 81.1
    //   bf16 N = 8  (112 B):  5: 66.0  6: 75.9  7: 84.0  8: 82.0  10: 80.9
    //   fp32 N = 4  (112 B):  6: 77.7  7: 82.3  8: 81.1  10: 80.2
    //   bf16 N = 12 (144 B):  5: 71.6  6: 80.4  7: 80.0  8: 79.0
    //   bf16 N = 16 (176 B):  5: 76.3  6: 81.8  7: 78.9  8: 78.3  10: 77.3
    //   fp32 N = 8  (176 B):  5: 81.0  6: 81.7  7: 78.2  8: 78.0
    //   bf16 N = 20 (208 B):  5: 78.6  6: 80.2  7: 76.7  8: 75.7
    //   bf16 N = 24 (240 B):  4: 80.5  5: 80.5  6: 78.0  7: 75.5
    //   bf16 N = 28 (272 B):  4: 78.1  5: 77.9  6: 76.2  7: 74.7
    //   fp32 N = 16 (304 B):  4: 79.3  5: 79.4  6: 77.0  7: 75.7
    //   bf16 N = 31 (296 B):  4: 77.9  5: 78.0  6: 75.6  7: 73.5
    //   fp32 N = 32 (560 B):  4: 74.1  5: 74.2  6: 72.4  7: 70.3
    //   bf16 N = 64 (560 B):  4: 72.5  5: 72.6  6: 71.8  7: 71.3
    // The run-time kernel issues the loads one batch of 128 bytes per lane
    // at a time, two batches in flight: bf16 takes it only above 32 ranks
    // (N = 48: 5: 63.9  6: 69.7  7: 73.7  8: 73.6  10: 72.8;  N = 128: 5:
    // 64.4  6: 69.3  7: 72.0  8: 71.6  10: 71.0), fp32 at the rank counts
    // without a kernel of their own (N = 3: 8: 77.5  10: 82.2  12: 84.6
    // 16: 80.5;  N = 12: 6: 77.2  7: 79.6  8: 78.4;  N = 24: 4: 76.4
    // 5: 76.4  6: 75.2  7: 73.0).
    int dflt;
    if (runtime_kernel) {
        dflt = grad_bytes == 2 ? 7 : n_grads <= 4 ? 12 : n_grads <= 12 ? 7 : 5;
    } else {
        const int lane_bytes = 4 * grad_bytes * n_grads + 48;
        dflt = lane_bytes <= 72 ? 10 : lane_bytes <= 88 ? 8 : lane_bytes <= 112 ? 7
             : lane_bytes <= 208 ? 6 : 5;
    }
    return cap_for(0, "ZERO_STEP_WAVES_PER_CU", dflt);
}

int step1_waves_per_cu(bool staged_chunk)
{
    // The step on one fp32 gradient (4 streams in flight): the clipped step
    // after the norm pass, best at 10 (8 and 12 within 0.3 points, 6: 3.5
    // lower, uncapped: 1.4 lower); the staged step's second half, whose
    // gradient chunk was just written and is mostly read back from the
    // memory-side cache (shorter load latency), best at 12 (8: 0.8 points
    // lower, 10: 0.2, 14 and 16: 0.2).
    return cap_for(1, "ZERO_STEP1_WAVES_PER_CU", staged_chunk ? 12 : 10);
}

int norm_waves_per_cu(int n_grads, bool runtime_kernel, int grad_bytes)
{
    // The norm pass and the staged step's reduction: N reads of 16 bytes per
    // lane and one write.  Measured (bench.py --sweep-waves norm:..., the 8B
    // shard at N ranks, three interleaved rounds; % of 8 TB/s):
    // compiled N = 64 (staged reduction) 4: 78.5  5: 78.6  6: 77.8
    // 7: 76.4, and N = 32 like it (3 starves at 57 %); compiled N = 24 best
    // at 6 (5 % above 5 and 7), N = 12 at 7 (6: 5 % lower).  The run-time
    // kernel (two batches of 128 bytes per lane in flight; bf16 above 32
    // ranks, fp32 at every N), as the staged step / the clipped workload's
    // norm pass:
    //   bf16 N = 40   5: 74.6 / 77.8  6: 77.0 / 80.5  7: 76.2 / 78.7  8: 75.6 / 77.8
    //   bf16 N = 48   5: 75.3 / 77.8  6: 77.1 / 80.6  7: 76.3 / 78.9  8: 75.4 / 77.9
    //   bf16 N = 96   5: 73.6 / 75.0  6: 75.1 / 77.7  7: 74.4 / 76.4  8: 74.3 / 75.9
    //   bf16 N = 128  5: 77.0 / 77.4  6: 77.9 / 79.6  7: 78.1 / 79.0  8: 77.3 / 78.1
    //   bf16 N = 192  5: 77.3 / 77.6  6: 77.4 / 79.7  7: 76.3 / 79.8  8: 75.7 / 78.9
    //   bf16 N = 256  5: 76.2 / 76.3  6: 78.4 / 78.4  7: 80.2 / 80.1  8: 79.5 / 79.4
    // fp32 gradients (the staged step from 33 ranks, the clipped workload's
    // norm pass at every N; the staged step only where measured):
    //   fp32 N = 8    4:   — / 77.8  5:   — / 77.9  6:   — / 76.5  7:   — / 75.8
    //   fp32 N = 16   4:   — / 83.1  5:   — / 81.8  6:   — / 81.2  7:   — / 80.8
    //   fp32 N = 32   4:   — / 81.8  5:   — / 80.7  6:   — / 79.7  7:   — / 78.2
    //   fp32 N = 48   4: 81.3 / 85.9  5: 81.1 / 85.0  6: 80.4 / 84.7  7: 79.7 / 84.6
    //   fp32 N = 64   4: 71.8 /   —   5: 72.7 /   —   6: 74.3 /   —   7: 74.8 /   —
    //   fp32 N = 128  4: 82.5 / 83.8  5: 82.7 / 82.9  6: 82.2 / 82.1  7: 81.6 / 81.2
    //   fp32 N = 256  4: 82.9 /   —   5: 84.5 /   —   6: 84.0 /   —   7: 83.7 /   —
    // so 6 for bf16 up to 192 ranks and 7 above; 4 for fp32 up to 128 ranks
    // and 5 above (an fp32 lane's two batches hold as many bytes as bf16's
    // over half the ranks).  The staged step at 64 fp32 ranks was swept on
    // buffers 32 MiB + 256 KiB apart modulo 64 MiB, a placement that cost it
    // 7 to 9 points at any cap; zero_arena_plan now moves such runs (79 %
    // at the cap above).
    int dflt;
    if (runtime_kernel)
        dflt = grad_bytes == 2 ? (n_grads <= 192 ? 6 : 7) : (n_grads <= 128 ? 4 : 5);
    else
        dflt = n_grads <= 16 ? 7 : n_grads <= 24 ? 6 : 5;
    return cap_for(2, "ZERO_NORM_WAVES_PER_CU", dflt);
}

zero_status hip_fail(int err, const char *where)
{
    char buf[256];
    std::snprintf(buf, sizeof buf, "%s: %s (%d)", where,
                  hipGetErrorString(static_cast<hipError_t>(err)), err);
    t_last_hip_error = buf;
    return ZERO_EHIP;
}

}  // namespace zero

using namespace zero;

zero_status zero::validate_step(const zero_layout *L, int32_t rank, const void *const *grads,
                               int32_t n_grads, int32_t grad_dtype, int32_t grad_index,
                               float divisor, const float *master, const float *exp_avg,
                               const float *exp_avg_sq, int32_t state_index, const uint16_t *out,
                               int32_t out_index, const zero_adamw_scalars *sc)
{
    return validate_step_ext(L, rank, grads, n_grads, grad_dtype, grad_index, divisor, master,
                             exp_avg, exp_avg_sq, state_index, out, out_index, sc,
                             layout_ok(L) && index_ok(grad_index) ? extent(L, grad_index) : 0);
}

zero_status zero::validate_step_ext(const zero_layout *L, int32_t rank, const void *const *grads,
                                   int32_t n_grads, int32_t grad_dtype, int32_t grad_index,
                                   float divisor, const float *master, const float *exp_avg,
                                   const float *exp_avg_sq, int32_t state_index,
                                   const uint16_t *out, int32_t out_index,
                                   const zero_adamw_scalars *sc, int64_t grad_extent)
{
    zero_status st = check_grads(L, rank, grads, n_grads, grad_dtype, grad_index, divisor,
                                 grad_extent == 0);
    if (st != ZERO_OK)
        return st;
    if (!index_ok(state_index) || !index_ok(out_index) || !master || !exp_avg || !exp_avg_sq ||
        !sc || sc->t < 1)
        return ZERO_EINVAL;
    if (rank < 0 && (grad_index != ZERO_GLOBAL || state_index != ZERO_GLOBAL ||
                     out_index != ZERO_GLOBAL))
        return ZERO_EINVAL;
    if (!aligned(master, 4) || !aligned(exp_avg, 4) || !aligned(exp_avg_sq, 4) ||
        (out && !aligned(out, 2)))
        return ZERO_EALIGN;

    // Aliasing: gradients are read-only and may alias each other; nothing
    // written may overlap a gradient or another written buffer.
    const int gsize = dsize(grad_dtype);
    const int64_t ge = grad_extent, se = extent(L, state_index), oe = extent(L, out_index);
    const Range w = range_of(master, se, 4), m = range_of(exp_avg, se, 4),
                v = range_of(exp_avg_sq, se, 4),
                o = out ? range_of(out, oe, 2) : Range{0, 0};
    if (overlap(w, m) || overlap(w, v) || overlap(m, v) || overlap(w, o) || overlap(m, o) ||
        overlap(v, o))
        return ZERO_EINVAL;
    for (int q = 0; q < n_grads; ++q) {
        const Range g = range_of(grads[q], ge, gsize);
        if (overlap(g, w) || overlap(g, m) || overlap(g, v) || overlap(g, o))
            return ZERO_EINVAL;
    }
    return ZERO_OK;
}

// Units [u0, u1) of the selection; from_range: the gradient buffers hold only
// those units (offsets from the range's start), of grad_extent elements.
// Arguments already validated.
static zero_status step_launch(const zero_layout *L, int32_t rank, const void *const *grads,
                               int32_t n_grads, int32_t grad_dtype, int32_t grad_index,
                               float divisor, float *master, float *exp_avg, float *exp_avg_sq,
                               int32_t state_index, uint16_t *out, int32_t out_index,
                               const zero_adamw_scalars *sc, const float *clip_dev, void *stream,
                               int32_t u0, int32_t u1, bool from_range)
{
    const int gsize = dsize(grad_dtype);
    StepConsts c = make_step_consts(sc, divisor);
    c.clip_dev = clip_dev;
    Request rq{};
    rq.layout = L;
    rq.rank = rank;
    rq.grads = grads;
    rq.n_grads = n_grads;
    rq.grad_dtype = grad_dtype;
    rq.grad_index = grad_index;
    rq.divisor = divisor;
    rq.state_index = state_index;
    rq.out_index = out_index;
    rq.state_ptrs[0] = master;
    rq.state_ptrs[1] = exp_avg;
    rq.state_ptrs[2] = exp_avg_sq;
    rq.n_state_ptrs = 3;
    rq.out_ptr = out;
    const std::vector<Piece> pieces = build_pieces(
        build_segments(L, rank, grad_index, state_index, out_index, u0, u1, from_range), rq);
    // Two or more vector pieces (one rank's slice of several units), or a
    // piece whose wave grid is shifted to cache lines, go out through the
    // shared-launch kernel when every base is quad-aligned; otherwise, and
    // for the heads, tails and unaligned runs, one launch per piece.
    std::vector<Piece> vec;
    bool aligned = (uintptr_t)master % 16 == 0 && (uintptr_t)exp_avg % 16 == 0 &&
                   (uintptr_t)exp_avg_sq % 16 == 0 && (!out || (uintptr_t)out % 8 == 0);
    for (int32_t q = 0; q < n_grads && aligned; ++q)
        aligned = (uintptr_t)grads[q] % (uintptr_t)(kQuad * gsize) == 0;
    for (const Piece &pc : pieces)
        if (pc.vec && aligned)
            vec.push_back(pc);
    bool batched = false;
    bool shifted = false;  // a grid phase only the shared-launch kernel applies
    for (const Piece &pc : vec)
        shifted = shifted || pc.phase != 0;
    if (vec.size() >= 2 || shifted) {
        const int err = launch_step_batch(vec.data(), (int)vec.size(), grads, n_grads, grad_dtype,
                                          master, exp_avg, exp_avg_sq, out, c, stream);
        if (err != hipSuccess && err != hipErrorNotSupported)
            return hip_fail(err, "zero_step launch");
        batched = err == hipSuccess;
    }
    for (const Piece &pc : pieces) {
        if (batched && pc.vec)
            continue;
        const std::vector<const void *> gp = offset_grads(grads, n_grads, pc.g_off, gsize);
        const int err = launch_step_piece(pc, gp.data(), n_grads, grad_dtype, master + pc.s_off,
                                          exp_avg + pc.s_off, exp_avg_sq + pc.s_off,
                                          out ? out + pc.o_off : nullptr, c, stream);
        if (err != hipSuccess)
            return hip_fail(err, "zero_step launch");
    }
    return ZERO_OK;
}

static zero_status step_impl(const zero_layout *L, int32_t rank, const void *const *grads,
                             int32_t n_grads, int32_t grad_dtype, int32_t grad_index,
                             float divisor, float *master, float *exp_avg, float *exp_avg_sq,
                             int32_t state_index, uint16_t *out, int32_t out_index,
                             const zero_adamw_scalars *sc, const float *clip_dev, void *stream)
{
    zero_status st = validate_step(L, rank, grads, n_grads, grad_dtype, grad_index, divisor,
                                   master, exp_avg, exp_avg_sq, state_index, out, out_index, sc);
    if (st != ZERO_OK)
        return st;
    return step_launch(L, rank, grads, n_grads, grad_dtype, grad_index, divisor, master, exp_avg,
                       exp_avg_sq, state_index, out, out_index, sc, clip_dev, stream, 0, -1, false);
}

extern "C" zero_status zero_step(const zero_layout *L, int32_t rank, const void *const *grads,
                                 int32_t n_grads, int32_t grad_dtype, int32_t grad_index,
                                 float divisor, float *master, float *exp_avg, float *exp_avg_sq,
                                 int32_t state_index, uint16_t *out, int32_t out_index,
                                 const zero_adamw_scalars *sc, void *stream)
{
    return step_impl(L, rank, grads, n_grads, grad_dtype, grad_index, divisor, master, exp_avg,
                     exp_avg_sq, state_index, out, out_index, sc, nullptr, stream);
}

extern "C" zero_status zero_step_device_clip(const zero_layout *L, int32_t rank,
                                             const void *const *grads, int32_t n_grads,
                                             int32_t grad_dtype, int32_t grad_index,
                                             float divisor, float *master, float *exp_avg,
                                             float *exp_avg_sq, int32_t state_index,
                                             uint16_t *out, int32_t out_index,
                                             const zero_adamw_scalars *sc,
                                             const float *clip_coef_dev, void *stream)
{
    if (!clip_coef_dev)
        return ZERO_EINVAL;
    if (!aligned(clip_coef_dev, 4))
        return ZERO_EALIGN;
    if (layout_ok(L) && index_ok(state_index) && index_ok(out_index)) {
        // the multiplier is read while the step writes: it must not alias
        const Range cr = range_of(clip_coef_dev, 1, 4);
        const int64_t se = extent(L, state_index), oe = extent(L, out_index);
        if (overlap(cr, range_of(master, se, 4)) || overlap(cr, range_of(exp_avg, se, 4)) ||
            overlap(cr, range_of(exp_avg_sq, se, 4)) || (out && overlap(cr, range_of(out, oe, 2))))
            return ZERO_EINVAL;
    }
    return step_impl(L, rank, grads, n_grads, grad_dtype, grad_index, divisor, master, exp_avg,
                     exp_avg_sq, state_index, out, out_index, sc, clip_coef_dev, stream);
}

extern "C" zero_status zero_clip_coef_async(const double *sumsq_dev, double max_norm,
                                            float *coef_dev, void *stream)
{
    if (!sumsq_dev || !coef_dev || !(max_norm > 0.0))
        return ZERO_EINVAL;
    if (!aligned(sumsq_dev, 8) || !aligned(coef_dev, 4))
        return ZERO_EALIGN;
    const int err = launch_clip_coef(sumsq_dev, 1, max_norm, coef_dev, nullptr, stream);
    return err == hipSuccess ? ZERO_OK : hip_fail(err, "zero_clip_coef_async");
}

extern "C" zero_status zero_clip_coef_ranks_async(const double *rank_sums_dev, int32_t n_ranks,
                                                  double max_norm, float *coef_dev,
                                                  double *total_dev, void *stream)
{
    if (!rank_sums_dev || !coef_dev || n_ranks < 1 || n_ranks > ZERO_MAX_UNITS ||
        !(max_norm > 0.0))
        return ZERO_EINVAL;
    if (!aligned(rank_sums_dev, 8) || !aligned(coef_dev, 4) || (total_dev && !aligned(total_dev, 8)))
        return ZERO_EALIGN;
    const int err = launch_clip_coef(rank_sums_dev, n_ranks, max_norm, coef_dev, total_dev, stream);
    return err == hipSuccess ? ZERO_OK : hip_fail(err, "zero_clip_coef_ranks_async");
}

// ---- the staged step ------------------------------------------------------

extern "C" zero_status zero_step_staged_workspace_bytes(const zero_layout *L, int32_t rank,
                                                        int32_t n_grads, size_t *bytes)
{
    if (!layout_ok(L) || !bytes || rank >= L->n_ranks)
        return ZERO_EINVAL;
    if (n_grads < 1 || n_grads > ZERO_MAX_RANKS)
        return ZERO_ERANGE;
    if (n_grads < kStageMinRanksF32) {  // the smaller threshold: the dtype is not known here
        *bytes = 0;
        return ZERO_OK;
    }
    int64_t e = selected_elements(L, rank);
    e = (e + kNormSpan - 1) / kNormSpan * kNormSpan;
    if (e < kNormSpan)
        e = kNormSpan;
    if (e > kStageMaxChunk)
        e = kStageMaxChunk;
    // one chunk, plus 16 bytes to place it at the state's 16-byte phase
    *bytes = (size_t)(e + kStageSlack) * sizeof(float);
    return ZERO_OK;
}

// The staged step over units [u0, u1) (from_range: gradient buckets of
// grad_extent elements holding only those units); step arguments validated,
// n_grads >= stage_min_ranks(grad_dtype).
static zero_status staged_launch(const zero_layout *L, int32_t rank, const void *const *grads,
                                 int32_t n_grads, int32_t grad_dtype, int32_t grad_index,
                                 float divisor, float *master, float *exp_avg, float *exp_avg_sq,
                                 int32_t state_index, uint16_t *out, int32_t out_index,
                                 const zero_adamw_scalars *sc, void *workspace,
                                 size_t workspace_bytes, void *stream, int32_t u0, int32_t u1,
                                 bool from_range, int64_t grad_extent)
{
    if (!workspace)
        return ZERO_EINVAL;
    if (!aligned(workspace, 16))
        return ZERO_EALIGN;
    if (workspace_bytes < (size_t)kNormSpan * sizeof(float))
        return ZERO_ENOSPC;
    // chunk: the workspace's whole 512-element tiles, at most kStageMaxChunk,
    // less kStageSlack elements when there is room for them: each chunk's g
    // then starts at the state's 16-byte phase, so that the second half's
    // quads line up with the state's.  The call writes no workspace byte past
    // chunk + slack elements.
    size_t ws_elems = workspace_bytes / sizeof(float);
    const bool shift_ok = ws_elems >= (size_t)(kNormSpan + kStageSlack);
    if (shift_ok)
        ws_elems -= kStageSlack;
    if (ws_elems > (size_t)kStageMaxChunk)
        ws_elems = (size_t)kStageMaxChunk;
    const int64_t chunk = (int64_t)ws_elems / kNormSpan * kNormSpan;
    const int gsize = dsize(grad_dtype);
    const Range ws =
        range_of(workspace, (chunk + (shift_ok ? kStageSlack : 0)) * (int64_t)sizeof(float), 1);
    const int64_t se = extent(L, state_index), oe = extent(L, out_index);
    if (overlap(ws, range_of(master, se, 4)) || overlap(ws, range_of(exp_avg, se, 4)) ||
        overlap(ws, range_of(exp_avg_sq, se, 4)) || (out && overlap(ws, range_of(out, oe, 2))))
        return ZERO_EINVAL;
    for (int q = 0; q < n_grads; ++q)
        if (overlap(ws, range_of(grads[q], grad_extent, gsize)))
            return ZERO_EINVAL;

    float *g = static_cast<float *>(workspace);
    const StepConsts ca = make_step_consts(nullptr, divisor);  // the average
    const StepConsts cb = make_step_consts(sc, 1.0f);          // g is averaged already
    const void *g1[1] = {g};
    Request rq{};  // the second half: one fp32 gradient (the workspace)
    rq.layout = L;
    rq.rank = rank;
    rq.grads = g1;
    rq.n_grads = 1;
    rq.grad_dtype = ZERO_F32;
    rq.grad_index = ZERO_LOCAL;
    rq.divisor = 1.0f;
    rq.state_index = state_index;
    rq.out_index = out_index;
    rq.state_ptrs[0] = master;
    rq.state_ptrs[1] = exp_avg;
    rq.state_ptrs[2] = exp_avg_sq;
    rq.n_state_ptrs = 3;
    rq.out_ptr = out;
    Request ra{};  // alignment of the first half: the gradients and the workspace
    ra.grads = grads;
    ra.n_grads = n_grads;
    ra.grad_dtype = grad_dtype;
    ra.state_ptrs[0] = g;
    ra.n_state_ptrs = 1;
    for (const Segment &sg :
         build_segments(L, rank, grad_index, state_index, out_index, u0, u1, from_range)) {
        for (int64_t off = 0; off < sg.len; off += chunk) {
            const int64_t cl = sg.len - off < chunk ? sg.len - off : chunk;
            const int64_t g0 = sg.g_off + off, s0 = sg.s_off + off;
            // Place the chunk's g at the state's phase p (elements past a
            // 16-byte boundary) and find the head h after which both the
            // gradients (16-byte octs) and g are 16-byte aligned, so both
            // halves run their vector kernels.  Such an h exists exactly when
            // the gradients and the state share a quad phase, which is also
            // when the fused step vectorizes; otherwise g starts at the
            // workspace's own alignment.
            int64_t p = 0, head = -1;
            if (shift_ok) {
                p = (int64_t)(((uintptr_t)master / sizeof(float) + (uint64_t)s0) % 4);
                ra.state_ptrs[0] = g + p;
                for (int64_t h = 0; h < 8 && head < 0; ++h)
                    if (segment_vec_aligned(Segment{g0 + h, h, 0, cl - h}, ra))
                        head = h;
                if (head < 0)
                    p = 0;
            }
            float *gb = g + p;
            ra.state_ptrs[0] = gb;
            const std::vector<const void *> gp = offset_grads(grads, n_grads, g0, gsize);
            int err = hipSuccess;
            if (head < 0) {  // no common phase: one launch, vector only if already aligned
                err = launch_stage_reduce(cl, segment_vec_aligned(Segment{g0, 0, 0, cl}, ra),
                                          gp.data(), n_grads, grad_dtype, gb, ca, stream);
            } else {
                const int64_t hl = head < cl ? head : cl;
                err = launch_stage_reduce(hl, false, gp.data(), n_grads, grad_dtype, gb, ca, stream);
                if (err == hipSuccess && cl > hl) {
                    const std::vector<const void *> gv = offset_grads(grads, n_grads, g0 + hl, gsize);
                    err = launch_stage_reduce(cl - hl, true, gv.data(), n_grads, grad_dtype, gb + hl,
                                              ca, stream);
                }
            }
            if (err != hipSuccess)
                return hip_fail(err, "zero_step_staged reduce");
            g1[0] = gb;  // the second half's gradient, for its alignment
            const Segment sb{0, s0, sg.o_off + off, cl};
            for (const Piece &pc : build_pieces({sb}, rq)) {
                const void *const gq[1] = {gb + pc.g_off};
                err = launch_step_piece(pc, gq, 1, ZERO_F32, master + pc.s_off,
                                        exp_avg + pc.s_off, exp_avg_sq + pc.s_off,
                                        out ? out + pc.o_off : nullptr, cb, stream,
                                        step1_waves_per_cu(true));
                if (err != hipSuccess)
                    return hip_fail(err, "zero_step_staged step");
            }
        }
    }
    return ZERO_OK;
}

extern "C" zero_status zero_step_staged(const zero_layout *L, int32_t rank,
                                        const void *const *grads, int32_t n_grads,
                                        int32_t grad_dtype, int32_t grad_index, float divisor,
                                        float *master, float *exp_avg, float *exp_avg_sq,
                                        int32_t state_index, uint16_t *out, int32_t out_index,
                                        const zero_adamw_scalars *sc, void *workspace,
                                        size_t workspace_bytes, void *stream)
{
    zero_status st = validate_step(L, rank, grads, n_grads, grad_dtype, grad_index, divisor,
                                   master, exp_avg, exp_avg_sq, state_index, out, out_index, sc);
    if (st != ZERO_OK)
        return st;
    if (n_grads < stage_min_ranks(grad_dtype))  // few streams: the fused step is the faster one
        return step_launch(L, rank, grads, n_grads, grad_dtype, grad_index, divisor, master,
                           exp_avg, exp_avg_sq, state_index, out, out_index, sc, nullptr, stream,
                           0, -1, false);
    return staged_launch(L, rank, grads, n_grads, grad_dtype, grad_index, divisor, master,
                         exp_avg, exp_avg_sq, state_index, out, out_index, sc, workspace,
                         workspace_bytes, stream, 0, -1, false, extent(L, grad_index));
}

extern "C" zero_status zero_step_units(const zero_layout *L, int32_t rank, int32_t unit_begin,
                                       int32_t unit_end, const void *const *grads,
                                       int32_t n_grads, int32_t grad_dtype, int32_t grad_index,
                                       float divisor, float *master, float *exp_avg,
                                       float *exp_avg_sq, int32_t state_index, uint16_t *out,
                                       int32_t out_index, const zero_adamw_scalars *sc,
                                       void *workspace, size_t workspace_bytes, void *stream)
{
    if (!layout_ok(L) || !index_ok(grad_index) || unit_begin < 0 || unit_end < unit_begin ||
        unit_end > L->n_units)
        return ZERO_EINVAL;
    // the buckets hold the range's units in the gradient's index space
    const int64_t ge = rank < 0 && grad_index == ZERO_LOCAL
                           ? 0
                           : unit_start(L, unit_end, grad_index) - unit_start(L, unit_begin, grad_index);
    zero_status st = validate_step_ext(L, rank, grads, n_grads, grad_dtype, grad_index, divisor,
                                       master, exp_avg, exp_avg_sq, state_index, out, out_index,
                                       sc, ge);
    if (st != ZERO_OK)
        return st;
    if (workspace && n_grads >= stage_min_ranks(grad_dtype))
        return staged_launch(L, rank, grads, n_grads, grad_dtype, grad_index, divisor, master,
                             exp_avg, exp_avg_sq, state_index, out, out_index, sc, workspace,
                             workspace_bytes, stream, unit_begin, unit_end, true, ge);
    return step_launch(L, rank, grads, n_grads, grad_dtype, grad_index, divisor, master,
                       exp_avg, exp_avg_sq, state_index, out, out_index, sc, nullptr, stream,
                       unit_begin, unit_end, true);
}

extern "C" zero_status zero_gradnorm_workspace_bytes(const zero_layout *L, int32_t rank,
                                                     size_t *bytes)
{
    if (!layout_ok(L) || !bytes || rank >= L->n_ranks)
        return ZERO_EINVAL;
    const int64_t np = norm_partials_bound(L, rank);
    *bytes = (size_t)(np + 1 + norm_tree_scratch(np)) * sizeof(double);
    return ZERO_OK;
}

namespace {

// The norm pass up to the device-side result: validation, stage 1 over the
// segments, the fixed-order tree.  *n_partials = 0 means nothing was selected
// (no launch; the caller reports 0).
zero_status gradnorm_launch(const zero_layout *L, int32_t rank, const void *const *grads,
                            int32_t n_grads, int32_t grad_dtype, int32_t grad_index,
                            float divisor, float *g_out, int32_t g_index, void *workspace,
                            size_t workspace_bytes, double *result, void *stream,
                            int64_t *n_partials)
{
    zero_status st = check_grads(L, rank, grads, n_grads, grad_dtype, grad_index, divisor);
    if (st != ZERO_OK)
        return st;
    if (!workspace || !index_ok(g_index) || !result)
        return ZERO_EINVAL;
    if (rank < 0 && (grad_index != ZERO_GLOBAL || g_index != ZERO_GLOBAL))
        return ZERO_EINVAL;
    if (!aligned(workspace, 8) || (g_out && !aligned(g_out, 4)) || !aligned(result, 8))
        return ZERO_EALIGN;
    size_t need = 0;
    zero_gradnorm_workspace_bytes(L, rank, &need);
    if (workspace_bytes < need)
        return ZERO_ENOSPC;
    const int gsize = dsize(grad_dtype);
    const Range ws = range_of(workspace, (int64_t)need, 1);
    const Range go = g_out ? range_of(g_out, extent(L, g_index), 4) : Range{0, 0};
    const Range rs = range_of(result, 1, 8);
    if (overlap(ws, go) || overlap(rs, go) || (result != static_cast<double *>(workspace) +
                                                          norm_partials_bound(L, rank) &&
                                               overlap(rs, ws)))
        return ZERO_EINVAL;
    for (int q = 0; q < n_grads; ++q) {
        const Range g = range_of(grads[q], extent(L, grad_index), gsize);
        if (overlap(g, ws) || overlap(g, go) || overlap(g, rs))
            return ZERO_EINVAL;
    }

    const StepConsts c = make_step_consts(nullptr, divisor);
    Request rq{};
    rq.layout = L;
    rq.rank = rank;
    rq.grads = grads;
    rq.n_grads = n_grads;
    rq.grad_dtype = grad_dtype;
    rq.grad_index = grad_index;
    rq.divisor = divisor;
    rq.state_index = g_index;
    rq.out_index = ZERO_LOCAL;
    rq.state_ptrs[0] = g_out;
    rq.n_state_ptrs = g_out ? 1 : 0;
    rq.out_ptr = nullptr;
    // workspace: [partials | result slot | tree levels]
    double *partials = static_cast<double *>(workspace);
    double *tree = partials + norm_partials_bound(L, rank) + 1;
    const std::vector<Segment> segs = build_segments(L, rank, grad_index, g_index, ZERO_LOCAL);
    // Two or more aligned segments (one rank's slice of several units) share
    // launches when every base is 16-byte aligned; each segment's tiles and
    // partial slots are the same either way.
    bool aligned = !g_out || (uintptr_t)g_out % 16 == 0;
    for (int32_t q = 0; q < n_grads && aligned; ++q)
        aligned = (uintptr_t)grads[q] % 16 == 0;
    std::vector<NormSegment> batch;
    std::vector<bool> in_batch(segs.size(), false);
    int64_t total = 0;
    for (size_t k = 0; k < segs.size(); ++k) {
        const Segment &sg = segs[k];
        const int phase = norm_segment_phase(sg.g_off, gsize);
        if (aligned && sg.g_off % kOct == 0 && segment_vec_aligned(sg, rq)) {
            batch.push_back(NormSegment{sg.g_off, sg.s_off, sg.len, total, phase});
            in_batch[k] = true;
        }
        total += norm_segment_blocks(sg.len, phase);
    }
    bool batched = false;
    if (batch.size() >= 2) {
        const int err = launch_norm_batch(batch.data(), (int)batch.size(), grads, n_grads,
                                          grad_dtype, g_out, c, partials, stream);
        if (err != hipSuccess && err != hipErrorNotSupported)
            return hip_fail(err, "zero_gradnorm stage 1");
        batched = err == hipSuccess;
    }
    total = 0;
    for (size_t k = 0; k < segs.size(); ++k) {
        const Segment &sg = segs[k];
        const int phase = norm_segment_phase(sg.g_off, gsize);
        if (!(batched && in_batch[k])) {
            const std::vector<const void *> gp = offset_grads(grads, n_grads, sg.g_off, gsize);
            const int err = launch_norm_segment(sg.len, phase, segment_vec_aligned(sg, rq),
                                                gp.data(), n_grads, grad_dtype,
                                                g_out ? g_out + sg.s_off : nullptr, c,
                                                partials + total, stream);
            if (err != hipSuccess)
                return hip_fail(err, "zero_gradnorm stage 1");
        }
        total += norm_segment_blocks(sg.len, phase);
    }
    *n_partials = total;
    if (total == 0)
        return ZERO_OK;
    const int err = launch_norm_tree(partials, total, tree, result, stream);
    if (err != hipSuccess)
        return hip_fail(err, "zero_gradnorm stage 2");
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_gradnorm(const zero_layout *L, int32_t rank,
                                     const void *const *grads, int32_t n_grads,
                                     int32_t grad_dtype, int32_t grad_index, float divisor,
                                     float *g_out, int32_t g_index, void *workspace,
                                     size_t workspace_bytes, double *sumsq, void *stream)
{
    if (!sumsq)
        return ZERO_EINVAL;
    if (!layout_ok(L) || rank >= L->n_ranks)
        return ZERO_EINVAL;
    // the result lives in the workspace's result slot
    double *result = workspace ? static_cast<double *>(workspace) + norm_partials_bound(L, rank)
                               : nullptr;
    int64_t np = 0;
    zero_status st = gradnorm_launch(L, rank, grads, n_grads, grad_dtype, grad_index, divisor,
                                     g_out, g_index, workspace, workspace_bytes, result, stream,
                                     &np);
    if (st != ZERO_OK)
        return st;
    if (np == 0) {
        *sumsq = 0.0;
        return ZERO_OK;
    }
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    double host = 0.0;
    int err = hipMemcpyAsync(&host, result, sizeof(double), hipMemcpyDeviceToHost, hs);
    if (err != hipSuccess)
        return hip_fail(err, "zero_gradnorm readback");
    err = hipStreamSynchronize(hs);
    if (err != hipSuccess)
        return hip_fail(err, "zero_gradnorm synchronize");
    *sumsq = host;
    return ZERO_OK;
}

extern "C" zero_status zero_gradnorm_async(const zero_layout *L, int32_t rank,
                                           const void *const *grads, int32_t n_grads,
                                           int32_t grad_dtype, int32_t grad_index, float divisor,
                                           float *g_out, int32_t g_index, void *workspace,
                                           size_t workspace_bytes, double *sumsq_dev,
                                           void *stream)
{
    if (!sumsq_dev)
        return ZERO_EINVAL;
    int64_t np = 0;
    zero_status st = gradnorm_launch(L, rank, grads, n_grads, grad_dtype, grad_index, divisor,
                                     g_out, g_index, workspace, workspace_bytes, sumsq_dev, stream,
                                     &np);
    if (st != ZERO_OK || np > 0)
        return st;
    // nothing selected: the sum is 0 (written by a kernel, not a memset, so
    // the call may sit in a captured graph)
    const int err = launch_fill_zero(sumsq_dev, ZERO_F32, 2, stream);
    return err == hipSuccess ? ZERO_OK : hip_fail(err, "zero_gradnorm_async");
}

extern "C" zero_status zero_gradnorm_async_noalloc(const zero_layout *L, int32_t rank,
                                                   const void *const *grads, int32_t n_grads,
                                                   int32_t grad_dtype, int32_t grad_index,
                                                   float divisor, float *g_out, int32_t g_index,
                                                   double *sumsq_dev, void *stream)
{
    // every argument check before the first HIP call
    if (!sumsq_dev)
        return ZERO_EINVAL;
    zero_status st = check_grads(L, rank, grads, n_grads, grad_dtype, grad_index, divisor);
    if (st != ZERO_OK)
        return st;
    if (!index_ok(g_index) || (rank < 0 && (grad_index != ZERO_GLOBAL || g_index != ZERO_GLOBAL)))
        return ZERO_EINVAL;
    if ((g_out && !aligned(g_out, 4)) || !aligned(sumsq_dev, 8))
        return ZERO_EALIGN;
    size_t need = 0;
    zero_gradnorm_workspace_bytes(L, rank, &need);
    if (need > (size_t)ZERO_NOALLOC_SCRATCH_BYTES)
        return ZERO_ENOSPC;
    void *ws = nullptr;
    const int err = noalloc_scratch(&ws);
    if (err != hipSuccess)
        return hip_fail(err, "zero_gradnorm_async_noalloc scratch");
    int64_t np = 0;
    st = gradnorm_launch(L, rank, grads, n_grads, grad_dtype, grad_index, divisor, g_out, g_index,
                         ws, (size_t)ZERO_NOALLOC_SCRATCH_BYTES, sumsq_dev, stream, &np);
    if (st != ZERO_OK || np > 0)
        return st;
    const int e2 = launch_fill_zero(sumsq_dev, ZERO_F32, 2, stream);
    return e2 == hipSuccess ? ZERO_OK : hip_fail(e2, "zero_gradnorm_async_noalloc");
}

// ---------------------------------------------------------------------------
// Packer copies.
// ---------------------------------------------------------------------------

namespace {

struct ParamPlace {
    int64_t start;  // global index of the parameter's first element
    int64_t numel;
};

// Validate the parameter list against the layout and place every parameter
// in the flat buffer (in list order within each unit).
zero_status place_params(const zero_layout *L, int32_t n_params, const void *const *ptrs,
                         const int64_t *numel, const int32_t *unit, int32_t dtype,
                         std::vector<ParamPlace> &place)
{
    if (n_params < 0 || (n_params > 0 && (!ptrs || !numel || !unit)) || !dtype_ok(dtype))
        return ZERO_EINVAL;
    std::vector<int64_t> fill((size_t)L->n_units, 0);
    place.resize((size_t)n_params);
    for (int32_t p = 0; p < n_params; ++p) {
        if (unit[p] < 0 || unit[p] >= L->n_units || numel[p] < 0 || (numel[p] > 0 && !ptrs[p]))
            return ZERO_EINVAL;
        if (ptrs[p] && !aligned(ptrs[p], (size_t)dsize(dtype)))
            return ZERO_EALIGN;
        const zero_unit &x = L->unit[unit[p]];
        place[(size_t)p] = {x.offset + fill[(size_t)unit[p]], numel[p]};
        fill[(size_t)unit[p]] += numel[p];
        if (fill[(size_t)unit[p]] > x.numel)
            return ZERO_EINVAL;
    }
    for (int32_t u = 0; u < L->n_units; ++u)
        if (fill[(size_t)u] != L->unit[u].numel)
            return ZERO_EINVAL;
    return ZERO_OK;
}

// Where global range [lo, hi) lands in the flat buffer of the copy: the
// global index itself (rank < 0) or rank r's local index.  Returns false if
// none of it belongs to rank r; otherwise clips [lo, hi) to rank r's slice.
bool to_flat(const zero_layout *L, int32_t rank, int32_t u, int64_t &lo, int64_t &hi,
             int64_t &flat_lo)
{
    const zero_unit &x = L->unit[u];
    if (rank < 0) {
        flat_lo = lo;
        return lo < hi;
    }
    const int64_t a = x.offset + (int64_t)rank * x.shard, b = a + x.shard;
    lo = lo > a ? lo : a;
    hi = hi < b ? hi : b;
    if (lo >= hi)
        return false;
    flat_lo = x.local_offset + (lo - a);
    return true;
}

zero_status pack_like(const zero_layout *L, int32_t rank, int32_t n_params,
                      const void *const *params, const int64_t *numel, const int32_t *unit,
                      int32_t param_dtype, void *flat, int32_t flat_dtype, void *stream, bool pack)
{
    if (!layout_ok(L) || rank >= L->n_ranks || !flat || !dtype_ok(flat_dtype))
        return ZERO_EINVAL;
    if (!aligned(flat, (size_t)dsize(flat_dtype)))
        return ZERO_EALIGN;
    std::vector<ParamPlace> place;
    zero_status st = place_params(L, n_params, params, numel, unit, param_dtype, place);
    if (st != ZERO_OK)
        return st;
    const Range fr = range_of(flat, rank < 0 ? L->padded : L->shard, dsize(flat_dtype));
    for (int32_t p = 0; p < n_params; ++p)
        if (params[p] && overlap(fr, range_of(params[p], numel[p], dsize(param_dtype))))
            return ZERO_EINVAL;
    char *fb = static_cast<char *>(flat);
    const int fs = dsize(flat_dtype), ps = dsize(param_dtype);
    for (int32_t p = 0; p < n_params; ++p) {
        int64_t lo = place[(size_t)p].start, hi = lo + place[(size_t)p].numel, flo = 0;
        if (!to_flat(L, rank, unit[p], lo, hi, flo))
            continue;
        char *pp = (char *)params[p] + (lo - place[(size_t)p].start) * ps;
        int err = pack ? launch_convert(pp, param_dtype, fb + flo * fs, flat_dtype, hi - lo, stream)
                       : launch_convert(fb + flo * fs, flat_dtype, pp, param_dtype, hi - lo, stream);
        if (err != hipSuccess)
            return hip_fail(err, pack ? "zero_pack_copy" : "zero_unpack_copy");
    }
    if (pack) {  // zero the padding of every unit
        for (int32_t u = 0; u < L->n_units; ++u) {
            const zero_unit &x = L->unit[u];
            int64_t lo = x.offset + x.numel, hi = x.offset + x.padded, flo = 0;
            if (!to_flat(L, rank, u, lo, hi, flo))
                continue;
            int err = launch_fill_zero(fb + flo * fs, flat_dtype, hi - lo, stream);
            if (err != hipSuccess)
                return hip_fail(err, "zero_pack_copy padding");
        }
    }
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_pack_copy(const zero_layout *L, int32_t rank, int32_t n_params,
                                      const void *const *params, const int64_t *src_numel,
                                      const int32_t *src_unit, int32_t src_dtype, void *dst,
                                      int32_t dst_dtype, void *stream)
{
    return pack_like(L, rank, n_params, params, src_numel, src_unit, src_dtype, dst, dst_dtype,
                     stream, true);
}

extern "C" zero_status zero_unpack_copy(const zero_layout *L, int32_t rank, const void *src,
                                        int32_t src_dtype, int32_t n_params,
                                        void *const *params, const int64_t *dst_numel,
                                        const int32_t *dst_unit, int32_t dst_dtype, void *stream)
{
    return pack_like(L, rank, n_params, (const void *const *)params, dst_numel, dst_unit,
                     dst_dtype, const_cast<void *>(src), src_dtype, stream, false);
}

// ---------------------------------------------------------------------------
// Diagnostics.
// ---------------------------------------------------------------------------

extern "C" const char *zero_strerror(zero_status s)
{
    switch (s) {
    case ZERO_OK: return "ok";
    case ZERO_EINVAL: return "invalid argument";
    case ZERO_ERANGE: return "size or rank count out of range";
    case ZERO_EALIGN: return "pointer not aligned to its element size";
    case ZERO_ENOSPC: return "caller buffer too small";
    case ZERO_EHIP: return "HIP runtime error";
    case ZERO_EIO: return "checkpoint file could not be opened, read or written";
    case ZERO_ECORRUPT: return "not a valid checkpoint shard (magic, version, size, checksum or mismatched shards)";
    default: return "unknown status";
    }
}

extern "C" const char *zero_last_hip_error(void) { return t_last_hip_error.c_str(); }

extern "C" zero_status zero_set_waves_per_cu(int32_t kind, int32_t waves)
{
    if (kind < ZERO_CAP_STEP || kind > ZERO_CAP_NORM || waves < -1 || waves > 64)
        return ZERO_EINVAL;
    g_cap_override[kind].store(waves, std::memory_order_relaxed);
    return ZERO_OK;
}

extern "C" zero_status zero_get_waves_per_cu(int32_t kind, int32_t n_grads, int32_t *waves)
{
    if (kind < ZERO_CAP_STEP || kind > ZERO_CAP_NORM || !waves || n_grads < 1 ||
        n_grads > ZERO_MAX_RANKS)
        return ZERO_EINVAL;
    // the kernels bf16 gradients take
    const bool runtime = !compiled_ranks(n_grads);
    *waves = kind == ZERO_CAP_STEP ? step_waves_per_cu(n_grads, runtime, 2)
           : kind == ZERO_CAP_STEP1 ? step1_waves_per_cu(false)
                                    : norm_waves_per_cu(n_grads, runtime, 2);
    return ZERO_OK;
}

extern "C" int32_t zero_abi_version(void) { return ZERO_ABI_VERSION; }
