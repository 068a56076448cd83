// step_kernels.hip -- the fused sharded optimizer step for gfx950.
//
// One pass over a rank's shard (or every rank's shards) does, per element:
// the rank-ordered binary32 sum of the N ranks' gradients (the reduction half
// of the reduce-scatter), the average, the clip scale, AdamW on the fp32
// master / m / v, and the bf16 cast into the all-gather's output slot
// ("ZeRO and FSDP sharding", How it works and Code).
//
// The work is elementwise and streams every byte once, so the kernel is
// bound by HBM bandwidth: no MFMA, and no LDS traffic.  Mapping: each
// workgroup is one wave64 and owns one tile of 256 consecutive elements;
// lane l owns the quad 4l .. 4l+3 of the tile.  Every wave-wide access is
// therefore one contiguous span -- 512 bytes per rank's bf16 gradients and
// per bf16 output, 1 KiB per fp32 state array -- so each cache line is
// filled by a single instruction and written back whole.  The grid is not
// persistent: one tile per workgroup, so the tiles in flight form one compact
// window that sweeps the buffers in address order.  Workgroups go to the
// eight XCDs in turn, so neighbouring tiles run on different XCDs; giving
// each XCD its own range of tiles instead (the tiles in flight then sit in
// eight separate windows) measured 8 to 12 points lower.  Loads carry the
// nontemporal hint; stores are
// whole-span stores with the nontemporal and device-scope bits (st_span).
// The number of resident waves is capped (7 per CU by default, 5 from 32
// ranks up, 10 or 12 for one fp32 gradient, through a dynamic LDS
// reservation the kernel never touches): fewer tiles in flight keep fewer
// DRAM rows competing per bank across the N + 7 streams.
#include <algorithm>
#include <utility>
#include <vector>

#include "device_common.h"

namespace zero {
namespace {

using namespace dev;

// One wave's tile of the step: lane `lane` owns quad t0 + lane of the
// state (W, M, V) and output (O) arrays and gradient quad gq (an index from
// every rank's gradient base); the wave's stores cover quads t0 .. t0 + 63.
template <int NR, int CAP, typename QD, bool POW2>
__device__ __forceinline__ void step_tile(const GradSet<CAP> &gs, int n, float *__restrict__ W,
                                          float *__restrict__ M, float *__restrict__ V,
                                          uint16_t *__restrict__ O, int64_t gq, int64_t t0,
                                          int lane, const StepConsts &c)
{
    const int64_t i = t0 + lane;
    f32x4 *w4 = reinterpret_cast<f32x4 *>(W) + i;
    f32x4 *m4 = reinterpret_cast<f32x4 *>(M) + i;
    f32x4 *v4 = reinterpret_cast<f32x4 *>(V) + i;

    float s[4];
    rank_sum<NR, CAP, QD>(gs, n, gq, s);
    const f32x4 wq = ld_stream(w4), mq = ld_stream(m4), vq = ld_stream(v4);
    const float clip = c.clip_dev ? *c.clip_dev : c.clip;  // uniform: one scalar load

    float w[4] = {wq.x, wq.y, wq.z, wq.w};
    float m[4] = {mq.x, mq.y, mq.z, mq.w};
    float v[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float g = average<POW2>(s[k], c);
        g = g * clip;
        adamw(g, w[k], m[k], v[k], c);
    }
    // a NaN multiplier from the device (the norm was not finite): the step is
    // skipped and the state left as it is (uniform over the launch); tested
    // here, after the loads, so that no scalar load delays them
    if (c.clip_dev && !(clip == clip))
        return;
    // whole-span stores of the wave's tile (lanes past the end returned)
    st_span(f32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<f32x4 *>(W) + t0, lane);
    st_span(f32x4{m[0], m[1], m[2], m[3]}, reinterpret_cast<f32x4 *>(M) + t0, lane);
    st_span(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(V) + t0, lane);
    if (O)
        st_span(u32x2{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3])},
                reinterpret_cast<u32x2 *>(O) + t0, lane);
}

template <int NR, int CAP, typename QD, bool POW2>
__global__ __launch_bounds__(kWave) void step_quad_kernel(GradSet<CAP> gs, int n,
                                                         float *__restrict__ W,
                                                         float *__restrict__ M,
                                                         float *__restrict__ V,
                                                         uint16_t *__restrict__ O,
                                                         int64_t nquads, StepConsts c)
{
    const int64_t t0 = (int64_t)blockIdx.x * kWave;
    const int lane = threadIdx.x;
    if (t0 + lane >= nquads)
        return;
    step_tile<NR, CAP, QD, POW2>(gs, n, W, M, V, O, t0 + lane, t0, lane, c);
}

// Several vector pieces in one launch -- one rank's slice of every unit, whose
// gradient slices are not contiguous in the gradient buffers -- instead of a
// launch per piece: each launch's drain and refill cost about as much as
// streaming 20 MB, so one rank's GPT-2 Large step (36 pieces of 2.5M
// elements) ran at 64-70 % of the HBM peak against 84 % for the same bytes
// in one piece.  A workgroup finds its piece from a group table (the grid's
// blocks in 512 groups of 512; per group the piece holding its first block,
// bit 7 set when the whole group lies in it) and a forward walk over piece
// ends only when its group holds a boundary.
constexpr int kStepPieces = 64;
constexpr int kStepGroups = 512;
constexpr int kStepGroupShift = 9;  // blocks per group
constexpr int64_t kStepBatchBlocks = int64_t(kStepGroups) << kStepGroupShift;

struct QuadPiece {
    int64_t g, s, o;         // quad offsets from the gradient, state and output bases
    uint32_t nq_phase;       // quads (low 24 bits, < 2^24) | the grid phase << 24
    uint32_t first;          // the launch's first block of this piece
};

struct StepBatch {
    QuadPiece p[kStepPieces];
    uint32_t end[kStepPieces];       // piece i covers blocks [p[i].first, end[i])
    uint32_t group[kStepGroups / 4];  // byte per group, as described above
    int32_t n_pieces, pad;
};
static_assert(sizeof(StepBatch) + sizeof(GradSet<64>) + sizeof(StepConsts) + 64 <= 4096,
              "kernel arguments are limited to 4 KB");

template <int NR, int CAP, typename QD, bool POW2>
__global__ __launch_bounds__(kWave) void step_batch_kernel(GradSet<CAP> gs, int n,
                                                          float *__restrict__ W,
                                                          float *__restrict__ M,
                                                          float *__restrict__ V,
                                                          uint16_t *__restrict__ O,
                                                          const StepBatch b, StepConsts c)
{
    const uint32_t blk = blockIdx.x;
    const uint32_t g = blk >> kStepGroupShift;
    const uint32_t entry = (b.group[g >> 2] >> ((g & 3u) * 8u)) & 0xffu;
    int i = (int)(entry & 0x7fu);
    if (!(entry & 0x80u))
        while (blk >= b.end[i])  // the last piece ends at the grid size: the walk stops there
            ++i;
    const QuadPiece pc = b.p[i];
    // the piece's waves start `phase` quads before it (lanes before the
    // piece, like lanes past its end, do nothing)
    const int64_t t0 = (int64_t)(blk - pc.first) * kWave - (int64_t)(pc.nq_phase >> 24);
    const int lane = threadIdx.x;
    if (t0 + lane < 0 || t0 + lane >= (int64_t)(pc.nq_phase & 0xffffffu))
        return;
    step_tile<NR, CAP, QD, POW2>(gs, n, W + kQuad * pc.s, M + kQuad * pc.s, V + kQuad * pc.s,
                                 O ? O + kQuad * pc.o : nullptr, pc.g + t0 + lane, t0, lane, c);
}

// Any alignment, one element per thread: heads and tails of vector bodies,
// and runs whose buffers cannot be aligned together.
template <typename GT, bool POW2>
__global__ __launch_bounds__(kBlock) void step_scalar_kernel(GradSet<ZERO_MAX_RANKS> gs, int n,
                                                            float *__restrict__ W,
                                                            float *__restrict__ M,
                                                            float *__restrict__ V,
                                                            uint16_t *__restrict__ O,
                                                            int64_t len, StepConsts c)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    const float clip = c.clip_dev ? *c.clip_dev : c.clip;
    if (c.clip_dev && !(clip == clip))  // skipped step, as in the quad kernel
        return;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < len; i += stride) {
        float s = grad_at<GT>(gs.p[0], i);
        for (int q = 1; q < n; ++q)
            s = s + grad_at<GT>(gs.p[q], i);
        float g = average<POW2>(s, c);
        g = g * clip;
        float w = W[i], m = M[i], v = V[i];
        adamw(g, w, m, v, c);
        W[i] = w;
        M[i] = m;
        V[i] = v;
        if (O)
            O[i] = to_bf16(w);
    }
}

int scalar_grid(int64_t len)
{
    int cus = device_cu_count();
    if (cus <= 0)
        cus = 256;
    int64_t g = (len + kBlock - 1) / kBlock;
    const int64_t cap = (int64_t)cus * 8;
    if (g > cap)
        g = cap;
    return g < 1 ? 1 : (int)g;
}

// Launch the quad kernel over nquads quads, in launches of at most
// kMaxQuadsPerLaunch quads (the dispatch grid size is 32-bit).
template <int NR, typename QD, bool POW2>
hipError_t launch_quads_nr(const void *const *grads, int n, int gsize_quad, float *w, float *m,
                           float *v, uint16_t *o, int64_t nquads, const StepConsts &c,
                           hipStream_t st, int waves = -1)
{
    constexpr int CAP = NR > 0 ? NR : ZERO_MAX_RANKS;
    const size_t lds =
        occupancy_cap_lds(waves >= 0 ? waves : step_waves_per_cu(n, NR == 0, gsize_quad / kQuad), 0);
    for (int64_t q0 = 0; q0 < nquads; q0 += kMaxQuadsPerLaunch) {
        const int64_t nq = nquads - q0 < kMaxQuadsPerLaunch ? nquads - q0 : kMaxQuadsPerLaunch;
        GradSet<CAP> gs{};
        for (int q = 0; q < n; ++q)
            gs.p[q] = static_cast<const char *>(grads[q]) + q0 * gsize_quad;
        const unsigned blocks = (unsigned)((nq + kWave - 1) / kWave);
        hipLaunchKernelGGL((step_quad_kernel<NR, CAP, QD, POW2>), dim3(blocks), dim3(kWave), lds, st,
                           gs, n, w + q0 * kQuad, m + q0 * kQuad, v + q0 * kQuad,
                           o ? o + q0 * kQuad : nullptr, nq, c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// bf16 gradients: a kernel compiled for each rank count up to
// kMaxCompiledRanks and for 64 (all N loads of a lane issued in batches of
// 16, none predicated), the run-time kernel for any other N.
template <bool POW2, int... Ks>
hipError_t bf16_quads_compiled(std::integer_sequence<int, Ks...>, const void *const *grads, int n,
                               float *w, float *m, float *v, uint16_t *o, int64_t nq,
                               const StepConsts &c, hipStream_t st)
{
    using QD = Bf16Quad;
    constexpr int B = 8;  // bytes of one bf16 quad
    hipError_t r = hipSuccess;
    const bool hit =
        ((n == Ks + 1 ? (r = launch_quads_nr<Ks + 1, QD, POW2>(grads, n, B, w, m, v, o, nq, c, st),
                         true)
                      : false) ||
         ...);
    if (hit)
        return r;
    if (n == 64)
        return launch_quads_nr<64, QD, POW2>(grads, n, B, w, m, v, o, nq, c, st);
    return launch_quads_nr<0, QD, POW2>(grads, n, B, w, m, v, o, nq, c, st);
}

template <bool POW2>
hipError_t launch_bf16_quads(const void *const *grads, int n, float *w, float *m, float *v,
                             uint16_t *o, int64_t nq, const StepConsts &c, hipStream_t st)
{
    return bf16_quads_compiled<POW2>(std::make_integer_sequence<int, kMaxCompiledRanks>{}, grads,
                                     n, w, m, v, o, nq, c, st);
}

// fp32 gradients (a reduce dtype of fp32): kernels compiled for the
// power-of-two rank counts up to 32, the run-time kernel for any other N.
template <bool POW2>
hipError_t launch_f32_quads(const void *const *grads, int n, float *w, float *m, float *v,
                            uint16_t *o, int64_t nq, const StepConsts &c, hipStream_t st)
{
    using QD = F32Quad;
    constexpr int B = 16;  // bytes of one fp32 quad
    switch (n) {
    case 2: return launch_quads_nr<2, QD, POW2>(grads, n, B, w, m, v, o, nq, c, st);
    case 4: return launch_quads_nr<4, QD, POW2>(grads, n, B, w, m, v, o, nq, c, st);
    case 8: return launch_quads_nr<8, QD, POW2>(grads, n, B, w, m, v, o, nq, c, st);
    case 16: return launch_quads_nr<16, QD, POW2>(grads, n, B, w, m, v, o, nq, c, st);
    case 32: return launch_quads_nr<32, QD, POW2>(grads, n, B, w, m, v, o, nq, c, st);
    default: return launch_quads_nr<0, QD, POW2>(grads, n, B, w, m, v, o, nq, c, st);
    }
}

template <typename GT, bool POW2>
hipError_t launch_scalar(const void *const *grads, int n, float *w, float *m, float *v,
                         uint16_t *o, int64_t len, const StepConsts &c, hipStream_t st)
{
    GradSet<ZERO_MAX_RANKS> gs{};
    for (int q = 0; q < n; ++q)
        gs.p[q] = grads[q];
    hipLaunchKernelGGL((step_scalar_kernel<GT, POW2>), dim3(scalar_grid(len)), dim3(kBlock), 0, st,
                       gs, n, w, m, v, o, len, c);
    return hipGetLastError();
}

// ---- several vector pieces per launch ----------------------------------

// The group table of a batch of `total` blocks.
void fill_step_groups(StepBatch &b, uint32_t total)
{
    int first_piece = 0, last_piece = 0;
    for (uint32_t g = 0; g < (uint32_t)kStepGroups; ++g) {
        const uint32_t a = g << kStepGroupShift;
        if (a >= total)
            break;
        const uint32_t z =
            std::min<uint64_t>((uint64_t)a + (1u << kStepGroupShift) - 1u, total - 1u);
        while (b.end[first_piece] <= a)
            ++first_piece;
        if (last_piece < first_piece)
            last_piece = first_piece;
        while (b.end[last_piece] <= z)
            ++last_piece;
        const uint32_t entry = (uint32_t)first_piece | (first_piece == last_piece ? 0x80u : 0u);
        b.group[g >> 2] |= entry << ((g & 3u) * 8u);
    }
}

// The batches of the vector pieces pcs[0..count), in order: at most
// kStepPieces pieces and kStepBatchBlocks blocks each, a longer piece cut at
// whole waves.  Offsets in quads (the caller checked that every base is
// quad-aligned, so every vector piece's offsets are whole quads).
std::vector<std::pair<StepBatch, uint32_t>> step_batches(const Piece *pcs, int count)
{
    std::vector<std::pair<StepBatch, uint32_t>> out;
    StepBatch b{};
    uint32_t blocks = 0;
    auto flush = [&]() {
        if (b.n_pieces == 0)
            return;
        fill_step_groups(b, blocks);
        out.emplace_back(b, blocks);
        b = StepBatch{};
        blocks = 0;
    };
    constexpr int64_t kMaxQuads = (kStepBatchBlocks - 1) * kWave;  // < 2^24
    for (int k = 0; k < count; ++k) {
        int64_t g = pcs[k].g_off / kQuad, st = pcs[k].s_off / kQuad, o = pcs[k].o_off / kQuad;
        int phase = pcs[k].phase;
        for (int64_t left = pcs[k].len / kQuad; left > 0;) {
            // a cut leaves the next part on the same wave grid, at phase 0
            const int64_t nq = std::min(left, kMaxQuads - phase);
            const uint32_t nb = (uint32_t)((nq + phase + kWave - 1) / kWave);
            if (b.n_pieces == kStepPieces || (int64_t)blocks + nb > kStepBatchBlocks)
                flush();
            QuadPiece &q = b.p[b.n_pieces];
            q.g = g;
            q.s = st;
            q.o = o;
            q.nq_phase = (uint32_t)nq | ((uint32_t)phase << 24);
            q.first = blocks;
            blocks += nb;
            b.end[b.n_pieces] = blocks;
            ++b.n_pieces;
            g += nq;
            st += nq;
            o += nq;
            left -= nq;
            phase = 0;
        }
    }
    flush();
    return out;
}

template <int NR, typename QD, bool POW2>
hipError_t launch_batch_nr(const Piece *pcs, int count, const void *const *grads, int n, float *w,
                           float *m, float *v, uint16_t *o, const StepConsts &c, hipStream_t st,
                           int waves)
{
    GradSet<NR> gs{};
    for (int q = 0; q < n; ++q)
        gs.p[q] = grads[q];
    const size_t lds = occupancy_cap_lds(
        waves >= 0 ? waves : step_waves_per_cu(n, false, QD::kBytes / kQuad), 0);
    for (const auto &bb : step_batches(pcs, count)) {
        hipLaunchKernelGGL((step_batch_kernel<NR, NR, QD, POW2>), dim3(bb.second), dim3(kWave), lds,
                           st, gs, n, w, m, v, o, bb.first, c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <bool POW2, int... Ks>
hipError_t bf16_batch_compiled(std::integer_sequence<int, Ks...>, const Piece *pcs, int count,
                               const void *const *grads, int n, float *w, float *m, float *v,
                               uint16_t *o, const StepConsts &c, hipStream_t st)
{
    hipError_t r = hipErrorNotSupported;
    const bool hit =
        ((n == Ks + 1
              ? (r = launch_batch_nr<Ks + 1, Bf16Quad, POW2>(pcs, count, grads, n, w, m, v, o, c, st,
                                                             -1),
                 true)
              : false) ||
         ...);
    if (!hit && n == 64)
        r = launch_batch_nr<64, Bf16Quad, POW2>(pcs, count, grads, n, w, m, v, o, c, st, -1);
    return r;
}

template <bool POW2>
hipError_t launch_batch(const Piece *pcs, int count, const void *const *grads, int n, bool bf,
                        float *w, float *m, float *v, uint16_t *o, const StepConsts &c,
                        hipStream_t st, int waves)
{
    if (bf)
        return bf16_batch_compiled<POW2>(std::make_integer_sequence<int, kMaxCompiledRanks>{}, pcs,
                                         count, grads, n, w, m, v, o, c, st);
    using QD = F32Quad;
    switch (n) {
    case 1:
        return launch_batch_nr<1, QD, POW2>(pcs, count, grads, n, w, m, v, o, c, st,
                                            waves >= 0 ? waves : step1_waves_per_cu(false));
    case 2: return launch_batch_nr<2, QD, POW2>(pcs, count, grads, n, w, m, v, o, c, st, -1);
    case 4: return launch_batch_nr<4, QD, POW2>(pcs, count, grads, n, w, m, v, o, c, st, -1);
    case 8: return launch_batch_nr<8, QD, POW2>(pcs, count, grads, n, w, m, v, o, c, st, -1);
    case 16: return launch_batch_nr<16, QD, POW2>(pcs, count, grads, n, w, m, v, o, c, st, -1);
    case 32: return launch_batch_nr<32, QD, POW2>(pcs, count, grads, n, w, m, v, o, c, st, -1);
    default: return hipErrorNotSupported;
    }
}

}  // namespace

int launch_step_piece(const Piece &pc, const void *const *grads, int n_grads, int grad_dtype,
                      float *w, float *m, float *v, uint16_t *out, const StepConsts &c,
                      void *stream, int waves_per_cu)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const bool bf = grad_dtype == ZERO_BF16;
    const bool p2 = c.div_pow2 != 0;
    if (pc.vec) {
        const int64_t nq = pc.len / kQuad;
        if (bf)
            return p2 ? launch_bf16_quads<true>(grads, n_grads, w, m, v, out, nq, c, st)
                      : launch_bf16_quads<false>(grads, n_grads, w, m, v, out, nq, c, st);
        if (n_grads == 1) {  // one reduced gradient, e.g. the clipped step after the norm pass
            const int wv = waves_per_cu >= 0 ? waves_per_cu : step1_waves_per_cu(false);
            return p2 ? launch_quads_nr<1, F32Quad, true>(grads, n_grads, 16, w, m, v, out, nq, c,
                                                          st, wv)
                      : launch_quads_nr<1, F32Quad, false>(grads, n_grads, 16, w, m, v, out, nq, c,
                                                           st, wv);
        }
        return p2 ? launch_f32_quads<true>(grads, n_grads, w, m, v, out, nq, c, st)
                  : launch_f32_quads<false>(grads, n_grads, w, m, v, out, nq, c, st);
    }
    if (bf)
        return p2 ? launch_scalar<uint16_t, true>(grads, n_grads, w, m, v, out, pc.len, c, st)
                  : launch_scalar<uint16_t, false>(grads, n_grads, w, m, v, out, pc.len, c, st);
    return p2 ? launch_scalar<float, true>(grads, n_grads, w, m, v, out, pc.len, c, st)
              : launch_scalar<float, false>(grads, n_grads, w, m, v, out, pc.len, c, st);
}

int launch_step_batch(const Piece *pcs, int count, const void *const *grads, int n_grads,
                      int grad_dtype, float *w, float *m, float *v, uint16_t *out,
                      const StepConsts &c, void *stream, int waves_per_cu)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const bool bf = grad_dtype == ZERO_BF16;
    return c.div_pow2 ? launch_batch<true>(pcs, count, grads, n_grads, bf, w, m, v, out, c, st,
                                           waves_per_cu)
                      : launch_batch<false>(pcs, count, grads, n_grads, bf, w, m, v, out, c, st,
                                            waves_per_cu);
}

}  // namespace zero
