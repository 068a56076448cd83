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
#include <utility>

#include "device_common.h"

namespace zero {
namespace {

using namespace dev;

template <int NR, int CAP, typename QD, bool POW2>
__global__ __launch_bounds__(kWave) void step_quad_kernel(GradSet<CAP> gs, int n,
                                                         float *__restrict__ W,
                                                         float *__restrict__ M,
                                                         float *__restrict__ V,
                                                         uint16_t *__restrict__ O,
                                                         int64_t nquads, StepConsts c)
{
    const int64_t i = (int64_t)blockIdx.x * kWave + threadIdx.x;  // quad index
    if (i >= nquads)
        return;
    f32x4 *w4 = reinterpret_cast<f32x4 *>(W) + i;
    f32x4 *m4 = reinterpret_cast<f32x4 *>(M) + i;
    f32x4 *v4 = reinterpret_cast<f32x4 *>(V) + i;

    float s[4];
    rank_sum<NR, CAP, QD>(gs, n, i, s);
    const f32x4 wq = ld_stream(w4), mq = ld_stream(m4), vq = ld_stream(v4);
    const float clip = c.clip_dev ? *c.clip_dev : c.clip;  // uniform: one scalar load

    float w[4] = {wq.x, wq.y, wq.z, wq.w};
    float m[4] = {mq.x, mq.y, mq.z, mq.w};
    float v[4] = {vq.x, vq.y, vq.z, vq.w};
    // a NaN multiplier from the device (the norm was not finite): the step is
    // skipped and the state left as it is (uniform over the launch)
    if (c.clip_dev && !(clip == clip))
        return;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float g = average<POW2>(s[k], c);
        g = g * clip;
        adamw(g, w[k], m[k], v[k], c);
    }
    // whole-span stores of the wave's tile (lanes past nquads returned above)
    const int64_t t0 = (int64_t)blockIdx.x * kWave;
    const int lane = threadIdx.x;
    st_span(f32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<f32x4 *>(W) + t0, lane);
    st_span(f32x4{m[0], m[1], m[2], m[3]}, reinterpret_cast<f32x4 *>(M) + t0, lane);
    st_span(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(V) + t0, lane);
    if (O)
        st_span(u32x2{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3])},
                reinterpret_cast<u32x2 *>(O) + t0, lane);
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

}  // namespace zero
