// step_kernels.hip -- the fused sharded optimizer step for gfx950.
//
// One pass over a rank's shard (or every rank's shards) does, per element:
// the rank-ordered binary32 sum of the N ranks' gradients (the reduction half
// of the reduce-scatter), the average, the clip scale, AdamW on the fp32
// master / m / v, and the bf16 cast into the all-gather's output slot
// ("ZeRO and FSDP sharding", How it works and Code).
//
// The work is elementwise and streams every byte once, so the kernel is bound
// by HBM bandwidth, not arithmetic: no MFMA, no LDS.  Each thread owns chunks
// of 8 consecutive elements: one 16-byte load per rank for bf16 gradients,
// two 16-byte loads / stores per fp32 state array and one 16-byte store of
// 8 bf16 outputs.  Workgroups walk the chunks grid-stride, with the grid sized
// to a fixed number of workgroups per compute unit.
#include <cstdlib>

#include "device_common.h"

namespace zero {
namespace {

using namespace dev;

template <int NR, int CAP, typename CH, bool POW2>
__global__ __launch_bounds__(kBlock) void step_vec_kernel(GradSet<CAP> gs, int n,
                                                         float *__restrict__ W,
                                                         float *__restrict__ M,
                                                         float *__restrict__ V,
                                                         uint16_t *__restrict__ O,
                                                         int64_t nchunks, StepConsts c)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < nchunks; i += stride) {
        f32x4 *w4 = reinterpret_cast<f32x4 *>(W) + 2 * i;
        f32x4 *m4 = reinterpret_cast<f32x4 *>(M) + 2 * i;
        f32x4 *v4 = reinterpret_cast<f32x4 *>(V) + 2 * i;
        const f32x4 wa = ld_stream(w4), wb = ld_stream(w4 + 1);
        const f32x4 ma = ld_stream(m4), mb = ld_stream(m4 + 1);
        const f32x4 va = ld_stream(v4), vb = ld_stream(v4 + 1);

        float s[8];
        rank_sum<NR, CAP, CH>(gs, n, i, s);

        float w[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
        float m[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
        float v[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float g = average<POW2>(s[k], c);
            g = g * c.clip;
            adamw(g, w[k], m[k], v[k], c);
        }
        st_stream(f32x4{w[0], w[1], w[2], w[3]}, w4);
        st_stream(f32x4{w[4], w[5], w[6], w[7]}, w4 + 1);
        st_stream(f32x4{m[0], m[1], m[2], m[3]}, m4);
        st_stream(f32x4{m[4], m[5], m[6], m[7]}, m4 + 1);
        st_stream(f32x4{v[0], v[1], v[2], v[3]}, v4);
        st_stream(f32x4{v[4], v[5], v[6], v[7]}, v4 + 1);
        if (O) {
            const u32x4 o = {pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]),
                             pack_bf16x2(w[4], w[5]), pack_bf16x2(w[6], w[7])};
            st_stream(o, reinterpret_cast<u32x4 *>(O) + i);
        }
    }
}

// Any alignment, one element per thread: heads and tails of vector bodies,
// and runs whose buffers cannot be 16-byte aligned together.
template <typename GT, bool POW2>
__global__ __launch_bounds__(kBlock) void step_scalar_kernel(GradSet<ZERO_MAX_RANKS> gs, int n,
                                                            float *__restrict__ W,
                                                            float *__restrict__ M,
                                                            float *__restrict__ V,
                                                            uint16_t *__restrict__ O,
                                                            int64_t len, StepConsts c)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < len; i += stride) {
        float s = grad_at<GT>(gs.p[0], i);
        for (int q = 1; q < n; ++q)
            s = s + grad_at<GT>(gs.p[q], i);
        float g = average<POW2>(s, c);
        g = g * c.clip;
        float w = W[i], m = M[i], v = V[i];
        adamw(g, w, m, v, c);
        W[i] = w;
        M[i] = m;
        V[i] = v;
        if (O)
            O[i] = to_bf16(w);
    }
}

int g_blocks_per_cu = -1;

int blocks_per_cu()
{
    if (g_blocks_per_cu < 0) {
        // Workgroups resident per compute unit for the streaming kernels;
        // ZERO_STEP_BLOCKS_PER_CU overrides it for launch-shape sweeps.
        int v = 8;
        if (const char *e = std::getenv("ZERO_STEP_BLOCKS_PER_CU")) {
            int x = std::atoi(e);
            if (x >= 1 && x <= 64)
                v = x;
        }
        g_blocks_per_cu = v;
    }
    return g_blocks_per_cu;
}

int64_t grid_for(int64_t work_items)
{
    int cus = device_cu_count();
    if (cus <= 0)
        cus = 256;
    int64_t g = (work_items + kBlock - 1) / kBlock;
    const int64_t cap = (int64_t)cus * blocks_per_cu();
    if (g > cap)
        g = cap;
    return g < 1 ? 1 : g;
}

template <int NR, typename CH, bool POW2>
hipError_t launch_vec_nr(const void *const *grads, int n, float *w, float *m, float *v,
                         uint16_t *o, int64_t nchunks, const StepConsts &c, hipStream_t st)
{
    constexpr int CAP = NR > 0 ? NR : ZERO_MAX_RANKS;
    GradSet<CAP> gs{};
    for (int q = 0; q < n; ++q)
        gs.p[q] = grads[q];
    const int64_t grid = grid_for(nchunks);
    hipLaunchKernelGGL((step_vec_kernel<NR, CAP, CH, POW2>), dim3((unsigned)grid), dim3(kBlock), 0,
                       st, gs, n, w, m, v, o, nchunks, c);
    return hipGetLastError();
}

template <typename CH, bool POW2>
hipError_t launch_vec(const void *const *grads, int n, float *w, float *m, float *v, uint16_t *o,
                      int64_t nchunks, const StepConsts &c, hipStream_t st)
{
    switch (n) {
    case 1: return launch_vec_nr<1, CH, POW2>(grads, n, w, m, v, o, nchunks, c, st);
    case 2: return launch_vec_nr<2, CH, POW2>(grads, n, w, m, v, o, nchunks, c, st);
    case 4: return launch_vec_nr<4, CH, POW2>(grads, n, w, m, v, o, nchunks, c, st);
    case 8: return launch_vec_nr<8, CH, POW2>(grads, n, w, m, v, o, nchunks, c, st);
    case 16: return launch_vec_nr<16, CH, POW2>(grads, n, w, m, v, o, nchunks, c, st);
    case 32: return launch_vec_nr<32, CH, POW2>(grads, n, w, m, v, o, nchunks, c, st);
    case 64: return launch_vec_nr<64, CH, POW2>(grads, n, w, m, v, o, nchunks, c, st);
    default: return launch_vec_nr<0, CH, POW2>(grads, n, w, m, v, o, nchunks, c, st);
    }
}

template <typename GT, bool POW2>
hipError_t launch_scalar(const void *const *grads, int n, float *w, float *m, float *v,
                         uint16_t *o, int64_t len, const StepConsts &c, hipStream_t st)
{
    GradSet<ZERO_MAX_RANKS> gs{};
    for (int q = 0; q < n; ++q)
        gs.p[q] = grads[q];
    hipLaunchKernelGGL((step_scalar_kernel<GT, POW2>), dim3((unsigned)grid_for(len)), dim3(kBlock),
                       0, st, gs, n, w, m, v, o, len, c);
    return hipGetLastError();
}

}  // namespace

int launch_step_piece(const Piece &pc, const void *const *grads, int n_grads, int grad_dtype,
                      float *w, float *m, float *v, uint16_t *out, const StepConsts &c,
                      void *stream)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const bool bf = grad_dtype == ZERO_BF16;
    if (pc.vec) {
        const int64_t nchunks = pc.len / kChunk;
        if (bf)
            return c.div_pow2 ? launch_vec<Bf16Chunk, true>(grads, n_grads, w, m, v, out, nchunks, c, st)
                              : launch_vec<Bf16Chunk, false>(grads, n_grads, w, m, v, out, nchunks, c, st);
        return c.div_pow2
                   ? launch_vec_nr<0, F32Chunk, true>(grads, n_grads, w, m, v, out, nchunks, c, st)
                   : launch_vec_nr<0, F32Chunk, false>(grads, n_grads, w, m, v, out, nchunks, c, st);
    }
    if (bf)
        return c.div_pow2 ? launch_scalar<uint16_t, true>(grads, n_grads, w, m, v, out, pc.len, c, st)
                          : launch_scalar<uint16_t, false>(grads, n_grads, w, m, v, out, pc.len, c, st);
    return c.div_pow2 ? launch_scalar<float, true>(grads, n_grads, w, m, v, out, pc.len, c, st)
                      : launch_scalar<float, false>(grads, n_grads, w, m, v, out, pc.len, c, st);
}

}  // namespace zero
