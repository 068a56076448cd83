// norm_kernels.hip -- two-stage sum of squares for global grad-norm clipping.
//
// "ZeRO and FSDP sharding", Implementation notes: clipping needs the global
// norm, i.e. the summed squared norms of the shards (then all-reduced across
// ranks).  "ZeRO: Three Ledgers", section 2: a norm is a decomposable
// reduction costing O(1) scalars per rank.
//
// Stage 1 fuses the reduction half of the reduce-scatter with the sum of
// squares: each thread forms g = (rank-ordered sum) / divisor for its chunks,
// optionally writes g (fp32) so the step can read one reduced gradient instead
// of N, and accumulates g^2 in binary64.  Each workgroup reduces its threads in
// a fixed order (wave64 butterfly, then the four waves in order) to one
// partial.  Stage 2 is one workgroup summing the partials in a fixed order.
// The partition (grid size and chunk assignment) depends only on the element
// count, never on the device, so the result is bitwise reproducible.
#include "device_common.h"

namespace zero {
namespace {

using namespace dev;

template <int NR, int CAP, typename CH, bool POW2>
__global__ __launch_bounds__(kBlock) void norm_vec_kernel(GradSet<CAP> gs, int n,
                                                         float *__restrict__ G, int64_t nchunks,
                                                         StepConsts c,
                                                         double *__restrict__ partials)
{
    double acc = 0.0;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < nchunks; i += stride) {
        float s[8];
        rank_sum<NR, CAP, CH>(gs, n, i, s);
        float g[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            g[k] = average<POW2>(s[k], c);
        if (G) {
            f32x4 *g4 = reinterpret_cast<f32x4 *>(G) + 2 * i;
            st_stream(f32x4{g[0], g[1], g[2], g[3]}, g4);
            st_stream(f32x4{g[4], g[5], g[6], g[7]}, g4 + 1);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const double x = (double)g[k];
            acc = acc + x * x;
        }
    }
    const double t = block_sum(acc);
    if (threadIdx.x == 0)
        partials[blockIdx.x] = t;
}

template <typename GT, bool POW2>
__global__ __launch_bounds__(kBlock) void norm_scalar_kernel(GradSet<ZERO_MAX_RANKS> gs, int n,
                                                            float *__restrict__ G, int64_t len,
                                                            StepConsts c,
                                                            double *__restrict__ partials)
{
    double acc = 0.0;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < len; i += stride) {
        float s = grad_at<GT>(gs.p[0], i);
        for (int q = 1; q < n; ++q)
            s = s + grad_at<GT>(gs.p[q], i);
        const float g = average<POW2>(s, c);
        if (G)
            G[i] = g;
        const double x = (double)g;
        acc = acc + x * x;
    }
    const double t = block_sum(acc);
    if (threadIdx.x == 0)
        partials[blockIdx.x] = t;
}

__global__ __launch_bounds__(kBlock) void norm_final_kernel(const double *__restrict__ partials,
                                                           int n, double *__restrict__ out)
{
    double acc = 0.0;
    for (int i = threadIdx.x; i < n; i += kBlock)
        acc = acc + partials[i];
    const double t = block_sum(acc);
    if (threadIdx.x == 0)
        *out = t;
}

int blocks_for(int64_t items)
{
    int64_t b = (items + kBlock - 1) / kBlock;
    if (b > kNormMaxBlocks)
        b = kNormMaxBlocks;
    return b < 1 ? 1 : (int)b;
}

template <int NR, typename CH, bool POW2>
hipError_t launch_norm_vec_nr(const void *const *grads, int n, float *G, int64_t nchunks,
                              const StepConsts &c, double *partials, int blocks, hipStream_t st)
{
    constexpr int CAP = NR > 0 ? NR : ZERO_MAX_RANKS;
    GradSet<CAP> gs{};
    for (int q = 0; q < n; ++q)
        gs.p[q] = grads[q];
    hipLaunchKernelGGL((norm_vec_kernel<NR, CAP, CH, POW2>), dim3(blocks), dim3(kBlock), 0, st, gs,
                       n, G, nchunks, c, partials);
    return hipGetLastError();
}

template <typename CH, bool POW2>
hipError_t launch_norm_vec(const void *const *grads, int n, float *G, int64_t nchunks,
                           const StepConsts &c, double *partials, int blocks, hipStream_t st)
{
    switch (n) {
    case 1: return launch_norm_vec_nr<1, CH, POW2>(grads, n, G, nchunks, c, partials, blocks, st);
    case 2: return launch_norm_vec_nr<2, CH, POW2>(grads, n, G, nchunks, c, partials, blocks, st);
    case 4: return launch_norm_vec_nr<4, CH, POW2>(grads, n, G, nchunks, c, partials, blocks, st);
    case 8: return launch_norm_vec_nr<8, CH, POW2>(grads, n, G, nchunks, c, partials, blocks, st);
    case 16: return launch_norm_vec_nr<16, CH, POW2>(grads, n, G, nchunks, c, partials, blocks, st);
    case 32: return launch_norm_vec_nr<32, CH, POW2>(grads, n, G, nchunks, c, partials, blocks, st);
    case 64: return launch_norm_vec_nr<64, CH, POW2>(grads, n, G, nchunks, c, partials, blocks, st);
    default: return launch_norm_vec_nr<0, CH, POW2>(grads, n, G, nchunks, c, partials, blocks, st);
    }
}

template <typename GT, bool POW2>
hipError_t launch_norm_scalar(const void *const *grads, int n, float *G, int64_t len,
                              const StepConsts &c, double *partials, int blocks, hipStream_t st)
{
    GradSet<ZERO_MAX_RANKS> gs{};
    for (int q = 0; q < n; ++q)
        gs.p[q] = grads[q];
    hipLaunchKernelGGL((norm_scalar_kernel<GT, POW2>), dim3(blocks), dim3(kBlock), 0, st, gs, n, G,
                       len, c, partials);
    return hipGetLastError();
}

}  // namespace

int norm_piece_blocks(const Piece &pc)
{
    return blocks_for(pc.vec ? pc.len / kChunk : pc.len);
}

int launch_norm_piece(const Piece &pc, const void *const *grads, int n_grads, int grad_dtype,
                      float *g_out, const StepConsts &c, double *partials, int *n_partials,
                      void *stream)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int blocks = norm_piece_blocks(pc);
    *n_partials = blocks;
    const bool bf = grad_dtype == ZERO_BF16;
    if (pc.vec) {
        const int64_t nchunks = pc.len / kChunk;
        if (bf)
            return c.div_pow2
                       ? launch_norm_vec<Bf16Chunk, true>(grads, n_grads, g_out, nchunks, c, partials, blocks, st)
                       : launch_norm_vec<Bf16Chunk, false>(grads, n_grads, g_out, nchunks, c, partials, blocks, st);
        return c.div_pow2
                   ? launch_norm_vec_nr<0, F32Chunk, true>(grads, n_grads, g_out, nchunks, c, partials, blocks, st)
                   : launch_norm_vec_nr<0, F32Chunk, false>(grads, n_grads, g_out, nchunks, c, partials, blocks, st);
    }
    if (bf)
        return c.div_pow2
                   ? launch_norm_scalar<uint16_t, true>(grads, n_grads, g_out, pc.len, c, partials, blocks, st)
                   : launch_norm_scalar<uint16_t, false>(grads, n_grads, g_out, pc.len, c, partials, blocks, st);
    return c.div_pow2
               ? launch_norm_scalar<float, true>(grads, n_grads, g_out, pc.len, c, partials, blocks, st)
               : launch_norm_scalar<float, false>(grads, n_grads, g_out, pc.len, c, partials, blocks, st);
}

int launch_norm_final(const double *partials, int n_partials, double *result, void *stream)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(norm_final_kernel, dim3(1), dim3(kBlock), 0, st, partials, n_partials,
                       result);
    return hipGetLastError();
}

}  // namespace zero
