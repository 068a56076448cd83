// stage_kernels.hip -- the first half of the staged step: the reduction half
// of the reduce-scatter for one chunk of elements, written to a workspace
// that the second half (the fused step with one reduced gradient) reads back
// ("ZeRO and FSDP sharding", Code: the reduce-scatter's average, then AdamW
// on the local slice).
//
// Why split what the fused step does in one pass: at large N the fused step
// keeps N + 7 streams live -- N gradient reads next to three state reads and
// four writes -- and MI355X streams that mix well below a plain copy (0.86 of
// it at N = 64).  Split by chunks, the first kernel is a pure N-stream
// reduction (the norm pass's mix, 0.93 of a copy) and the second a small
// 4-read / 4-write mix.  A chunk's reduced gradient (up to 32M elements, 128
// MB of fp32, within MI355X's 256 MB memory-side cache) is written with the
// device-scope, non-streaming store policy and read back by the next kernel.
// Measured at N = 64 (2^27-element shard): 78.2-78.5 % of 8 TB/s with chunks
// of 32M or 64M elements, 76.0 % with one 512 MB chunk (larger than the
// cache), 74.7 % fused: the split mix gains about 1.3 points and the
// cache-sized chunk, which keeps most of the round trip out of HBM, the rest.
// The stores with the streaming bit too lost 2 points.
//
// The arithmetic is the fused step's, split at a point where the value is
// stored in binary32 and read back unchanged: g = (rank-ordered binary32
// sum) / N here, then g * clip and AdamW in the step kernel (divisor 1), so
// every element gets the same bits as from zero_step.
#include "device_common.h"

namespace zero {
namespace {

using namespace dev;

// One 512-element tile per wave64 workgroup, lane l owning one oct of it, as
// in the norm pass: elements 8l .. 8l+7 for bf16 gradients (one 16-byte
// load per rank), whose g goes through LDS so the wave stores it as two
// contiguous 1 KiB spans; elements 4l .. 4l+3 and 256+4l .. +3 for fp32
// gradients (two 1 KiB loads per rank), whose g the wave stores as it is.  VEC: the gradients are 16-byte aligned at the chunk start (the
// workspace always is); the last, partial tile and unaligned chunks go
// element by element.
template <int NR, int CAP, typename GT, typename OD, bool POW2, bool VEC>
__global__ __launch_bounds__(kWave) void stage_reduce_kernel(GradSet<CAP> gs, int n,
                                                            float *__restrict__ G, int64_t len,
                                                            StepConsts c)
{
    static_assert(OD::kN == kOct, "one oct per lane");
    __shared__ f32x4 xg[2 * kWave];
    const int64_t tile = blockIdx.x;
    const int lane = threadIdx.x;
    if (VEC && (tile + 1) * kNormSpan <= len) {  // uniform over the workgroup
        float s[kOct];
        rank_sum<NR, CAP, OD>(gs, n, tile * kWave + lane, s);
        float g[kOct];
#pragma unroll
        for (int k = 0; k < kOct; ++k)
            g[k] = average<POW2>(s[k], c);
        f32x4 *t4 = reinterpret_cast<f32x4 *>(G) + tile * (2 * kWave);
        if constexpr (OD::kBytes == 32) {  // fp32: the lane holds quads l and 64 + l
            st_span<f32x4, kKeepStorePolicy>(f32x4{g[0], g[1], g[2], g[3]}, t4, lane);
            st_span<f32x4, kKeepStorePolicy>(f32x4{g[4], g[5], g[6], g[7]}, t4 + kWave, lane);
        } else {
            xg[2 * lane] = f32x4{g[0], g[1], g[2], g[3]};
            xg[2 * lane + 1] = f32x4{g[4], g[5], g[6], g[7]};
            __syncthreads();
            st_span<f32x4, kKeepStorePolicy>(xg[lane], t4, lane);
            st_span<f32x4, kKeepStorePolicy>(xg[kWave + lane], t4 + kWave, lane);
        }
    } else {
        const int64_t e0 = tile * kNormSpan + (int64_t)lane * kOct;
#pragma unroll
        for (int k = 0; k < kOct; ++k) {
            if (e0 + k < len) {
                float s = grad_at<GT>(gs.p[0], e0 + k);
                for (int q = 1; q < n; ++q)
                    s = s + grad_at<GT>(gs.p[q], e0 + k);
                G[e0 + k] = average<POW2>(s, c);
            }
        }
    }
}

template <int NR, typename GT, typename OD, bool POW2, bool VEC>
hipError_t launch_nr(const void *const *grads, int n, float *G, int64_t len, const StepConsts &c,
                     hipStream_t st)
{
    constexpr int CAP = NR > 0 ? NR : ZERO_MAX_RANKS;
    GradSet<CAP> gs{};
    for (int q = 0; q < n; ++q)
        gs.p[q] = grads[q];
    const int64_t blocks = (len + kNormSpan - 1) / kNormSpan;
    const size_t lds = occupancy_cap_lds(norm_waves_per_cu(n, NR == 0, (int)sizeof(GT)),
                                         2 * kWave * sizeof(f32x4));
    hipLaunchKernelGGL((stage_reduce_kernel<NR, CAP, GT, OD, POW2, VEC>), dim3((unsigned)blocks),
                       dim3(kWave), lds, st, gs, n, G, len, c);
    return hipGetLastError();
}

template <bool POW2>
hipError_t launch_bf16_vec(const void *const *grads, int n, float *G, int64_t len,
                           const StepConsts &c, hipStream_t st)
{
    using T = uint16_t;
    using OD = Bf16Oct;
    switch (n) {
    case 32: return launch_nr<32, T, OD, POW2, true>(grads, n, G, len, c, st);
    case 64: return launch_nr<64, T, OD, POW2, true>(grads, n, G, len, c, st);
    default: return launch_nr<0, T, OD, POW2, true>(grads, n, G, len, c, st);
    }
}

}  // namespace

int launch_stage_reduce(int64_t len, bool vec, const void *const *grads, int n_grads,
                        int grad_dtype, float *g_out, const StepConsts &c, void *stream)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (len <= 0)
        return hipSuccess;
    if ((len + kNormSpan - 1) / kNormSpan > 0xffffffffLL / kWave)
        return hipErrorInvalidValue;  // larger than one dispatch can address
    const bool bf = grad_dtype == ZERO_BF16;
    const bool p2 = c.div_pow2 != 0;
    if (bf && vec)
        return p2 ? launch_bf16_vec<true>(grads, n_grads, g_out, len, c, st)
                  : launch_bf16_vec<false>(grads, n_grads, g_out, len, c, st);
    if (bf)
        return p2 ? launch_nr<0, uint16_t, Bf16Oct, true, false>(grads, n_grads, g_out, len, c, st)
                  : launch_nr<0, uint16_t, Bf16Oct, false, false>(grads, n_grads, g_out, len, c, st);
    if (vec)
        return p2 ? launch_nr<0, float, F32Oct, true, true>(grads, n_grads, g_out, len, c, st)
                  : launch_nr<0, float, F32Oct, false, true>(grads, n_grads, g_out, len, c, st);
    return p2 ? launch_nr<0, float, F32Oct, true, false>(grads, n_grads, g_out, len, c, st)
              : launch_nr<0, float, F32Oct, false, false>(grads, n_grads, g_out, len, c, st);
}

}  // namespace zero
