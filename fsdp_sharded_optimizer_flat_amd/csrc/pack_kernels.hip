// pack_kernels.hip -- device copies of the flat-buffer packer: copy a
// parameter into (or out of) its range of the flat buffer with an optional
// fp32 <-> bf16 conversion, and zero-fill the padding ("ZeRO and FSDP
// sharding", How it works: flatten each unit into one buffer padded to a
// multiple of N).  Run once at setup; the step never calls them.
#include "device_common.h"

namespace zero {
namespace {

using namespace dev;

template <typename S, typename D>
__device__ __forceinline__ D convert(S x);
template <>
__device__ __forceinline__ float convert<float, float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t convert<uint16_t, uint16_t>(uint16_t x) { return x; }
template <>
__device__ __forceinline__ uint16_t convert<float, uint16_t>(float x) { return to_bf16(x); }
template <>
__device__ __forceinline__ float convert<uint16_t, float>(uint16_t x)
{
    return __uint_as_float((unsigned)x << 16);
}

template <typename S, typename D>
__global__ __launch_bounds__(kBlock) void convert_kernel(const S *__restrict__ src,
                                                        D *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        dst[i] = convert<S, D>(src[i]);
}

template <typename T>
__global__ __launch_bounds__(kBlock) void fill_zero_kernel(T *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        dst[i] = T(0);
}

unsigned grid_of(int64_t n)
{
    int64_t g = (n + kBlock - 1) / kBlock;
    if (g > 4096)
        g = 4096;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

int launch_convert(const void *src, int src_dtype, void *dst, int dst_dtype, int64_t n,
                   void *stream)
{
    if (n <= 0)
        return hipSuccess;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const unsigned g = grid_of(n);
    if (src_dtype == ZERO_F32 && dst_dtype == ZERO_F32)
        hipLaunchKernelGGL((convert_kernel<float, float>), dim3(g), dim3(kBlock), 0, st,
                           (const float *)src, (float *)dst, n);
    else if (src_dtype == ZERO_F32 && dst_dtype == ZERO_BF16)
        hipLaunchKernelGGL((convert_kernel<float, uint16_t>), dim3(g), dim3(kBlock), 0, st,
                           (const float *)src, (uint16_t *)dst, n);
    else if (src_dtype == ZERO_BF16 && dst_dtype == ZERO_F32)
        hipLaunchKernelGGL((convert_kernel<uint16_t, float>), dim3(g), dim3(kBlock), 0, st,
                           (const uint16_t *)src, (float *)dst, n);
    else
        hipLaunchKernelGGL((convert_kernel<uint16_t, uint16_t>), dim3(g), dim3(kBlock), 0, st,
                           (const uint16_t *)src, (uint16_t *)dst, n);
    return hipGetLastError();
}

int launch_fill_zero(void *dst, int dtype, int64_t n, void *stream)
{
    if (n <= 0)
        return hipSuccess;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == ZERO_F32)
        hipLaunchKernelGGL((fill_zero_kernel<float>), dim3(grid_of(n)), dim3(kBlock), 0, st,
                           (float *)dst, n);
    else
        hipLaunchKernelGGL((fill_zero_kernel<uint16_t>), dim3(grid_of(n)), dim3(kBlock), 0, st,
                           (uint16_t *)dst, n);
    return hipGetLastError();
}

}  // namespace zero
