// fp_probe.hip -- test support, not part of the library: binary32 square
// root and division as bare elementwise kernels, compiled with exactly the
// library's floating-point flags, so the GPU tests can check every input
// pattern against the host's IEEE operations.  The library's kernels use the
// same operators under the same flags.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

__global__ __launch_bounds__(256) void sqrt_kernel(const float *__restrict__ x,
                                                   float *__restrict__ y, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        y[i] = sqrtf(x[i]);
}

__global__ __launch_bounds__(256) void div_kernel(const float *__restrict__ a,
                                                  const float *__restrict__ b,
                                                  float *__restrict__ y, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        y[i] = a[i] / b[i];
}

}  // namespace

// n <= 2^32 - 256 elements per call (one dispatch); returns a hipError_t.
extern "C" int probe_sqrt(const float *x, float *y, int64_t n, void *stream)
{
    if (n <= 0)
        return hipSuccess;
    if (n > (int64_t(1) << 32) - 256)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(sqrt_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), x, y, n);
    return hipGetLastError();
}

extern "C" int probe_div(const float *a, const float *b, float *y, int64_t n, void *stream)
{
    if (n <= 0)
        return hipSuccess;
    if (n > (int64_t(1) << 32) - 256)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(div_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), a, b, y, n);
    return hipGetLastError();
}
