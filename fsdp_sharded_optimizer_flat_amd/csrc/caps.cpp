// caps.cpp -- zero_get_waves_per_cu_for: the occupancy cap a launch would
// use, for either gradient type and for the staged step's kernels.
//
// Which rank counts have a kernel compiled for them decides whether the
// compile-time or the run-time cap applies.  The sets below are the ones the
// launchers dispatch on for 16-byte aligned buffers:
//   fused step, bf16 gradients:   1..32 and 64          (step_kernels.hip)
//   fused step, fp32 gradients:   2, 4, 8, 16, 32       (step_kernels.hip)
//   norm pass, bf16 gradients:    1..32 and 64          (norm_kernels.hip)
//   staged reduction, bf16:       32 and 64             (stage_kernels.hip)
//   norm pass and staged reduction, fp32 gradients: none (run-time kernel)
#include "zero_internal.h"

namespace zero {
namespace {

bool step_compiled(int n, int grad_bytes)
{
    return grad_bytes == 2 ? compiled_ranks(n) : (n == 2 || n == 4 || n == 8 || n == 16 || n == 32);
}

bool reduction_compiled(int n, int grad_bytes, bool staged)
{
    if (grad_bytes != 2)
        return false;
    return staged ? (n == 32 || n == 64) : compiled_ranks(n);
}

}  // namespace
}  // namespace zero

extern "C" zero_status zero_get_waves_per_cu_for(int32_t kind, int32_t n_grads, int32_t grad_dtype,
                                                 int32_t staged, int32_t *waves)
{
    using namespace zero;
    if (kind < ZERO_CAP_STEP || kind > ZERO_CAP_NORM || !waves || n_grads < 1 ||
        n_grads > ZERO_MAX_RANKS || (grad_dtype != ZERO_F32 && grad_dtype != ZERO_BF16))
        return ZERO_EINVAL;
    const int gb = grad_dtype == ZERO_BF16 ? 2 : 4;
    if (kind == ZERO_CAP_STEP)
        *waves = step_waves_per_cu(n_grads, !step_compiled(n_grads, gb), gb);
    else if (kind == ZERO_CAP_STEP1)
        *waves = step1_waves_per_cu(staged != 0);
    else
        *waves = norm_waves_per_cu(n_grads, !reduction_compiled(n_grads, gb, staged != 0), gb);
    return ZERO_OK;
}
