// ledger.cpp -- host-side memory and communication ledger, and the
// algorithmic byte counts the measurements divide by.
//
// "Learn: ZeRO & FSDP", section 3: model state is (2 + 2 + K) psi bytes,
// K = 12 (bf16 parameters 2, bf16 gradients 2, fp32 master + m + v 12);
// section 4: stage 1 shards the optimizer state, stage 2 also the gradients,
// stage 3 also the parameters, and communication per step is 2 psi elements
// for stages 0-2 and 3 psi for stage 3.
// "ZeRO: Three Ledgers", section 2: a ring reduce-scatter plus all-gather
// moves 2 (N-1)/N of the data; section 4: bucketed reduce-scatter makes the
// gradients transient (stage 1 = stage 2 in resident memory).
// "ZeRO and FSDP sharding", Complexity and constants: ZeRO-3's extra memory is
// about two units of gathered bf16 weights (current and prefetched).
#include <cmath>

#include "zero_internal.h"

namespace {
constexpr double kOptimBytes = 12.0;  // K: fp32 master, m, v
constexpr double kParamBytes = 2.0;   // bf16 working copy
constexpr double kGradBytes = 2.0;    // bf16 gradient
}  // namespace

extern "C" zero_status zero_ledger(double psi, int32_t n_ranks, int32_t stage,
                                   int32_t grads_transient, zero_ledger_out *out)
{
    if (!out || !(psi >= 0.0) || n_ranks < 1 || stage < 0 || stage > 3)
        return ZERO_EINVAL;
    const double n = (double)n_ranks;
    zero_ledger_out o{};
    o.params_bytes = kParamBytes * psi / (stage >= 3 ? n : 1.0);
    o.grads_bytes = grads_transient ? 0.0 : kGradBytes * psi / (stage >= 2 ? n : 1.0);
    o.optim_bytes = kOptimBytes * psi / (stage >= 1 ? n : 1.0);
    o.model_state_bytes = o.params_bytes + o.grads_bytes + o.optim_bytes;
    o.comm_elements = (stage == 3 ? 3.0 : 2.0) * psi;
    o.comm_elements_ring = o.comm_elements * (n - 1.0) / n;
    o.optimizer_floats_per_rank = 3.0 * psi / (stage >= 1 ? n : 1.0);
    *out = o;
    return ZERO_OK;
}

extern "C" zero_status zero_gather_buffer_bytes(const zero_layout *L, int32_t units_in_flight,
                                                double *bytes)
{
    if (!zero::layout_ok(L) || units_in_flight < 0 || !bytes)
        return ZERO_EINVAL;
    int64_t largest = 0;
    for (int32_t u = 0; u < L->n_units; ++u)
        if (L->unit[u].padded > largest)
            largest = L->unit[u].padded;
    *bytes = kParamBytes * (double)largest * units_in_flight;
    return ZERO_OK;
}

extern "C" zero_status zero_step_traffic(const zero_layout *L, int32_t rank, int32_t n_grads,
                                         int32_t grad_dtype, int32_t with_out, double *bytes,
                                         int64_t *elements)
{
    if (!zero::layout_ok(L) || !bytes || !elements || n_grads < 1 ||
        (grad_dtype != ZERO_F32 && grad_dtype != ZERO_BF16) || rank >= L->n_ranks)
        return ZERO_EINVAL;
    const int64_t e = zero::selected_elements(L, rank);
    const double gsize = grad_dtype == ZERO_BF16 ? 2.0 : 4.0;
    const double per = n_grads * gsize + 12.0 + 12.0 + (with_out ? 2.0 : 0.0);
    *elements = e;
    *bytes = per * (double)e;
    return ZERO_OK;
}

extern "C" zero_status zero_gradnorm_traffic(const zero_layout *L, int32_t rank, int32_t n_grads,
                                             int32_t grad_dtype, int32_t with_g_out,
                                             double *bytes, int64_t *elements)
{
    if (!zero::layout_ok(L) || !bytes || !elements || n_grads < 1 ||
        (grad_dtype != ZERO_F32 && grad_dtype != ZERO_BF16) || rank >= L->n_ranks)
        return ZERO_EINVAL;
    const int64_t e = zero::selected_elements(L, rank);
    const double gsize = grad_dtype == ZERO_BF16 ? 2.0 : 4.0;
    *elements = e;
    *bytes = (n_grads * gsize + (with_g_out ? 4.0 : 0.0)) * (double)e;
    return ZERO_OK;
}

// "Learn: ZeRO & FSDP", section 3's bytes per element (2 gradient, 12 fp32
// state, 2 bf16 parameters) over the buffers of the one-GPU simulation.
extern "C" zero_status zero_sim_footprint(const zero_layout *L, int32_t n_grads, int32_t grad_dtype,
                                          int32_t grad_index, int32_t state_index,
                                          int32_t out_index, int32_t with_out, int32_t with_g,
                                          zero_footprint_out *out)
{
    const auto index_ok = [](int32_t x) { return x == ZERO_GLOBAL || x == ZERO_LOCAL; };
    if (!zero::layout_ok(L) || !out || n_grads < 1 ||
        (grad_dtype != ZERO_F32 && grad_dtype != ZERO_BF16) || !index_ok(grad_index) ||
        !index_ok(state_index) || !index_ok(out_index))
        return ZERO_EINVAL;
    const auto extent = [L](int32_t x) { return (double)(x == ZERO_GLOBAL ? L->padded : L->shard); };
    zero_footprint_out o{};
    o.grads_bytes = n_grads * (grad_dtype == ZERO_BF16 ? kGradBytes : 4.0) * extent(grad_index);
    o.state_bytes = kOptimBytes * extent(state_index);
    o.out_bytes = with_out ? kParamBytes * extent(out_index) : 0.0;
    o.g_bytes = with_g ? 4.0 * extent(state_index) : 0.0;
    o.total_bytes = o.grads_bytes + o.state_bytes + o.out_bytes + o.g_bytes;
    *out = o;
    return ZERO_OK;
}

// "ZeRO and FSDP sharding", Complexity and constants: a unit's all-gather
// (2 psi_unit (N-1)/N bytes of bf16 weights per rank) is hidden when it takes
// no longer than the unit's compute (6 psi_unit flops per token).
extern "C" zero_status zero_overlap(double psi_unit, int32_t n_ranks, double busbw_bytes_per_s,
                                    double tokens_per_gpu, double flops_per_s,
                                    zero_overlap_out *out)
{
    if (!out || !(psi_unit >= 0.0) || n_ranks < 1 || !(busbw_bytes_per_s > 0.0) ||
        !(tokens_per_gpu >= 0.0) || !(flops_per_s > 0.0))
        return ZERO_EINVAL;
    const double n = (double)n_ranks;
    zero_overlap_out o{};
    o.gather_bytes = kParamBytes * psi_unit * (n - 1.0) / n;
    o.gather_s = o.gather_bytes / busbw_bytes_per_s;
    o.compute_flops = 6.0 * psi_unit * tokens_per_gpu;
    o.compute_s = o.compute_flops / flops_per_s;
    o.ratio = o.compute_s > 0.0 ? o.gather_s / o.compute_s : (o.gather_s > 0.0 ? INFINITY : 0.0);
    o.hidden = o.gather_s <= o.compute_s ? 1 : 0;
    *out = o;
    return ZERO_OK;
}
