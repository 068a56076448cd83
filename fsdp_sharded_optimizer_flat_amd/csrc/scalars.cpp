// scalars.cpp -- host-side AdamW step scalars and the clip coefficient.
//
// "ZeRO and FSDP sharding", Code: AdamW with b1, b2, eps, decoupled weight
// decay wd, step counter t (1 at the first step) and bias corrections
// 1 - b1^t and sqrt(1 - b2^t); lr / bc1 and 1 - lr * wd are per-step
// constants, so they are formed once here instead of per element.
//
// Everything is binary32 with one rounding per operation; this file is
// compiled without FMA contraction (see the build flags) so the compiler
// keeps each product and sum separately rounded.
#include <cfloat>
#include <cmath>

#include "zero_internal.h"

static void finish_scalars(zero_adamw_scalars *s)
{
    s->one_minus_b1 = 1.0f - s->b1;
    s->one_minus_b2 = 1.0f - s->b2;
    s->bc1 = 1.0f - s->pow1;
    const float one_minus_pow2 = 1.0f - s->pow2;
    s->bc2 = std::sqrt(one_minus_pow2);
    s->step_size = s->lr / s->bc1;
    const float lr_wd = s->lr * s->wd;
    s->decay = 1.0f - lr_wd;
}

extern "C" zero_status zero_adamw_scalars_for(int32_t t, float lr, float b1, float b2, float eps,
                                              float wd, float clip_coef, zero_adamw_scalars *out)
{
    if (!out || t < 1 || std::isnan(lr) || std::isnan(b1) || std::isnan(b2) || std::isnan(eps) ||
        std::isnan(wd) || std::isnan(clip_coef))
        return ZERO_EINVAL;
    zero_adamw_scalars s{};
    s.t = t;
    s.lr = lr;
    s.b1 = b1;
    s.b2 = b2;
    s.eps = eps;
    s.wd = wd;
    s.clip_coef = clip_coef;
    // beta^t as the running binary32 product, the value a stateful optimizer
    // carries from step to step.
    volatile float p1 = 1.0f, p2 = 1.0f;  // volatile: keep every product rounded to binary32
    for (int32_t i = 0; i < t; ++i) {
        p1 = p1 * b1;
        p2 = p2 * b2;
        if (p1 == 0.0f && p2 == 0.0f)
            break;  // both products have underflowed to zero; they stay there
    }
    s.pow1 = p1;
    s.pow2 = p2;
    finish_scalars(&s);
    *out = s;
    return ZERO_OK;
}

extern "C" zero_status zero_adamw_scalars_next(const zero_adamw_scalars *prev,
                                               zero_adamw_scalars *out)
{
    if (!prev || !out || prev->t < 0 || prev->t == INT32_MAX)
        return ZERO_EINVAL;
    zero_adamw_scalars s = *prev;
    s.t = prev->t + 1;
    if (prev->t == 0) {  // a zero-initialised struct carrying the hyperparameters
        s.pow1 = 1.0f;
        s.pow2 = 1.0f;
    }
    volatile float p1 = s.pow1 * s.b1;
    volatile float p2 = s.pow2 * s.b2;
    s.pow1 = p1;
    s.pow2 = p2;
    finish_scalars(&s);
    *out = s;
    return ZERO_OK;
}

// "ZeRO and FSDP sharding", Implementation notes: clipping uses the global
// norm, the square root of the summed squared shard norms; the coefficient
// follows clip_grad_norm_'s convention max_norm / (norm + 1e-6), capped at 1.
extern "C" zero_status zero_clip_coef(double sumsq, double max_norm, float *coef)
{
    // a sum of squares that is negative, NaN or infinite (a non-finite
    // gradient) has no clip coefficient
    if (!coef || !(sumsq >= 0.0 && sumsq <= DBL_MAX) || !(max_norm > 0.0))
        return ZERO_EINVAL;
    const double norm = std::sqrt(sumsq);
    double c = max_norm / (norm + 1e-6);
    if (c > 1.0)
        c = 1.0;
    *coef = (float)c;
    return ZERO_OK;
}

// "ZeRO and FSDP sharding", Implementation notes: the global norm combines
// every shard's sum of squares.  Rank order, binary64, one rounding per add.
extern "C" zero_status zero_clip_coef_ranks(const double *rank_sums, int32_t n_ranks,
                                            double max_norm, float *coef, double *total)
{
    if (!rank_sums || !coef || n_ranks < 1 || n_ranks > ZERO_MAX_UNITS)
        return ZERO_EINVAL;
    double t = rank_sums[0];
    if (!(t >= 0.0))
        return ZERO_EINVAL;
    for (int32_t r = 1; r < n_ranks; ++r) {
        if (!(rank_sums[r] >= 0.0))
            return ZERO_EINVAL;
        t = t + rank_sums[r];
    }
    const zero_status st = zero_clip_coef(t, max_norm, coef);
    if (st == ZERO_OK && total)
        *total = t;
    return st;
}
