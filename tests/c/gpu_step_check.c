/*
 * gpu_step_check.c -- the library driven from plain C on the GPU, with no
 * Python and no torch: HIP's C runtime API for device memory, the C ABI of
 * include/zero.h for the work, and the CPU oracle (test infrastructure,
 * linked from oracle/liboracle.so) for the expected values.
 *
 * N = 8 simulated ranks, two ragged units, bf16 gradients:
 *   - zero_step over every shard (GLOBAL), 3 steps, vs orc_zero_step_all:
 *     master, m, v and the bf16 all-gather slots bit for bit;
 *   - zero_gradnorm of rank 5 (LOCAL chunks) vs the oracle's reduced
 *     gradient and binary64 sum (relative 1e-12), the clip coefficients
 *     equal, and the reduced gradient it writes bit for bit;
 *   - rank 5's clipped step with no host synchronization
 *     (zero_gradnorm_async -> zero_clip_coef_async -> zero_step_device_clip
 *     on the reduced gradient), 2 steps, vs the oracle's clipped rank step on
 *     the 8 chunks with the oracle's own coefficient;
 * and, at N2 = 40 ranks (a run-time rank count), rank 3's staged step
 * through a workspace of 4096-element chunks, 2 steps, vs the oracle's rank
 * step.  Prints "ok" and exits 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero.h"

/* the oracle's entry points (oracle/oracle.c) */
uint16_t orc_bf16(float x);
int orc_zero_step_all(int32_t n, int32_t n_units, const int64_t *numel, const void *const *grads,
                      int32_t n_grads, int32_t grad_bf16, float divisor, float clip, float *master,
                      float *m, float *v, uint16_t *out, int32_t t, float lr, float b1, float b2,
                      float eps, float wd);
int orc_zero_step_rank(int32_t n, int32_t n_units, const int64_t *numel, int32_t r,
                       const void *const *grads, int32_t n_grads, int32_t grad_bf16,
                       int32_t grad_local, float divisor, float clip, float *master, float *m,
                       float *v, int32_t state_global, uint16_t *out, int32_t out_gather,
                       int32_t t, float lr, float b1, float b2, float eps, float wd);
int orc_reduced_grad(int32_t n, int32_t n_units, const int64_t *numel, int32_t r,
                     const void *const *grads, int32_t n_grads, int32_t grad_bf16,
                     int32_t grad_local, float divisor, float *g_out);
double orc_sumsq(const float *g, int64_t n);
float orc_clip_coef(double sumsq, double max_norm);

#define N 8
#define N2 40
#define LR 3e-4f
#define B1 0.9f
#define B2 0.95f
#define EPS 1e-8f
#define WD 0.1f
#define FAIL(...) do { fprintf(stderr, __VA_ARGS__); fprintf(stderr, "\n"); exit(1); } while (0)
#define HIPCHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) FAIL("%s: %s", #x, hipGetErrorString(e_)); } while (0)
#define ZCHECK(x) do { zero_status s_ = (x); if (s_ != ZERO_OK) FAIL("%s: %s (%s)", #x, zero_strerror(s_), zero_last_hip_error()); } while (0)

/* test data: a 64-bit LCG and a sum of uniforms (no method arithmetic) */
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) * 0x1p-53;
}
static float normalish(double scale)
{
    double s = 0.0;
    for (int i = 0; i < 12; ++i)
        s += uniform();
    return (float)((s - 6.0) * scale);
}

static void *dev_copy(const void *h, size_t bytes)
{
    void *d = NULL;
    HIPCHECK(hipMalloc(&d, bytes ? bytes : 16));
    if (bytes)
        HIPCHECK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    return d;
}

static void same_bits(const void *a, const void *b, size_t bytes, const char *what)
{
    if (memcmp(a, b, bytes) != 0)
        FAIL("%s differs from the oracle", what);
}

static void fetch(void *h, const void *d, size_t bytes)
{
    HIPCHECK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
}

/* Rank r's shard state (LOCAL, S elements): random master, zero m, v, out,
 * on the host and copied to the device. */
typedef struct shard_state {
    int64_t S;
    float *w, *m, *v;
    uint16_t *out;
    float *dw, *dm, *dv;
    uint16_t *dout;
} shard_state;

static shard_state new_state(int64_t S)
{
    shard_state st;
    st.S = S;
    st.w = (float *)calloc((size_t)S, 4);
    st.m = (float *)calloc((size_t)S, 4);
    st.v = (float *)calloc((size_t)S, 4);
    st.out = (uint16_t *)calloc((size_t)S, 2);
    for (int64_t i = 0; i < S; ++i)
        st.w[i] = normalish(0.02);
    st.dw = (float *)dev_copy(st.w, (size_t)S * 4);
    st.dm = (float *)dev_copy(st.m, (size_t)S * 4);
    st.dv = (float *)dev_copy(st.v, (size_t)S * 4);
    st.dout = (uint16_t *)dev_copy(st.out, (size_t)S * 2);
    return st;
}

static void check_state(const shard_state *st, const char *what)
{
    const size_t S = (size_t)st->S;
    float *h = (float *)malloc(S * 4);
    uint16_t *ho = (uint16_t *)malloc(S * 2);
    char name[96];
    fetch(h, st->dw, S * 4);
    snprintf(name, sizeof name, "%s: master", what);
    same_bits(h, st->w, S * 4, name);
    fetch(h, st->dm, S * 4);
    snprintf(name, sizeof name, "%s: m", what);
    same_bits(h, st->m, S * 4, name);
    fetch(h, st->dv, S * 4);
    snprintf(name, sizeof name, "%s: v", what);
    same_bits(h, st->v, S * 4, name);
    fetch(ho, st->dout, S * 2);
    snprintf(name, sizeof name, "%s: bf16 shard", what);
    same_bits(ho, st->out, S * 2, name);
    free(h);
    free(ho);
}

/* Rank r's clipped step with every stage on the device: norm pass writing
 * the reduced gradient and the sum to device memory, the coefficient formed
 * on the device, the step on the reduced gradient scaled by it. */
static void clipped_chain(const zero_layout *L, const int64_t *numel, int r,
                          const void *const *dchunk, const void *const *chunk, void *ws,
                          size_t wsb)
{
    const double max_norm = 0.01;
    shard_state st = new_state(L->shard);
    float *dgred = NULL, *dcoef = NULL;
    double *dsum = NULL;
    HIPCHECK(hipMalloc((void **)&dgred, (size_t)L->shard * 4));
    HIPCHECK(hipMalloc((void **)&dcoef, 4));
    HIPCHECK(hipMalloc((void **)&dsum, 8));
    zero_adamw_scalars sc;
    ZCHECK(zero_adamw_scalars_for(1, LR, B1, B2, EPS, WD, 1.0f, &sc));
    float *og = (float *)malloc((size_t)L->shard * 4);
    if (orc_reduced_grad(N, 2, numel, r, chunk, N, 1, 1, (float)N, og) != 0)
        FAIL("oracle reduced gradient failed");
    const float ocoef = orc_clip_coef(orc_sumsq(og, L->shard), max_norm);
    if (!(ocoef < 1.0f))
        FAIL("the clipped-chain case must clip (coefficient %.9g)", ocoef);
    for (int t = 1; t <= 2; ++t) {
        const void *g1[1] = {dgred};
        ZCHECK(zero_gradnorm_async(L, r, dchunk, N, ZERO_BF16, ZERO_LOCAL, (float)N, dgred,
                                   ZERO_LOCAL, ws, wsb, dsum, NULL));
        ZCHECK(zero_clip_coef_async(dsum, max_norm, dcoef, NULL));
        ZCHECK(zero_step_device_clip(L, r, g1, 1, ZERO_F32, ZERO_LOCAL, 1.0f, st.dw, st.dm, st.dv,
                                     ZERO_LOCAL, st.dout, ZERO_LOCAL, &sc, dcoef, NULL));
        if (orc_zero_step_rank(N, 2, numel, r, chunk, N, 1, 1, (float)N, ocoef, st.w, st.m, st.v, 0,
                               st.out, 0, t, LR, B1, B2, EPS, WD) != 0)
            FAIL("oracle clipped step failed");
        zero_adamw_scalars next;
        ZCHECK(zero_adamw_scalars_next(&sc, &next));
        sc = next;
    }
    HIPCHECK(hipDeviceSynchronize());
    float dc = 0.0f;
    fetch(&dc, dcoef, 4);
    if (dc != ocoef)
        FAIL("device clip coefficient %.9g vs oracle %.9g", dc, ocoef);
    check_state(&st, "clipped chain");
}

/* Rank 3's staged step at N2 ranks from its LOCAL reduce-scatter chunks,
 * through a workspace of 4096-element chunks (several per unit). */
static void staged_step(void)
{
    const int r = 3;
    const int64_t numel[2] = {(int64_t)N2 * 9000 + 17, 5003};
    size_t lbytes = 0;
    ZCHECK(zero_pack(N2, 2, numel, NULL, 0, &lbytes));
    zero_layout *L = (zero_layout *)malloc(lbytes);
    ZCHECK(zero_pack(N2, 2, numel, L, lbytes, NULL));
    const int64_t S = L->shard;
    uint16_t *chunk[N2];
    const void *dchunk[N2];
    for (int q = 0; q < N2; ++q) {
        chunk[q] = (uint16_t *)malloc((size_t)S * 2);
        for (int64_t i = 0; i < S; ++i)
            chunk[q][i] = orc_bf16(normalish(1e-3));
        dchunk[q] = dev_copy(chunk[q], (size_t)S * 2);
    }
    shard_state st = new_state(S);
    const size_t wsb = (4096 + 4) * 4;
    void *ws = NULL;
    HIPCHECK(hipMalloc(&ws, wsb));
    zero_adamw_scalars sc;
    ZCHECK(zero_adamw_scalars_for(1, LR, B1, B2, EPS, WD, 1.0f, &sc));
    for (int t = 1; t <= 2; ++t) {
        ZCHECK(zero_step_staged(L, r, dchunk, N2, ZERO_BF16, ZERO_LOCAL, (float)N2, st.dw, st.dm,
                                st.dv, ZERO_LOCAL, st.dout, ZERO_LOCAL, &sc, ws, wsb, NULL));
        if (orc_zero_step_rank(N2, 2, numel, r, (const void *const *)chunk, N2, 1, 1, (float)N2,
                               1.0f, st.w, st.m, st.v, 0, st.out, 0, t, LR, B1, B2, EPS, WD) != 0)
            FAIL("oracle staged-case step failed");
        zero_adamw_scalars next;
        ZCHECK(zero_adamw_scalars_next(&sc, &next));
        sc = next;
    }
    HIPCHECK(hipDeviceSynchronize());
    check_state(&st, "staged step");
}

int main(void)
{
    const int64_t numel[2] = {N * 5000 + 3, 1001};
    size_t lbytes = 0;
    ZCHECK(zero_pack(N, 2, numel, NULL, 0, &lbytes));
    zero_layout *L = (zero_layout *)malloc(lbytes);
    ZCHECK(zero_pack(N, 2, numel, L, lbytes, NULL));
    const int64_t P = L->padded, S = L->shard;

    /* every rank's whole padded bf16 gradient; padding zero */
    uint16_t *g[N];
    for (int q = 0; q < N; ++q) {
        g[q] = (uint16_t *)calloc((size_t)P, 2);
        for (int u = 0; u < 2; ++u)
            for (int64_t i = 0; i < L->unit[u].numel; ++i)
                g[q][L->unit[u].offset + i] = orc_bf16(normalish(1e-3));
    }
    float *w = (float *)calloc((size_t)P, 4), *m = (float *)calloc((size_t)P, 4),
          *v = (float *)calloc((size_t)P, 4);
    for (int u = 0; u < 2; ++u)
        for (int64_t i = 0; i < L->unit[u].numel; ++i)
            w[L->unit[u].offset + i] = normalish(0.02);
    uint16_t *out = (uint16_t *)calloc((size_t)P, 2);

    const void *dg[N];
    for (int q = 0; q < N; ++q)
        dg[q] = dev_copy(g[q], (size_t)P * 2);
    float *dw = (float *)dev_copy(w, (size_t)P * 4), *dm = (float *)dev_copy(m, (size_t)P * 4),
          *dv = (float *)dev_copy(v, (size_t)P * 4);
    uint16_t *dout = (uint16_t *)dev_copy(out, (size_t)P * 2);

    /* three steps, every shard */
    zero_adamw_scalars sc;
    ZCHECK(zero_adamw_scalars_for(1, LR, B1, B2, EPS, WD, 1.0f, &sc));
    for (int t = 1; t <= 3; ++t) {
        ZCHECK(zero_step(L, -1, dg, N, ZERO_BF16, ZERO_GLOBAL, (float)N, dw, dm, dv, ZERO_GLOBAL,
                         dout, ZERO_GLOBAL, &sc, NULL));
        if (orc_zero_step_all(N, 2, numel, (const void *const *)g, N, 1, (float)N, 1.0f, w, m, v,
                              out, t, LR, B1, B2, EPS, WD) != 0)
            FAIL("oracle step failed");
        zero_adamw_scalars next;
        ZCHECK(zero_adamw_scalars_next(&sc, &next));
        sc = next;
    }
    HIPCHECK(hipDeviceSynchronize());
    float *hw = (float *)malloc((size_t)P * 4), *hm = (float *)malloc((size_t)P * 4),
          *hv = (float *)malloc((size_t)P * 4);
    uint16_t *hout = (uint16_t *)malloc((size_t)P * 2);
    HIPCHECK(hipMemcpy(hw, dw, (size_t)P * 4, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(hm, dm, (size_t)P * 4, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(hv, dv, (size_t)P * 4, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(hout, dout, (size_t)P * 2, hipMemcpyDeviceToHost));
    same_bits(hw, w, (size_t)P * 4, "master");
    same_bits(hm, m, (size_t)P * 4, "m");
    same_bits(hv, v, (size_t)P * 4, "v");
    same_bits(hout, out, (size_t)P * 2, "bf16 parameters");

    /* norm of rank 5 from its reduce-scatter chunks (LOCAL) */
    const int r = 5;
    uint16_t *chunk[N];
    const void *dchunk[N];
    for (int q = 0; q < N; ++q) {
        chunk[q] = (uint16_t *)malloc((size_t)S * 2);
        for (int u = 0; u < 2; ++u)
            memcpy(chunk[q] + L->unit[u].local_offset,
                   g[q] + L->unit[u].offset + (int64_t)r * L->unit[u].shard,
                   (size_t)L->unit[u].shard * 2);
        dchunk[q] = dev_copy(chunk[q], (size_t)S * 2);
    }
    size_t wsb = 0;
    ZCHECK(zero_gradnorm_workspace_bytes(L, r, &wsb));
    void *ws = NULL;
    float *dgred = NULL;
    HIPCHECK(hipMalloc(&ws, wsb));
    HIPCHECK(hipMalloc((void **)&dgred, (size_t)S * 4));
    double sumsq = -1.0;
    ZCHECK(zero_gradnorm(L, r, dchunk, N, ZERO_BF16, ZERO_LOCAL, (float)N, dgred, ZERO_LOCAL, ws,
                         wsb, &sumsq, NULL));
    float *og = (float *)malloc((size_t)S * 4), *hg = (float *)malloc((size_t)S * 4);
    if (orc_reduced_grad(N, 2, numel, r, (const void *const *)chunk, N, 1, 1, (float)N, og) != 0)
        FAIL("oracle reduced gradient failed");
    HIPCHECK(hipMemcpy(hg, dgred, (size_t)S * 4, hipMemcpyDeviceToHost));
    same_bits(hg, og, (size_t)S * 4, "reduced gradient");
    const double osum = orc_sumsq(og, S);
    if (!(fabs(sumsq - osum) <= 1e-12 * osum))
        FAIL("sum of squares %.17g vs oracle %.17g", sumsq, osum);
    float coef = 0.0f;
    ZCHECK(zero_clip_coef(sumsq, 0.01, &coef));
    if (coef != orc_clip_coef(osum, 0.01))
        FAIL("clip coefficient %.9g vs oracle %.9g", coef, orc_clip_coef(osum, 0.01));

    clipped_chain(L, numel, r, dchunk, (const void *const *)chunk, ws, wsb);
    staged_step();
    printf("ok\n");
    return 0;
}
