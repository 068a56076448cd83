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
 *     equal, and the reduced gradient it writes bit for bit.
 * Prints "ok" and exits 0 on success.
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
int orc_reduced_grad(int32_t n, int32_t n_units, const int64_t *numel, int32_t r,
                     const void *const *grads, int32_t n_grads, int32_t grad_bf16,
                     int32_t grad_local, float divisor, float *g_out);
double orc_sumsq(const float *g, int64_t n);
float orc_clip_coef(double sumsq, double max_norm);

#define N 8
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
    ZCHECK(zero_adamw_scalars_for(1, 3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, &sc));
    for (int t = 1; t <= 3; ++t) {
        ZCHECK(zero_step(L, -1, dg, N, ZERO_BF16, ZERO_GLOBAL, (float)N, dw, dm, dv, ZERO_GLOBAL,
                         dout, ZERO_GLOBAL, &sc, NULL));
        if (orc_zero_step_all(N, 2, numel, (const void *const *)g, N, 1, (float)N, 1.0f, w, m, v,
                              out, t, 3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f) != 0)
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
    printf("ok\n");
    return 0;
}
