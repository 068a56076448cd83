/*
 * host_sanitize_check.c -- the library's host code under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Built against a copy of libzero.so whose host
 * code is instrumented (the device code is not), run without a GPU: every
 * host-only entry point on many small random cases, the host step and the
 * host reshard checked against the oracle's C library (test infrastructure,
 * oracle/liboracle.so), and the validation paths of the device entry points
 * with fake device addresses that never reach a device call.
 * Prints "ok" and exits 0 on success; a sanitizer report aborts the run.
 */
#define _POSIX_C_SOURCE 200809L
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include "zero.h"

/* the oracle's entry points (oracle/oracle.c) */
int orc_zero_step_rank(int32_t n, int32_t n_units, const int64_t *numel, int32_t r,
                       const void *const *grads, int32_t n_grads, int32_t grad_bf16,
                       int32_t grad_local, float divisor, float clip, float *master, float *m,
                       float *v, int32_t state_global, uint16_t *out, int32_t out_gather,
                       int32_t t, float lr, float b1, float b2, float eps, float wd);
int orc_zero_step_all(int32_t n, int32_t n_units, const int64_t *numel, const void *const *grads,
                      int32_t n_grads, int32_t grad_bf16, float divisor, float clip, float *master,
                      float *m, float *v, uint16_t *out, int32_t t, float lr, float b1, float b2,
                      float eps, float wd);
int orc_reshard(int32_t units_a, const int64_t *numel_a, int32_t n_a, const int64_t *row_a,
                const void *const *src, int32_t units_b, const int64_t *numel_b, int32_t n_b,
                const int64_t *row_b, int32_t dst_rank, void *dst, int32_t elem);

#define FAIL(...)                                                                          \
    do {                                                                                   \
        printf("FAIL line %d: ", __LINE__);                                                \
        printf(__VA_ARGS__);                                                               \
        printf("\n");                                                                      \
        exit(1);                                                                           \
    } while (0)
#define CHECK(c)                                                                           \
    do {                                                                                   \
        if (!(c))                                                                          \
            FAIL("%s", #c);                                                                \
    } while (0)

static uint64_t rng = 0x243f6a8885a308d3ull;
static uint64_t next_u64(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return rng;
}
static int64_t rnd(int64_t lo, int64_t hi) /* [lo, hi] */
{
    return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1));
}
static float rndf(float scale)
{
    return (float)((double)(next_u64() >> 11) * 0x1p-53 - 0.5) * 2.0f * scale;
}

static zero_layout *make_layout(int32_t n, int32_t U, const int64_t *numel, const int64_t *gran)
{
    size_t need = 0;
    CHECK(zero_pack(n, U, numel, NULL, 0, &need) == ZERO_OK);
    zero_layout *L = (zero_layout *)malloc(need);
    if (gran)
        CHECK(zero_pack_rows(n, U, numel, gran, L, need, NULL) == ZERO_OK);
    else
        CHECK(zero_pack(n, U, numel, L, need, NULL) == ZERO_OK);
    return L;
}

/* layouts, index maps, traffic and workspace queries */
static void check_layouts(void)
{
    for (int it = 0; it < 400; ++it) {
        const int32_t n = (int32_t)rnd(1, 9), U = (int32_t)rnd(0, 4);
        int64_t numel[4], gran[4];
        for (int u = 0; u < U; ++u) {
            gran[u] = rnd(1, 5);
            numel[u] = gran[u] * rnd(0, 12);
        }
        zero_layout *L = make_layout(n, U, numel, (it & 1) ? gran : NULL);
        for (int32_t r = 0; r < n; ++r)
            for (int64_t k = 0; k < L->shard; ++k) {
                int64_t j = -1, k2 = -1;
                int32_t r2 = -1;
                CHECK(zero_global_index(L, r, k, &j) == ZERO_OK);
                CHECK(zero_owner(L, j, &r2, &k2) == ZERO_OK && r2 == r && k2 == k);
            }
        int64_t j = 0;
        int32_t r2 = 0;
        CHECK(zero_global_index(L, n, 0, &j) == ZERO_EINVAL);
        CHECK(zero_owner(L, L->padded, &r2, &j) == ZERO_EINVAL);
        for (int32_t r = -1; r < n; ++r) {
            size_t ws = 0;
            double b = 0;
            int64_t e = 0;
            CHECK(zero_gradnorm_workspace_bytes(L, r, &ws) == ZERO_OK && ws > 0);
            CHECK(zero_step_traffic(L, r, n, ZERO_BF16, 1, &b, &e) == ZERO_OK);
            CHECK(e == (r < 0 ? L->padded : L->shard));
            CHECK(zero_gradnorm_traffic(L, r, n, ZERO_F32, 1, &b, &e) == ZERO_OK);
        }
        double gb = 0;
        CHECK(zero_gather_buffer_bytes(L, 2, &gb) == ZERO_OK);
        free(L);
    }
}

static void check_scalars_ledger_arena(void)
{
    zero_adamw_scalars a, b, c;
    CHECK(zero_adamw_scalars_for(1, 3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, &a) == ZERO_OK);
    for (int t = 2; t <= 3000; ++t) {
        CHECK(zero_adamw_scalars_next(&a, &b) == ZERO_OK);
        a = b;
    }
    CHECK(zero_adamw_scalars_for(3000, 3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, &c) == ZERO_OK);
    CHECK(memcmp(&a, &c, sizeof a) == 0);
    CHECK(zero_adamw_scalars_for(0, 3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, &c) == ZERO_EINVAL);
    CHECK(zero_adamw_scalars_for(1, NAN, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, &c) == ZERO_EINVAL);
    for (int32_t stage = 0; stage <= 3; ++stage)
        for (int32_t tr = 0; tr <= 1; ++tr) {
            zero_ledger_out o;
            CHECK(zero_ledger(7.74e8, 8, stage, tr, &o) == ZERO_OK);
        }
    zero_ledger_out o;
    CHECK(zero_ledger(1.0, 8, 4, 0, &o) == ZERO_EINVAL);
    zero_overlap_out ov;
    CHECK(zero_overlap(8.75e8, 8, 4e11, 8192, 7e14, &ov) == ZERO_OK);
    CHECK(zero_overlap(8.75e8, 8, 0.0, 8192, 7e14, &ov) == ZERO_EINVAL);
    float coef = 0;
    double sums[64], total = 0;
    for (int r = 0; r < 64; ++r)
        sums[r] = (double)rnd(0, 1000) * 1e-3;
    CHECK(zero_clip_coef(2.0, 1.0, &coef) == ZERO_OK);
    CHECK(zero_clip_coef_ranks(sums, 64, 1.0, &coef, &total) == ZERO_OK);
    CHECK(zero_clip_coef_ranks(sums, 0, 1.0, &coef, &total) == ZERO_EINVAL);
    for (int it = 0; it < 300; ++it) {
        const int32_t nb = (int32_t)rnd(0, 70);
        int64_t bytes[70], offs[70], tot = 0;
        for (int i = 0; i < nb; ++i)
            bytes[i] = rnd(0, (int64_t)5 << 21);
        CHECK(zero_arena_plan(nb, bytes, offs, &tot) == ZERO_OK);
        for (int i = 1; i < nb; ++i)
            CHECK(offs[i] >= offs[i - 1] + bytes[i - 1]);
    }
    for (zero_status s = 1; s >= -6; --s)
        CHECK(zero_strerror(s) != NULL);
    CHECK(zero_last_hip_error() != NULL);
}

/* the host step against the oracle, every selection mode */
static void check_host_step(void)
{
    const float lr = 3e-4f, b1 = 0.9f, b2 = 0.95f, eps = 1e-8f, wd = 0.1f;
    for (int it = 0; it < 160; ++it) {
        const int32_t n = (int32_t)(it % 5 == 4 ? rnd(17, 40) : rnd(1, 9));
        const int32_t U = (int32_t)rnd(1, 3);
        int64_t numel[3];
        for (int u = 0; u < U; ++u)
            numel[u] = rnd(0, 300);
        zero_layout *L = make_layout(n, U, numel, NULL);
        const int32_t rank = (int32_t)rnd(-1, n - 1);
        const int bf = (int)rnd(0, 1);
        const int gl = rank >= 0 ? (int)rnd(0, 1) : 0;    /* gradients LOCAL */
        const int sg = rank < 0 ? 1 : (int)rnd(0, 1);    /* state GLOBAL */
        const int og = rank < 0 ? 1 : (int)rnd(0, 1);    /* out GLOBAL */
        const int shift = (int)rnd(0, 3), threads = (int)rnd(1, 4);
        const int64_t ge = gl ? L->shard : L->padded, se = sg ? L->padded : L->shard;
        const int64_t oe = og ? L->padded : L->shard;
        const int gsz = bf ? 2 : 4;
        unsigned char *gbuf = (unsigned char *)malloc((size_t)(n * (ge + 4) * gsz) + 16);
        void *gp[64];
        for (int q = 0; q < n; ++q) {
            gp[q] = gbuf + (size_t)q * (ge + 4) * gsz + shift * gsz;
            for (int64_t i = 0; i < ge; ++i) {
                const float x = rndf(1e-2f);
                if (bf) {
                    uint32_t u;
                    memcpy(&u, &x, 4);
                    ((uint16_t *)gp[q])[i] = (uint16_t)(u >> 16);
                } else {
                    ((float *)gp[q])[i] = x;
                }
            }
        }
        /* padding positions of GLOBAL gradients hold zero (the packer's contract) */
        float *st[2][3];
        uint16_t *out[2];
        for (int s = 0; s < 2; ++s) {
            for (int k = 0; k < 3; ++k)
                st[s][k] = (float *)calloc((size_t)(se + 4), sizeof(float)) + (s ? 0 : shift);
            out[s] = (uint16_t *)calloc((size_t)(oe + 4), sizeof(uint16_t)) + (s ? 0 : shift);
        }
        for (int64_t i = 0; i < se; ++i)
            st[0][0][i] = st[1][0][i] = rndf(0.02f);
        for (int t = 1; t <= 2; ++t) {
            zero_adamw_scalars sc;
            CHECK(zero_adamw_scalars_for(t, lr, b1, b2, eps, wd, 1.0f, &sc) == ZERO_OK);
            const zero_status zs = zero_step_host(
                L, rank, (const void *const *)gp, n, bf ? ZERO_BF16 : ZERO_F32,
                gl ? ZERO_LOCAL : ZERO_GLOBAL, (float)n, st[0][0], st[0][1], st[0][2],
                sg ? ZERO_GLOBAL : ZERO_LOCAL, out[0], og ? ZERO_GLOBAL : ZERO_LOCAL, &sc, threads);
            CHECK(zs == ZERO_OK);
            int rc;
            if (rank < 0)
                rc = orc_zero_step_all(n, U, numel, (const void *const *)gp, n, bf, (float)n, 1.0f,
                                       st[1][0], st[1][1], st[1][2], out[1], t, lr, b1, b2, eps, wd);
            else
                rc = orc_zero_step_rank(n, U, numel, rank, (const void *const *)gp, n, bf, gl,
                                        (float)n, 1.0f, st[1][0], st[1][1], st[1][2], sg, out[1],
                                        og, t, lr, b1, b2, eps, wd);
            CHECK(rc == 0);
        }
        /* only the selected elements are compared: the oracle writes exactly those */
        for (int k = 0; k < 3; ++k)
            CHECK(memcmp(st[0][k], st[1][k], (size_t)se * sizeof(float)) == 0);
        CHECK(memcmp(out[0], out[1], (size_t)oe * sizeof(uint16_t)) == 0);
        for (int s = 0; s < 2; ++s) {
            for (int k = 0; k < 3; ++k)
                free(st[s][k] - (s ? 0 : shift));
            free(out[s] - (s ? 0 : shift));
        }
        free(gbuf);
        free(L);
    }
}

/* the host reshard against the oracle: flat or row-aligned layouts, any N */
static void check_host_reshard(void)
{
    for (int it = 0; it < 120; ++it) {
        const int32_t P = (int32_t)rnd(1, 4);
        int64_t rows[4], cols[4], pnum[4];
        int64_t total = 0;
        for (int p = 0; p < P; ++p) {
            rows[p] = rnd(0, 9);
            cols[p] = rnd(1, 4);
            pnum[p] = rows[p] * cols[p];
            total += pnum[p];
        }
        /* A: the parameters as one flat unit; B: one row-aligned unit per parameter */
        int64_t a_numel[1] = {total};
        const int32_t na = (int32_t)rnd(1, 8), nb = (int32_t)rnd(1, 8);
        zero_layout *A = make_layout(na, 1, a_numel, NULL);
        zero_layout *B = make_layout(nb, P, pnum, cols);
        const int elem = it & 1 ? 2 : 4;
        unsigned char *src = (unsigned char *)malloc((size_t)(na * A->shard * elem) + 1);
        const void *sp[8];
        for (int q = 0; q < na; ++q) {
            sp[q] = src + (size_t)q * A->shard * elem;
            for (int64_t i = 0; i < A->shard * elem; ++i)
                ((unsigned char *)sp[q])[i] = (unsigned char)next_u64();
        }
        for (int32_t r = 0; r < nb; ++r) {
            unsigned char *d0 = (unsigned char *)malloc((size_t)(B->shard * elem) + 1);
            unsigned char *d1 = (unsigned char *)malloc((size_t)(B->shard * elem) + 1);
            CHECK(zero_reshard_host(A, sp, B, r, d0, elem == 4 ? ZERO_F32 : ZERO_BF16) == ZERO_OK);
            CHECK(orc_reshard(1, a_numel, na, NULL, sp, P, pnum, nb, cols, r, d1, elem) == 0);
            CHECK(memcmp(d0, d1, (size_t)(B->shard * elem)) == 0);
            free(d0);
            free(d1);
        }
        CHECK(zero_reshard_host(A, sp, B, nb, NULL, ZERO_F32) == ZERO_EINVAL);
        free(src);
        free(A);
        free(B);
    }
}

/* sharded checkpoint: every rank's shard saved, each rank of another layout
 * loaded (resharded at load time) and compared with the oracle's reshard of
 * the saved arrays; then the error paths */
static void check_checkpoint(void)
{
    char dir[] = "/tmp/zero_ckpt_sanXXXXXX";
    CHECK(mkdtemp(dir) != NULL);
    char path[8][128];
    const char *paths[8];
    for (int it = 0; it < 30; ++it) {
        const int32_t P = (int32_t)rnd(1, 4);
        int64_t rows[4], cols[4], pnum[4], total = 0;
        for (int p = 0; p < P; ++p) {
            rows[p] = rnd(0, 9);
            cols[p] = rnd(1, 4);
            pnum[p] = rows[p] * cols[p];
            total += pnum[p];
        }
        int64_t a_numel[1] = {total};
        const int32_t na = (int32_t)rnd(1, 8), nb = (int32_t)rnd(1, 8);
        zero_layout *A = make_layout(na, 1, a_numel, NULL);
        zero_layout *B = make_layout(nb, P, pnum, cols);
        float *src = (float *)malloc(sizeof(float) * (size_t)(3 * na * A->shard + 1));
        const void *sp[3][8];
        for (int q = 0; q < na; ++q) {
            for (int a = 0; a < 3; ++a) {
                float *x = src + (size_t)(3 * q + a) * A->shard;
                for (int64_t i = 0; i < A->shard; ++i)
                    x[i] = rndf(1.0f);
                /* the padding holds zeros, as the step keeps it */
                const int64_t live = total - (int64_t)q * A->shard;
                for (int64_t i = live < 0 ? 0 : live; i < A->shard; ++i)
                    x[i] = 0.0f;
                sp[a][q] = x;
            }
            snprintf(path[q], sizeof path[q], "%s/r%d.zck", dir, q);
            paths[q] = path[q];
            CHECK(zero_ckpt_save(paths[q], A, q, it + 1, (const float *)sp[0][q],
                                 (const float *)sp[1][q], (const float *)sp[2][q]) == ZERO_OK);
        }
        zero_ckpt_info info;
        size_t need = 0;
        CHECK(zero_ckpt_inspect(paths[0], 1, &info, NULL, 0, &need) == ZERO_OK);
        CHECK(info.n_ranks == na && info.step == it + 1 && info.shard == A->shard);
        for (int32_t r = 0; r < nb; ++r) {
            float *d = (float *)malloc(sizeof(float) * (size_t)(3 * B->shard + 1));
            float *e = (float *)malloc(sizeof(float) * (size_t)(B->shard + 1));
            int32_t step = -1;
            CHECK(zero_ckpt_load(paths, na, B, r, 1, &step, d, d + B->shard, d + 2 * B->shard) == ZERO_OK);
            CHECK(step == it + 1);
            for (int a = 0; a < 3; ++a) {
                CHECK(orc_reshard(1, a_numel, na, NULL, sp[a], P, pnum, nb, cols, r, e, 4) == 0);
                CHECK(memcmp(d + (size_t)a * B->shard, e, sizeof(float) * (size_t)B->shard) == 0);
            }
            free(d);
            free(e);
        }
        if (na > 1) {
            const char *swapped[8];
            for (int q = 0; q < na; ++q)
                swapped[q] = paths[q == 0 ? 1 : q == 1 ? 0 : q];
            float dummy[1];
            CHECK(zero_ckpt_load(swapped, na, B, 0, 0, NULL, dummy, dummy, dummy) == ZERO_EINVAL);
        }
        for (int q = 0; q < na; ++q)
            remove(paths[q]);
        free(src);
        free(A);
        free(B);
    }
    CHECK(zero_ckpt_inspect("/nonexistent/zero.zck", 0, &(zero_ckpt_info){0}, NULL, 0, NULL) == ZERO_EIO);
    rmdir(dir);
}

/* argument errors of the device entry points: rejected before any device work */
static void check_device_validation(void)
{
    const int64_t numel[2] = {1000, 17};
    zero_layout *L = make_layout(8, 2, numel, NULL);
    zero_adamw_scalars sc;
    CHECK(zero_adamw_scalars_for(1, 3e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, &sc) == ZERO_OK);
    char *base = (char *)(uintptr_t)0x100000000ull; /* fake device addresses, never dereferenced */
    const void *g[8];
    for (int q = 0; q < 8; ++q)
        g[q] = base + (size_t)q * 0x10000;
    float *w = (float *)(base + 0x100000), *m = (float *)(base + 0x200000);
    float *v = (float *)(base + 0x300000);
    uint16_t *o = (uint16_t *)(base + 0x400000);
    const int G = ZERO_GLOBAL, Lc = ZERO_LOCAL;
    CHECK(zero_step(L, -1, NULL, 8, ZERO_BF16, G, 8.0f, w, m, v, G, o, G, &sc, NULL) == ZERO_EINVAL);
    /* unit ranges: outside the layout refused; an empty range (NULL buckets) is a no-op */
    CHECK(zero_step_units(L, -1, 1, 0, g, 8, ZERO_BF16, G, 8.0f, w, m, v, G, o, G, &sc, NULL, 0,
                          NULL) == ZERO_EINVAL);
    CHECK(zero_step_units(L, -1, 0, 3, g, 8, ZERO_BF16, G, 8.0f, w, m, v, G, o, G, &sc, NULL, 0,
                          NULL) == ZERO_EINVAL);
    CHECK(zero_step_units(L, -1, -1, 1, g, 8, ZERO_BF16, G, 8.0f, w, m, v, G, o, G, &sc, NULL, 0,
                          NULL) == ZERO_EINVAL);
    {
        const void *none[8] = {0};
        CHECK(zero_step_units(L, 3, 1, 1, none, 8, ZERO_BF16, Lc, 8.0f, w, m, v, Lc, o, Lc, &sc,
                              NULL, 0, NULL) == ZERO_OK);
        CHECK(zero_step_units(L, 3, 0, 1, none, 8, ZERO_BF16, Lc, 8.0f, w, m, v, Lc, o, Lc, &sc,
                              NULL, 0, NULL) == ZERO_EINVAL);
    }
    CHECK(zero_step(L, -1, g, 0, ZERO_BF16, G, 8.0f, w, m, v, G, o, G, &sc, NULL) == ZERO_ERANGE);
    CHECK(zero_step(L, -1, g, 8, 7, G, 8.0f, w, m, v, G, o, G, &sc, NULL) == ZERO_EINVAL);
    CHECK(zero_step(L, -1, g, 8, ZERO_BF16, Lc, 8.0f, w, m, v, G, o, G, &sc, NULL) == ZERO_EINVAL);
    CHECK(zero_step(L, 8, g, 8, ZERO_BF16, Lc, 8.0f, w, m, v, Lc, o, Lc, &sc, NULL) == ZERO_EINVAL);
    CHECK(zero_step(L, 0, g, 8, ZERO_BF16, Lc, 0.0f, w, m, v, Lc, o, Lc, &sc, NULL) == ZERO_EINVAL);
    CHECK(zero_step(L, 0, g, 8, ZERO_BF16, Lc, 8.0f, w, w, v, Lc, o, Lc, &sc, NULL) == ZERO_EINVAL);
    CHECK(zero_step(L, 0, g, 8, ZERO_BF16, Lc, 8.0f, (float *)(base + 0x100002), m, v, Lc, o, Lc,
                    &sc, NULL) == ZERO_EALIGN);
    CHECK(zero_step(L, -1, g, 8, ZERO_BF16, G, 8.0f, (float *)g[0], m, v, G, o, G, &sc, NULL) ==
          ZERO_EINVAL);
    CHECK(zero_step_device_clip(L, 0, g, 8, ZERO_BF16, Lc, 8.0f, w, m, v, Lc, o, Lc, &sc, NULL,
                                NULL) == ZERO_EINVAL);
    size_t wsb = 0;
    CHECK(zero_gradnorm_workspace_bytes(L, 0, &wsb) == ZERO_OK);
    double ss = 0;
    void *ws = base + 0x800000;
    CHECK(zero_gradnorm(L, 0, g, 8, ZERO_BF16, Lc, 8.0f, NULL, Lc, ws, wsb - 8, &ss, NULL) ==
          ZERO_ENOSPC);
    CHECK(zero_gradnorm(L, 0, g, 8, ZERO_BF16, Lc, 8.0f, NULL, Lc, NULL, wsb, &ss, NULL) ==
          ZERO_EINVAL);
    CHECK(zero_gradnorm_async(L, 0, g, 8, ZERO_BF16, Lc, 8.0f, NULL, Lc, ws, wsb, NULL, NULL) ==
          ZERO_EINVAL);
    CHECK(zero_clip_coef_async(NULL, 1.0, NULL, NULL) == ZERO_EINVAL);
    CHECK(zero_clip_coef_ranks_async(NULL, 8, 1.0, NULL, NULL, NULL) == ZERO_EINVAL);
    const int64_t pn[2] = {1000, 17};
    const int32_t pu[2] = {0, 1};
    CHECK(zero_pack_copy(L, -1, 2, g, pn, pu, ZERO_F32, NULL, ZERO_F32, NULL) == ZERO_EINVAL);
    const int64_t bad[2] = {999, 17};
    CHECK(zero_pack_copy(L, -1, 2, g, bad, pu, ZERO_F32, w, ZERO_F32, NULL) == ZERO_EINVAL);
    CHECK(zero_reshard(L, g, L, 8, w, ZERO_F32, NULL) == ZERO_EINVAL);
    CHECK(zero_offload_step(L, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, &sc, 1, NULL,
                            NULL) == ZERO_EINVAL);
    /* the staged step (up to 32 gradients it runs fused, so the workspace checks need more) */
    const int64_t n64[1] = {64 * 1000};
    zero_layout *L64 = make_layout(64, 1, n64, NULL);
    const void *g64[64];
    for (int q = 0; q < 64; ++q)
        g64[q] = base + 0x10000000 + (size_t)q * 0x10000; /* clear of w, m, v, o and wsp */
    size_t sb = 0;
    /* one chunk of whole 512-element tiles, plus 4 elements to place it at the state's phase */
    CHECK(zero_step_staged_workspace_bytes(L64, 0, 64, &sb) == ZERO_OK && sb == (1024 + 4) * 4);
    size_t sb8 = 1;
    CHECK(zero_step_staged_workspace_bytes(L64, 0, 8, &sb8) == ZERO_OK && sb8 == 0);
    void *wsp = base + 0x2000000;
    CHECK(zero_step_staged(L64, 0, g64, 64, ZERO_BF16, Lc, 64.0f, w, m, v, Lc, o, Lc, &sc, NULL,
                           sb, NULL) == ZERO_EINVAL);
    CHECK(zero_step_staged(L64, 0, g64, 64, ZERO_BF16, Lc, 64.0f, w, m, v, Lc, o, Lc, &sc,
                           (char *)wsp + 4, sb, NULL) == ZERO_EALIGN);
    CHECK(zero_step_staged(L64, 0, g64, 64, ZERO_BF16, Lc, 64.0f, w, m, v, Lc, o, Lc, &sc, wsp, 100,
                           NULL) == ZERO_ENOSPC);
    CHECK(zero_step_staged(L64, 0, g64, 64, ZERO_BF16, Lc, 64.0f, w, m, v, Lc, o, Lc, &sc,
                           (void *)w, sb, NULL) == ZERO_EINVAL);
    CHECK(zero_step_staged(L64, 0, g64, 0, ZERO_BF16, Lc, 64.0f, w, m, v, Lc, o, Lc, &sc, wsp, sb,
                           NULL) == ZERO_ERANGE);
    free(L64);
    free(L);
}

int main(void)
{
    check_layouts();
    check_scalars_ledger_arena();
    check_host_step();
    check_host_reshard();
    check_checkpoint();
    check_device_validation();
    printf("ok\n");
    return 0;
}
