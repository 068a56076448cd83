/*
 * oracle.c -- plain serial CPU oracle for the ZeRO sharded AdamW step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path (the HIP
 * library and its Python binding) never calls, links or imports it, and this
 * file includes no header and shares no helper, table or constant with it.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC
 *   - no fused multiply-add: every + - * / sqrt below rounds once, to
 *     nearest-even, in IEEE binary32 (x86-64 SSE arithmetic, FLT_EVAL_METHOD 0);
 *   - default MXCSR, so binary32 subnormals are kept (no flush-to-zero).
 *
 * What it computes (cited by page title and section; the pages are
 *   p1 "ZeRO and FSDP sharding" (tirogla.com),
 *   p3 "ZeRO: Three Ledgers, Zero Redundancy" (dominator-index.github.io),
 *   p4 "Learn: ZeRO & FSDP" (gunjandhanuka.github.io)):
 *
 *   layout      p1 "How it works" and "Pitfalls": each unit's parameters are
 *               flattened into one buffer padded to a multiple of N ranks, and
 *               rank r owns the r-th equal slice of every unit.
 *   step        p1 "Code": reduce-scatter (rank r receives the rank-ordered sum
 *               of every rank's gradient over its slice), divide by N, AdamW with
 *               decoupled weight decay and bias corrections on the fp32 master
 *               slice, then all-gather; p1 "How it works": the updated master is
 *               cast to bf16 for the gather.
 *   invariant   p1 "Code": the sharded result equals plain unsharded AdamW on
 *               the rank-averaged gradient, bit for bit.
 *   clip        p1 "Implementation notes": the global norm is the sum of the
 *               shards' squared norms; the coefficient follows the convention
 *               of the clip_grad_norm_ routine that note names.
 *   ledger      p4 section 3 (16 bytes per parameter) and section 4 (per-stage
 *               memory and communication); p3 section 4 (gradients transient).
 *
 * Fixed by p1 "Code" itself: its update lines are Rust binary32 expressions,
 * where * and / are left-associative, so v's increment is ((1 - b2) * g) * g
 * and the update is ((lr / bc1) * m) / (sqrt(v) / bc2 + eps), both true
 * divisions; the weight decays before the update is subtracted.
 *
 * Readings where the pages leave a step open (each is listed with its reason
 * in the design notes of the repository):
 *   - rank sum starts from rank 0's value and adds ranks 1..N-1 in order;
 *   - beta^t is the running binary32 product p_t = p_{t-1} * beta, p_0 = 1;
 *   - 1 - beta is formed in binary32 from the binary32 beta;
 *   - the bf16 cast rounds to nearest, ties to even;
 *   - padding elements are processed like any other (they stay +0);
 *   - the sum of squares adds the binary64 squares serially in element order
 *     (the pages fix no order for it; a serial sum of n terms is exact to
 *     n * 2^-53 relative, so at large n tests hold the device's sum to an
 *     accurate pairwise binary64 sum and this one to that bound).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-2)

/* ------------------------------------------------------------------------ */
/* Layout: p1 "How it works" (pad to a multiple of N, rank r owns slice r),  */
/* p1 "Pitfalls" (the flat numel must divide by N).                          */
/* ------------------------------------------------------------------------ */

/* For every unit u: padded[u] = the smallest multiple of n that is >= numel[u];
 * shard[u] = padded[u] / n; offset[u] = where unit u starts in the padded flat
 * buffer; local_offset[u] = where unit u's slice starts inside one rank's local
 * shard (the concatenation of that rank's slice of every unit, in unit order). */
int orc_layout(int32_t n, int32_t n_units, const int64_t *numel,
               int64_t *padded, int64_t *shard, int64_t *offset,
               int64_t *local_offset, int64_t *total_padded,
               int64_t *total_shard)
{
    if (n < 1 || n_units < 0)
        return ORC_EINVAL;
    int64_t next_offset = 0, next_local = 0;
    for (int32_t u = 0; u < n_units; ++u) {
        if (numel[u] < 0)
            return ORC_EINVAL;
        int64_t p = numel[u];
        while (p % n != 0)     /* pad one element at a time: obviously minimal */
            p += 1;
        padded[u] = p;
        shard[u] = p / n;
        offset[u] = next_offset;
        local_offset[u] = next_local;
        next_offset += padded[u];
        next_local += shard[u];
    }
    *total_padded = next_offset;
    *total_shard = next_local;
    return ORC_OK;
}

/* Global flat index of element k of rank r's local shard. */
int64_t orc_global_of_local(int32_t n_units, const int64_t *shard,
                            const int64_t *offset, const int64_t *local_offset,
                            int32_t r, int64_t k)
{
    for (int32_t u = 0; u < n_units; ++u)
        if (k >= local_offset[u] && k < local_offset[u] + shard[u])
            return offset[u] + (int64_t)r * shard[u] + (k - local_offset[u]);
    return -1;
}

/* Owning rank and local index of global flat index j. */
int orc_owner_of_global(int32_t n, int32_t n_units, const int64_t *shard,
                        const int64_t *offset, const int64_t *local_offset,
                        int64_t j, int32_t *rank, int64_t *k)
{
    for (int32_t u = 0; u < n_units; ++u) {
        int64_t unit_len = shard[u] * n;
        if (j >= offset[u] && j < offset[u] + unit_len) {
            int64_t within = j - offset[u];
            *rank = (int32_t)(within / shard[u]);
            *k = local_offset[u] + within % shard[u];
            return ORC_OK;
        }
    }
    return ORC_EINVAL;
}

/* Row-aligned layout: p4 section 5, "FSDP1 vs FSDP2" (FSDP2 keeps each
 * parameter as its own tensor, chunked along dim 0); p3's note after its
 * section 5 names this row-aligned sharding.  Unit u is one parameter
 * of rows[u] = numel[u] / row_len[u] rows; torch.chunk over the rows gives
 * every rank ceil(rows / n) rows (the last ranks fewer, or none), and FSDP2
 * pads each rank's piece to that many rows.  So the unit is padded one whole
 * row at a time until the row count divides by n, and rank r's slice is rows
 * [r c, (r + 1) c), c = padded rows / n.  The outputs mean what they mean in
 * orc_layout; row_len[u] must divide numel[u]. */
int orc_layout_rows(int32_t n, int32_t n_units, const int64_t *numel,
                    const int64_t *row_len, int64_t *padded, int64_t *shard,
                    int64_t *offset, int64_t *local_offset,
                    int64_t *total_padded, int64_t *total_shard)
{
    if (n < 1 || n_units < 0)
        return ORC_EINVAL;
    int64_t next_offset = 0, next_local = 0;
    for (int32_t u = 0; u < n_units; ++u) {
        if (numel[u] < 0 || row_len[u] < 1 || numel[u] % row_len[u] != 0)
            return ORC_EINVAL;
        int64_t rows = numel[u] / row_len[u];
        while (rows % n != 0)   /* pad one row at a time */
            rows += 1;
        padded[u] = rows * row_len[u];
        shard[u] = padded[u] / n;
        offset[u] = next_offset;
        local_offset[u] = next_local;
        next_offset += padded[u];
        next_local += shard[u];
    }
    *total_padded = next_offset;
    *total_shard = next_local;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* bfloat16 rounding (p1 "How it works": the updated master is cast to bf16). */
/* ------------------------------------------------------------------------ */

/* Magnitude of a non-negative bfloat16 bit pattern p <= 0x7f80 as a double.
 * 0x7f80 is given the value 2^128, the next power of two past the largest
 * finite bf16: rounding to nearest overflows to infinity exactly when that
 * unbounded-exponent neighbour is the nearer one. */
static double bf16_magnitude(uint32_t p)
{
    uint32_t e = p >> 7, f = p & 0x7fu;
    if (e == 0)
        return ldexp((double)f, -133);          /* f * 2^-7 * 2^-126 */
    return ldexp((double)(128u + f), (int)e - 134);  /* 1.f * 2^(e-127) */
}

/* Nearest bfloat16 to x, ties to the pattern with an even last bit.  NaN maps
 * to a quiet NaN with x's sign; only NaN-ness is part of the contract.  */
uint16_t orc_bf16(float x)
{
    uint32_t bits;
    memcpy(&bits, &x, sizeof bits);
    uint32_t sign = bits & 0x80000000u, mag = bits & 0x7fffffffu;
    if (mag > 0x7f800000u)
        return (uint16_t)((sign >> 16) | 0x7fc0u);
    if (mag == 0x7f800000u)
        return (uint16_t)(bits >> 16);
    uint32_t below = mag >> 16;                 /* largest bf16 magnitude <= |x| */
    uint32_t above = below + 1;                 /* next bf16 magnitude up */
    double ax = fabs((double)x);
    double d_below = ax - bf16_magnitude(below);  /* both differences exact */
    double d_above = bf16_magnitude(above) - ax;
    uint32_t pick;
    if (d_below < d_above)
        pick = below;
    else if (d_above < d_below)
        pick = above;
    else
        pick = (below & 1u) ? above : below;
    return (uint16_t)((sign >> 16) | pick);
}

void orc_bf16_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16(x[i]);
}

/* binary32 value of a bf16 pattern (exact widening). */
static float bf16_to_f32(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* ------------------------------------------------------------------------ */
/* AdamW (p1 "Code": AdamW with b1, b2, eps, decoupled weight decay wd,      */
/* step counter t starting at 1, bias corrections 1 - b1^t and               */
/* sqrt(1 - b2^t)).                                                         */
/* ------------------------------------------------------------------------ */

typedef struct {
    float b1, b2, eps;
    float one_minus_b1, one_minus_b2;
    float pow1, pow2;        /* b1^t, b2^t as running binary32 products */
    float bc1, bc2;          /* 1 - b1^t ; sqrt(1 - b2^t) */
    float lr_over_bc1;       /* lr / bc1 */
    float decay;             /* 1 - lr * wd */
} orc_hyper;

static void orc_hyper_for_step(int32_t t, float lr, float b1, float b2,
                               float eps, float wd, orc_hyper *h)
{
    float pow1 = 1.0f, pow2 = 1.0f;
    for (int32_t i = 0; i < t; ++i) {
        pow1 = pow1 * b1;
        pow2 = pow2 * b2;
    }
    h->b1 = b1;
    h->b2 = b2;
    h->eps = eps;
    h->one_minus_b1 = 1.0f - b1;
    h->one_minus_b2 = 1.0f - b2;
    h->pow1 = pow1;
    h->pow2 = pow2;
    h->bc1 = 1.0f - pow1;
    float one_minus_pow2 = 1.0f - pow2;
    h->bc2 = sqrtf(one_minus_pow2);
    h->lr_over_bc1 = lr / h->bc1;
    float lr_wd = lr * wd;
    h->decay = 1.0f - lr_wd;
}

/* The step scalars, exported so tests can pin them:
 * out = {1-b1, 1-b2, b1^t, b2^t, bc1, bc2, lr/bc1, 1-lr*wd}. */
void orc_adamw_scalars(int32_t t, float lr, float b1, float b2, float wd,
                       float *out)
{
    orc_hyper h;
    orc_hyper_for_step(t, lr, b1, b2, 1e-8f, wd, &h);
    out[0] = h.one_minus_b1;
    out[1] = h.one_minus_b2;
    out[2] = h.pow1;
    out[3] = h.pow2;
    out[4] = h.bc1;
    out[5] = h.bc2;
    out[6] = h.lr_over_bc1;
    out[7] = h.decay;
}

/* One element of AdamW: updates master w, first moment m, second moment v
 * with gradient g.  One rounding per operation, in the order written. */
static void adamw_element(float *w, float *m, float *v, float g,
                          const orc_hyper *h)
{
    /* m <- b1 m + (1 - b1) g */
    float m_decayed = h->b1 * (*m);
    float m_incr = h->one_minus_b1 * g;
    *m = m_decayed + m_incr;
    /* v <- b2 v + ((1 - b2) g) g */
    float v_decayed = h->b2 * (*v);
    float v_incr = (h->one_minus_b2 * g) * g;
    *v = v_decayed + v_incr;
    /* denominator sqrt(v) / bc2 + eps; update (lr / bc1) m / denominator */
    float root = sqrtf(*v);
    float den = root / h->bc2 + h->eps;
    float numer = h->lr_over_bc1 * (*m);
    float update = numer / den;
    /* decoupled weight decay, then the Adam update */
    float w_decayed = (*w) * h->decay;
    *w = w_decayed - update;
}

/* Per-element AdamW over a plain vector (no sharding), exported so tests can
 * compare it with other AdamW implementations. */
void orc_adamw_vector(int64_t n, float *w, float *m, float *v, const float *g,
                      int32_t t, float lr, float b1, float b2, float eps,
                      float wd)
{
    orc_hyper h;
    orc_hyper_for_step(t, lr, b1, b2, eps, wd, &h);
    for (int64_t i = 0; i < n; ++i)
        adamw_element(&w[i], &m[i], &v[i], g[i], &h);
}

/* ------------------------------------------------------------------------ */
/* The sharded step, structured as the pages' ZeRO step (p1 "Code"):        */
/*   reduce-scatter -> / N -> (clip) -> AdamW on my slice -> all-gather.     */
/* ------------------------------------------------------------------------ */

static float load_grad(const void *buf, int32_t is_bf16, int64_t idx)
{
    if (is_bf16)
        return bf16_to_f32(((const uint16_t *)buf)[idx]);
    return ((const float *)buf)[idx];
}

typedef struct {
    int32_t n, n_units;
    int64_t *padded, *shard, *offset, *local_offset;
    int64_t total_padded, total_shard;
} orc_lay;

static int lay_make(int32_t n, int32_t n_units, const int64_t *numel,
                    orc_lay *L)
{
    L->n = n;
    L->n_units = n_units;
    size_t bytes = sizeof(int64_t) * (size_t)(n_units > 0 ? n_units : 1);
    L->padded = malloc(bytes);
    L->shard = malloc(bytes);
    L->offset = malloc(bytes);
    L->local_offset = malloc(bytes);
    if (!L->padded || !L->shard || !L->offset || !L->local_offset)
        return ORC_ENOMEM;
    return orc_layout(n, n_units, numel, L->padded, L->shard, L->offset,
                      L->local_offset, &L->total_padded, &L->total_shard);
}

static void lay_free(orc_lay *L)
{
    free(L->padded);
    free(L->shard);
    free(L->offset);
    free(L->local_offset);
}

/* Either layout: row_len == NULL gives the flat layout (orc_layout). */
static int lay_make_any(int32_t n, int32_t n_units, const int64_t *numel,
                        const int64_t *row_len, orc_lay *L)
{
    if (!row_len)
        return lay_make(n, n_units, numel, L);
    L->n = n;
    L->n_units = n_units;
    size_t bytes = sizeof(int64_t) * (size_t)(n_units > 0 ? n_units : 1);
    L->padded = malloc(bytes);
    L->shard = malloc(bytes);
    L->offset = malloc(bytes);
    L->local_offset = malloc(bytes);
    if (!L->padded || !L->shard || !L->offset || !L->local_offset)
        return ORC_ENOMEM;
    return orc_layout_rows(n, n_units, numel, row_len, L->padded, L->shard,
                           L->offset, L->local_offset, &L->total_padded,
                           &L->total_shard);
}

/* Reshard: p1 "Implementation notes" (a checkpoint saved as per-rank shards
 * is resharded when loaded under a different N) and p4 section 5, "FSDP1 vs
 * FSDP2" (checkpoints carry over between the flat and per-parameter
 * layouts).  An element is named by its stream position: its index in all
 * units' unpadded elements laid end to end.  Layout A has units numel_a,
 * n_a ranks and row lengths row_a (NULL: flat); layout B likewise; both hold
 * the same number of elements.  src[q] is rank q's local shard in A; dst
 * receives rank dst_rank's local shard in B.  Element by element: local index
 * k of B -> B's global index -> (unit, position in the unit); a position at or
 * past the unit's numel is padding and becomes zero, any other gives a stream
 * position, which gives A's unit and position, A's global index and its owner
 * (rank, local index), read from src.  elem: bytes per element. */
int orc_reshard_span(int32_t units_a, const int64_t *numel_a, int32_t n_a,
                     const int64_t *row_a, const void *const *src,
                     int32_t units_b, const int64_t *numel_b, int32_t n_b,
                     const int64_t *row_b, int32_t dst_rank, int64_t k_begin,
                     int64_t k_end, void *dst, int32_t elem);

int orc_reshard(int32_t units_a, const int64_t *numel_a, int32_t n_a,
                const int64_t *row_a, const void *const *src, int32_t units_b,
                const int64_t *numel_b, int32_t n_b, const int64_t *row_b,
                int32_t dst_rank, void *dst, int32_t elem)
{
    return orc_reshard_span(units_a, numel_a, n_a, row_a, src, units_b, numel_b,
                            n_b, row_b, dst_rank, 0, -1, dst, elem);
}

/* The same for local indices k_begin <= k < k_end of the destination shard
 * only (k_end < 0: to the end); dst[k - k_begin] receives element k. */
int orc_reshard_span(int32_t units_a, const int64_t *numel_a, int32_t n_a,
                     const int64_t *row_a, const void *const *src,
                     int32_t units_b, const int64_t *numel_b, int32_t n_b,
                     const int64_t *row_b, int32_t dst_rank, int64_t k_begin,
                     int64_t k_end, void *dst, int32_t elem)
{
    if (dst_rank < 0 || dst_rank >= n_b || (elem != 2 && elem != 4))
        return ORC_EINVAL;
    int64_t total_a = 0, total_b = 0;
    for (int32_t u = 0; u < units_a; ++u)
        total_a += numel_a[u];
    for (int32_t u = 0; u < units_b; ++u)
        total_b += numel_b[u];
    if (total_a != total_b)
        return ORC_EINVAL;
    orc_lay A = {0}, B = {0};
    int st = lay_make_any(n_a, units_a, numel_a, row_a, &A);
    if (st == ORC_OK)
        st = lay_make_any(n_b, units_b, numel_b, row_b, &B);
    if (st == ORC_OK && k_end < 0)
        k_end = B.total_shard;
    if (st == ORC_OK && (k_begin < 0 || k_begin > k_end || k_end > B.total_shard))
        st = ORC_EINVAL;
    for (int64_t k = k_begin; st == ORC_OK && k < k_end; ++k) {
        int64_t j = orc_global_of_local(units_b, B.shard, B.offset,
                                        B.local_offset, dst_rank, k);
        int32_t u = 0;
        int64_t stream = 0;
        while (!(j >= B.offset[u] && j < B.offset[u] + B.padded[u])) {
            stream += numel_b[u];
            ++u;
        }
        int64_t pos = j - B.offset[u];
        char *d = (char *)dst + (k - k_begin) * elem;
        if (pos >= numel_b[u]) {
            memset(d, 0, (size_t)elem);
            continue;
        }
        stream += pos;
        int32_t w = 0;                       /* A's unit holding the position */
        while (stream >= numel_a[w]) {
            stream -= numel_a[w];
            ++w;
        }
        int32_t q;
        int64_t ka;
        st = orc_owner_of_global(n_a, units_a, A.shard, A.offset,
                                 A.local_offset, A.offset[w] + stream, &q, &ka);
        if (st == ORC_OK)
            memcpy(d, (const char *)src[q] + ka * elem, (size_t)elem);
    }
    lay_free(&A);
    lay_free(&B);
    return st;
}

/* One rank's step.
 *   grads[q], q = 0..n_grads-1: rank q's gradient.  grad_local == 0: rank q's
 *     whole padded flat gradient, indexed by the global index j.  grad_local
 *     == 1: the chunk rank q sends to rank r in the reduce-scatter, indexed by
 *     rank r's local index k.  Values are binary32 or bf16 (grad_bf16).
 *   divisor: the averaging divisor (N; 1 when the gradient is already reduced).
 *   clip: multiplier applied to the averaged gradient (1 = no clipping).
 *   master, m, v: rank r's state, indexed by k (state_global == 0) or by j.
 *   out: bf16 copy of the updated master, at j (out_gather == 1: the slot of
 *     the all-gather's output buffer) or at k; NULL skips it. */
int orc_zero_step_rank(int32_t n, int32_t n_units, const int64_t *numel,
                       int32_t r, const void *const *grads, int32_t n_grads,
                       int32_t grad_bf16, int32_t grad_local, float divisor,
                       float clip, float *master, float *m, float *v,
                       int32_t state_global, uint16_t *out, int32_t out_gather,
                       int32_t t, float lr, float b1, float b2, float eps,
                       float wd)
{
    if (r < 0 || r >= n || n_grads < 1)
        return ORC_EINVAL;
    orc_lay L;
    int rc = lay_make(n, n_units, numel, &L);
    if (rc != ORC_OK) {
        lay_free(&L);
        return rc;
    }
    orc_hyper h;
    orc_hyper_for_step(t, lr, b1, b2, eps, wd, &h);

    for (int32_t u = 0; u < n_units; ++u) {
        for (int64_t i = 0; i < L.shard[u]; ++i) {
            int64_t k = L.local_offset[u] + i;
            int64_t j = L.offset[u] + (int64_t)r * L.shard[u] + i;
            int64_t gi = grad_local ? k : j;
            /* reduce-scatter: the sum over ranks, in rank order */
            float sum = load_grad(grads[0], grad_bf16, gi);
            for (int32_t q = 1; q < n_grads; ++q)
                sum = sum + load_grad(grads[q], grad_bf16, gi);
            float g = sum / divisor;    /* average */
            g = g * clip;               /* global-norm clipping */
            int64_t si = state_global ? j : k;
            adamw_element(&master[si], &m[si], &v[si], g, &h);
            if (out)
                out[out_gather ? j : k] = orc_bf16(master[si]);
        }
    }
    lay_free(&L);
    return ORC_OK;
}

/* Every rank's step, one after another, with state and output indexed by the
 * global index j (the all-gathered view).  Rank r touches only its own slices,
 * so the result does not depend on the order the ranks run in. */
int orc_zero_step_all(int32_t n, int32_t n_units, const int64_t *numel,
                      const void *const *grads, int32_t n_grads,
                      int32_t grad_bf16, float divisor, float clip,
                      float *master, float *m, float *v, uint16_t *out,
                      int32_t t, float lr, float b1, float b2, float eps,
                      float wd)
{
    for (int32_t r = 0; r < n; ++r) {
        int rc = orc_zero_step_rank(n, n_units, numel, r, grads, n_grads,
                                    grad_bf16, 0, divisor, clip, master, m, v,
                                    1, out, 1, t, lr, b1, b2, eps, wd);
        if (rc != ORC_OK)
            return rc;
    }
    return ORC_OK;
}

/* The unsharded reference the sharded step must equal (p1 "Code"): plain
 * AdamW over the unpadded P-vector on the rank-averaged gradient.
 * grads[q] are unpadded P-vectors. */
void orc_adamw_unsharded(int64_t P, const void *const *grads, int32_t n_grads,
                         int32_t grad_bf16, float divisor, float clip,
                         float *w, float *m, float *v, int32_t t, float lr,
                         float b1, float b2, float eps, float wd)
{
    orc_hyper h;
    orc_hyper_for_step(t, lr, b1, b2, eps, wd, &h);
    for (int64_t i = 0; i < P; ++i) {
        float sum = load_grad(grads[0], grad_bf16, i);
        for (int32_t q = 1; q < n_grads; ++q)
            sum = sum + load_grad(grads[q], grad_bf16, i);
        float g = (sum / divisor) * clip;
        adamw_element(&w[i], &m[i], &v[i], g, &h);
    }
}

/* The averaged gradient over rank r's shard (the reduction half of the
 * reduce-scatter followed by the division), indexed by k. */
int orc_reduced_grad(int32_t n, int32_t n_units, const int64_t *numel,
                     int32_t r, const void *const *grads, int32_t n_grads,
                     int32_t grad_bf16, int32_t grad_local, float divisor,
                     float *g_out)
{
    if (r < 0 || r >= n || n_grads < 1)
        return ORC_EINVAL;
    orc_lay L;
    int rc = lay_make(n, n_units, numel, &L);
    if (rc != ORC_OK) {
        lay_free(&L);
        return rc;
    }
    for (int32_t u = 0; u < n_units; ++u)
        for (int64_t i = 0; i < L.shard[u]; ++i) {
            int64_t k = L.local_offset[u] + i;
            int64_t j = L.offset[u] + (int64_t)r * L.shard[u] + i;
            int64_t gi = grad_local ? k : j;
            float sum = load_grad(grads[0], grad_bf16, gi);
            for (int32_t q = 1; q < n_grads; ++q)
                sum = sum + load_grad(grads[q], grad_bf16, gi);
            g_out[k] = sum / divisor;
        }
    lay_free(&L);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Global gradient norm and clip coefficient (p1 "Implementation notes").    */
/* ------------------------------------------------------------------------ */

/* Sum of squares of g in index order, accumulated in binary64. */
double orc_sumsq(const float *g, int64_t n)
{
    double acc = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double x = (double)g[i];
        acc = acc + x * x;
    }
    return acc;
}

/* Clip coefficient: max_norm / (norm + 1e-6), capped at 1, computed in
 * binary64 and rounded once to binary32. */
float orc_clip_coef(double sumsq, double max_norm)
{
    double norm = sqrt(sumsq);
    double coef = max_norm / (norm + 1e-6);
    if (coef > 1.0)
        coef = 1.0;
    return (float)coef;
}

/* ------------------------------------------------------------------------ */
/* The pages' toy (p1 "Code"): N ranks, P parameters starting at 0, rank r's */
/* local loss 0.5 ||w - t_r||^2 with t_r[i] = (7 i + 13 r) mod 11, so its     */
/* gradient is w - t_r; lr 0.01, b1 0.9, b2 0.95, eps 1e-8, wd 0.1.          */
/* ------------------------------------------------------------------------ */

/* Runs `steps` sharded steps (P padded to a multiple of n, one unit) and
 * `steps` unsharded steps from the same start.  Writes the final gathered fp32
 * parameters of both (first P elements), the final bf16 gather (P elements)
 * and, per step, the sharded run's mean |w_i - mean_r t_r[i]| (binary64). */
int orc_toy(int32_t n, int64_t P, int32_t steps, float lr, float *w_sharded,
            float *w_unsharded, uint16_t *out_bf16, double *trace)
{
    const float b1 = 0.9f, b2 = 0.95f, eps = 1e-8f, wd = 0.1f;
    if (n < 1 || P < 0 || steps < 0)
        return ORC_EINVAL;
    orc_lay L;
    int64_t numel = P;
    int rc = lay_make(n, 1, &numel, &L);
    if (rc != ORC_OK) {
        lay_free(&L);
        return rc;
    }
    int64_t Ph = L.total_padded, S = L.total_shard;
    float *target = calloc((size_t)n * (size_t)(P > 0 ? P : 1), sizeof(float));
    float *w = calloc((size_t)(Ph > 0 ? Ph : 1), sizeof(float));  /* gathered */
    float *grad = calloc((size_t)n * (size_t)(Ph > 0 ? Ph : 1), sizeof(float));
    float *mst = calloc((size_t)n * (size_t)(S > 0 ? S : 1), sizeof(float));
    float *mm = calloc((size_t)n * (size_t)(S > 0 ? S : 1), sizeof(float));
    float *vv = calloc((size_t)n * (size_t)(S > 0 ? S : 1), sizeof(float));
    uint16_t *gath = calloc((size_t)(Ph > 0 ? Ph : 1), sizeof(uint16_t));
    const void **gp = calloc((size_t)n, sizeof(void *));
    float *wu = calloc((size_t)(P > 0 ? P : 1), sizeof(float));
    float *mu = calloc((size_t)(P > 0 ? P : 1), sizeof(float));
    float *vu = calloc((size_t)(P > 0 ? P : 1), sizeof(float));
    float *gu = calloc((size_t)n * (size_t)(P > 0 ? P : 1), sizeof(float));
    const void **gup = calloc((size_t)n, sizeof(void *));
    if (!target || !w || !grad || !mst || !mm || !vv || !gath || !gp || !wu ||
        !mu || !vu || !gu || !gup) {
        rc = ORC_ENOMEM;
        goto done;
    }
    for (int32_t r = 0; r < n; ++r)
        for (int64_t i = 0; i < P; ++i)
            target[(size_t)r * P + i] = (float)((i * 7 + (int64_t)r * 13) % 11);

    /* sharded run: each rank holds only its slice of master / m / v */
    for (int32_t s = 0; s < steps; ++s) {
        for (int32_t r = 0; r < n; ++r) {
            float *gr = grad + (size_t)r * Ph;
            for (int64_t j = 0; j < Ph; ++j)   /* padding has no loss: grad 0 */
                gr[j] = (j < P) ? w[j] - target[(size_t)r * P + j] : 0.0f;
            gp[r] = gr;
        }
        for (int32_t r = 0; r < n; ++r) {
            if (s == 0)   /* the master slice starts as my slice of w */
                for (int64_t k = 0; k < S; ++k)
                    mst[(size_t)r * S + k] = w[(int64_t)r * S + k];
            rc = orc_zero_step_rank(n, 1, &numel, r, gp, n, 0, 0, (float)n,
                                    1.0f, mst + (size_t)r * S,
                                    mm + (size_t)r * S, vv + (size_t)r * S, 0,
                                    gath, 1, s + 1, lr, b1, b2, eps, wd);
            if (rc != ORC_OK)
                goto done;
        }
        /* all-gather (fp32): w is the concatenation of the ranks' slices */
        for (int32_t r = 0; r < n; ++r)
            for (int64_t k = 0; k < S; ++k)
                w[(int64_t)r * S + k] = mst[(size_t)r * S + k];
        if (trace) {
            double acc = 0.0;
            for (int64_t i = 0; i < P; ++i) {
                double tbar = 0.0;
                for (int32_t r = 0; r < n; ++r)
                    tbar += target[(size_t)r * P + i];
                tbar /= n;
                acc += fabs((double)w[i] - tbar);
            }
            trace[s] = P > 0 ? acc / (double)P : 0.0;
        }
    }

    /* unsharded reference run */
    for (int32_t s = 0; s < steps; ++s) {
        for (int32_t r = 0; r < n; ++r) {
            float *gr = gu + (size_t)r * P;
            for (int64_t i = 0; i < P; ++i)
                gr[i] = wu[i] - target[(size_t)r * P + i];
            gup[r] = gr;
        }
        orc_adamw_unsharded(P, gup, n, 0, (float)n, 1.0f, wu, mu, vu, s + 1,
                            lr, b1, b2, eps, wd);
    }
    for (int64_t i = 0; i < P; ++i) {
        w_sharded[i] = w[i];
        w_unsharded[i] = wu[i];
        out_bf16[i] = gath[i];
    }
    rc = ORC_OK;
done:
    free(target); free(w); free(grad); free(mst); free(mm); free(vv);
    free(gath); free(gp); free(wu); free(mu); free(vu); free(gu); free(gup);
    lay_free(&L);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Memory and communication ledger (p4 sections 3-4, p3 section 4,          */
/* p1 "How it works").  psi = parameter count, n = data-parallel ranks.      */
/* ------------------------------------------------------------------------ */

/* Model-state bytes per GPU.  K = 12 optimizer bytes per parameter (fp32
 * master, m, v); 2 bytes of bf16 parameters; 2 bytes of bf16 gradients.
 * Stage 0 replicates all three, stage 1 shards the optimizer state, stage 2
 * also the gradients, stage 3 also the parameters.  grads_transient == 1
 * drops the gradient line (gradients streamed through bucketed
 * reduce-scatter and freed, as measured on p3). */
double orc_ledger_bytes(double psi, int32_t n, int32_t stage,
                        int32_t grads_transient)
{
    const double K = 12.0, param_b = 2.0, grad_b = 2.0;
    double params = psi * param_b, grads = psi * grad_b, optim = psi * K;
    if (stage >= 1)
        optim = optim / n;
    if (stage >= 2)
        grads = grads / n;
    if (stage >= 3)
        params = params / n;
    if (grads_transient)
        grads = 0.0;
    return params + grads + optim;
}

/* Bytes the one-GPU simulation keeps resident, from p4 section 3's bytes per
 * element (bf16 gradient 2, fp32 master + m + v 12, bf16 parameters 2) over
 * the simulation's buffers: n_grads gradients of grad_bytes per element, the
 * three state arrays, the bf16 output (with_out) and the clipped step's fp32
 * reduced gradient (with_g).  every_rank == 1: every rank's shards at once,
 * so each buffer spans the padded flat buffer; 0: one rank's local shard. */
double orc_sim_footprint(int32_t n, int32_t n_units, const int64_t *numel,
                         int32_t every_rank, int32_t n_grads, int32_t grad_bytes,
                         int32_t with_out, int32_t with_g)
{
    orc_lay L;
    if (lay_make(n, n_units, numel, &L) != ORC_OK) {
        lay_free(&L);
        return -1.0;
    }
    double elems = (double)(every_rank ? L.total_padded : L.total_shard);
    lay_free(&L);
    double per = (double)n_grads * grad_bytes + 12.0;
    if (with_out)
        per += 2.0;
    if (with_g)
        per += 4.0;
    return per * elems;
}

/* Elements communicated per step: all-reduce = reduce-scatter + all-gather =
 * 2 psi for stages 0-2; stage 3 gathers twice (forward, backward) and
 * reduce-scatters once = 3 psi.  exact_ring == 1 applies the (N-1)/N factor
 * of a ring collective. */
double orc_comm_elements(double psi, int32_t n, int32_t stage,
                         int32_t exact_ring)
{
    double passes = (stage >= 3) ? 3.0 : 2.0;
    double elems = passes * psi;
    if (exact_ring)
        elems = elems * (double)(n - 1) / (double)n;
    return elems;
}
