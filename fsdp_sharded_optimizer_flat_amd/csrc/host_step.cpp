// host_step.cpp -- the sharded optimizer step on host cores, for ZeRO-Offload.
//
// "Learn: ZeRO & FSDP", section 6: ZeRO-Offload keeps the optimizer state and
// runs the fp32 optimizer step on the CPU; gradients come down from the GPU
// and updated parameters go back.  "ZeRO and FSDP sharding", Implementation
// notes: offload trades PCIe bandwidth for capacity.
//
// Same selection, index rules and arithmetic as the GPU step (rank-ordered
// binary32 sum, average, clip, AdamW, bf16 round-to-nearest-even), eight
// elements at a time with AVX2.  The file is compiled with -mavx2 and without
// FMA or fast-math, so every add / mul / div / sqrt below is one correctly
// rounded IEEE binary32 operation, exactly as on the GPU.  Worker threads
// take contiguous element ranges; the step is elementwise, so the result does
// not depend on the thread count.
#include <immintrin.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "zero_internal.h"

namespace zero {
namespace {

struct HostJob {
    const void *const *grads;
    int n;
    bool bf16;
    float *w, *m, *v;
    uint16_t *out;
    StepConsts c;
};

// One element, scalar: heads and tails of the 8-wide loop.
inline float h_grad(const void *base, bool bf16, int64_t i)
{
    if (bf16) {
        const uint32_t b = (uint32_t)static_cast<const uint16_t *>(base)[i] << 16;
        float f;
        std::memcpy(&f, &b, 4);
        return f;
    }
    return static_cast<const float *>(base)[i];
}

inline uint16_t h_bf16(float x)
{
    uint32_t b;
    std::memcpy(&b, &x, 4);
    if ((b & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((b >> 16) | 0x0040u);  // NaN stays a (quiet) NaN
    return (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}

void scalar_element(const HostJob &j, int64_t gi, int64_t si, int64_t oi)
{
    float s = h_grad(j.grads[0], j.bf16, gi);
    for (int q = 1; q < j.n; ++q)
        s = s + h_grad(j.grads[q], j.bf16, gi);
    float g = j.c.div_pow2 ? s * j.c.inv_divisor : s / j.c.divisor;
    g = g * j.c.clip;
    float w = j.w[si], m = j.m[si], v = j.v[si];
    const float m_dec = j.c.b1 * m, m_inc = j.c.omb1 * g;
    m = m_dec + m_inc;
    const float v_dec = j.c.b2 * v, v_inc = (j.c.omb2 * g) * g;
    v = v_dec + v_inc;
    const float den = std::sqrt(v) / j.c.bc2 + j.c.eps;
    const float upd = (j.c.step_size * m) / den;
    const float w_dec = w * j.c.decay;
    w = w_dec - upd;
    j.w[si] = w;
    j.m[si] = m;
    j.v[si] = v;
    if (j.out)
        j.out[oi] = h_bf16(w);
}

inline __m256 load_grad8(const void *base, bool bf16, int64_t i)
{
    if (bf16) {
        const __m128i h = _mm_loadu_si128(reinterpret_cast<const __m128i *>(
            static_cast<const uint16_t *>(base) + i));
        return _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(h), 16));
    }
    return _mm256_loadu_ps(static_cast<const float *>(base) + i);
}

// bf16 round-to-nearest-even of 8 floats, packed to 8 uint16 in order.
inline __m128i bf16x8(__m256 x)
{
    const __m256i b = _mm256_castps_si256(x);
    const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(b, 16), _mm256_set1_epi32(1));
    __m256i r = _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(b, _mm256_set1_epi32(0x7fff)), lsb), 16);
    const __m256i mag = _mm256_and_si256(b, _mm256_set1_epi32(0x7fffffff));
    const __m256i nan = _mm256_cmpgt_epi32(mag, _mm256_set1_epi32(0x7f800000));
    const __m256i qnan = _mm256_or_si256(_mm256_srli_epi32(b, 16), _mm256_set1_epi32(0x0040));
    r = _mm256_blendv_epi8(r, qnan, nan);
    // 32 -> 16 bit: pack within 128-bit lanes, then put the two halves in order
    const __m256i packed = _mm256_packus_epi32(r, r);  // values are < 2^16
    const __m256i ordered = _mm256_permute4x64_epi64(packed, 0x08);  // qwords 0, 2
    return _mm256_castsi256_si128(ordered);
}

void run_range(const HostJob &j, const Segment &sg, int64_t a, int64_t b)
{
    const __m256 vb1 = _mm256_set1_ps(j.c.b1), vb2 = _mm256_set1_ps(j.c.b2);
    const __m256 vomb1 = _mm256_set1_ps(j.c.omb1), vomb2 = _mm256_set1_ps(j.c.omb2);
    const __m256 vbc2 = _mm256_set1_ps(j.c.bc2), veps = _mm256_set1_ps(j.c.eps);
    const __m256 vstep = _mm256_set1_ps(j.c.step_size), vdecay = _mm256_set1_ps(j.c.decay);
    const __m256 vclip = _mm256_set1_ps(j.c.clip), vinv = _mm256_set1_ps(j.c.inv_divisor);
    const __m256 vdiv = _mm256_set1_ps(j.c.divisor);
    int64_t e = a;
    for (; e + 8 <= b; e += 8) {
        const int64_t gi = sg.g_off + e, si = sg.s_off + e, oi = sg.o_off + e;
        __m256 s = load_grad8(j.grads[0], j.bf16, gi);
        for (int q = 1; q < j.n; ++q)
            s = _mm256_add_ps(s, load_grad8(j.grads[q], j.bf16, gi));
        __m256 g = j.c.div_pow2 ? _mm256_mul_ps(s, vinv) : _mm256_div_ps(s, vdiv);
        g = _mm256_mul_ps(g, vclip);
        __m256 w = _mm256_loadu_ps(j.w + si), m = _mm256_loadu_ps(j.m + si),
               v = _mm256_loadu_ps(j.v + si);
        m = _mm256_add_ps(_mm256_mul_ps(vb1, m), _mm256_mul_ps(vomb1, g));
        v = _mm256_add_ps(_mm256_mul_ps(vb2, v), _mm256_mul_ps(_mm256_mul_ps(vomb2, g), g));
        const __m256 den = _mm256_add_ps(_mm256_div_ps(_mm256_sqrt_ps(v), vbc2), veps);
        const __m256 upd = _mm256_div_ps(_mm256_mul_ps(vstep, m), den);
        w = _mm256_sub_ps(_mm256_mul_ps(w, vdecay), upd);
        _mm256_storeu_ps(j.w + si, w);
        _mm256_storeu_ps(j.m + si, m);
        _mm256_storeu_ps(j.v + si, v);
        if (j.out)
            _mm_storeu_si128(reinterpret_cast<__m128i *>(j.out + oi), bf16x8(w));
    }
    for (; e < b; ++e)
        scalar_element(j, sg.g_off + e, sg.s_off + e, sg.o_off + e);
}

}  // namespace
}  // namespace zero

using namespace zero;

extern "C" zero_status zero_step_host(const zero_layout *L, int32_t rank,
                                      const void *const *grads, int32_t n_grads,
                                      int32_t grad_dtype, int32_t grad_index, float divisor,
                                      float *master, float *exp_avg, float *exp_avg_sq,
                                      int32_t state_index, uint16_t *out, int32_t out_index,
                                      const zero_adamw_scalars *sc, int32_t n_threads)
{
    zero_status st = validate_step(L, rank, grads, n_grads, grad_dtype, grad_index, divisor,
                                   master, exp_avg, exp_avg_sq, state_index, out, out_index, sc);
    if (st != ZERO_OK)
        return st;
    HostJob j{};
    j.grads = grads;
    j.n = n_grads;
    j.bf16 = grad_dtype == ZERO_BF16;
    j.w = master;
    j.m = exp_avg;
    j.v = exp_avg_sq;
    j.out = out;
    j.c = make_step_consts(sc, divisor);
    const std::vector<Segment> segs = build_segments(L, rank, grad_index, state_index, out_index);
    int64_t total = 0;
    for (const Segment &s : segs)
        total += s.len;
    if (total == 0)
        return ZERO_OK;
    int nt = n_threads > 0 ? n_threads : (int)std::thread::hardware_concurrency();
    if (nt < 1)
        nt = 1;
    // at least 64 Ki elements per thread: below that, thread start-up dominates
    const int64_t max_threads = std::max<int64_t>(1, total / 65536);
    if (nt > max_threads)
        nt = (int)max_threads;
    // thread t owns elements [t*total/nt, (t+1)*total/nt) of the concatenated
    // segments, rounded to multiples of 8 so every range but the last is whole
    // vectors (the result is the same for any split: the step is elementwise)
    auto work = [&](int t) {
        int64_t lo = (total * t / nt) / 8 * 8, hi = t + 1 == nt ? total : (total * (t + 1) / nt) / 8 * 8;
        int64_t base = 0;
        for (const Segment &s : segs) {
            const int64_t a = std::max<int64_t>(lo, base), b = std::min<int64_t>(hi, base + s.len);
            if (a < b)
                run_range(j, s, a - base, b - base);
            base += s.len;
        }
    };
    if (nt == 1) {
        work(0);
        return ZERO_OK;
    }
    std::vector<std::thread> pool;
    pool.reserve((size_t)nt - 1);
    for (int t = 1; t < nt; ++t)
        pool.emplace_back(work, t);
    work(0);
    for (auto &th : pool)
        th.join();
    return ZERO_OK;
}
