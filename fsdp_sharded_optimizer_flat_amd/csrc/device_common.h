// device_common.h -- device helpers shared by the step and norm kernels:
// the rank-ordered gradient sum over a chunk, the average, the AdamW element
// update and the bf16 packing.  gfx950 only.
//
// Bit-exactness rests on three things the build passes explicitly: no FMA
// contraction (-ffp-contract=off), IEEE binary32 denormals
// (-fno-gpu-flush-denormals-to-zero), and correctly rounded '/' and sqrtf
// (-fhip-fp32-correctly-rounded-divide-sqrt).
#pragma once

#include <hip/hip_runtime.h>

#include "zero_internal.h"

namespace zero {
namespace dev {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Gradient base pointers, passed by value in the kernel arguments so the
// rank loop reads them with scalar loads.  CAP is the compile-time rank
// count, or ZERO_MAX_RANKS for the runtime-count kernels.
template <int CAP>
struct GradSet {
    const void *p[CAP];
};

// Streaming loads: every byte is read once per step, so they bypass the
// caches' reuse policy (stores go through st_span below).
template <typename T>
__device__ __forceinline__ T ld_stream(const T *p)
{
    return __builtin_nontemporal_load(p);
}

// Store of one wave's contiguous span: lane l writes v at span[l], where
// `span` is the same for every lane of the wave.  It is issued as a raw
// buffer store whose resource (base `span`, 64 elements, held in scalar
// registers) confines it to the span, with the nontemporal and device-scope
// cache-policy bits (nt sc1).  MI355X's XCDs each have their own L2, so a
// device-scope store is written through to memory at once instead of waiting
// in L2 as a dirty line; on whole 512-byte / 1 KiB spans that measured 0.3 to
// 1.8 points of the 8 TB/s peak above nt alone (the N = 8 step: 81.7% ->
// 83.5%).  Only for whole spans: stores that each cover half of every cache
// line lost 15 points with the same bits.
//
// kKeepStorePolicy (sc1 without nt) is for data read back soon from the
// memory-side cache: the staged step's chunk of reduced gradients.
constexpr int kRawBufferWord3 = 0x00020000;  // raw (stride 0) buffer, 32-bit format
constexpr int kSpanStorePolicy = 2 | 16;     // nt | sc1: streamed out, not read again
constexpr int kKeepStorePolicy = 16;         // sc1: read back by the next kernel
constexpr int kLoadStreamPolicy = 2;         // nt: the streaming loads' hint

template <typename T, int POLICY = kSpanStorePolicy>
__device__ __forceinline__ void st_span(T v, T *span, int lane)
{
    static_assert(sizeof(T) == 8 || sizeof(T) == 16, "8- or 16-byte lanes");
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(span, 0, 64 * (int)sizeof(T), kRawBufferWord3);
    if constexpr (sizeof(T) == 16)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, lane * 16, 0,
                                               POLICY);
    else
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rs, lane * 8, 0,
                                              POLICY);
}

// binary32 value of the low / high bf16 of a packed pair (exact widening).
__device__ __forceinline__ float bf_lo(unsigned x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(unsigned x) { return __uint_as_float(x & 0xffff0000u); }

// Loads of one lane's group of gradient elements: a quad (4 elements: 8
// bytes of bf16, 16 of fp32) or an oct (8 elements: 16 bytes of bf16, two
// 16-byte quads of fp32).  Lane l of a wave reads group i = i0 + l (i0 the
// same over the wave), and each wave instruction covers one contiguous span.
// A quad and a bf16 oct are the consecutive elements kN*i .. kN*i + kN-1.
// An fp32 oct is two quads 256 elements apart: elements 8*i0 + 4l .. +3 and
// 8*i0 + 256 + 4l .. +3, so that each of its two loads is a whole 1 KiB span
// (reading the oct's 32 consecutive bytes per lane instead, every load
// instruction touched half of each of 16 cache lines: the staged step on
// fp32 gradients ran 10-13 points slower at 48 and 128 ranks).
struct Bf16Quad {
    static constexpr int kN = 4, kBytes = 8;
    u32x2 r;
    __device__ __forceinline__ void load(const void *base, int64_t i)
    {
        r = ld_stream(reinterpret_cast<const u32x2 *>(base) + i);
    }
    __device__ __forceinline__ void load_span(__amdgpu_buffer_rsrc_t rs, int lane)
    {
        r = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, lane * kBytes, 0,
                                                                           kLoadStreamPolicy));
    }
    __device__ __forceinline__ void add_sel(float s[kN], bool on) const
    {
        const float e[kN] = {bf_lo(r.x), bf_hi(r.x), bf_lo(r.y), bf_hi(r.y)};
#pragma unroll
        for (int k = 0; k < kN; ++k)
            s[k] = on ? s[k] + e[k] : s[k];
    }
    template <bool FIRST>
    __device__ __forceinline__ void add_to(float s[kN]) const
    {
        const float e[kN] = {bf_lo(r.x), bf_hi(r.x), bf_lo(r.y), bf_hi(r.y)};
#pragma unroll
        for (int k = 0; k < kN; ++k)
            s[k] = FIRST ? e[k] : s[k] + e[k];
    }
};
struct F32Quad {
    static constexpr int kN = 4, kBytes = 16;
    f32x4 a;
    __device__ __forceinline__ void load(const void *base, int64_t i)
    {
        a = ld_stream(reinterpret_cast<const f32x4 *>(base) + i);
    }
    __device__ __forceinline__ void load_span(__amdgpu_buffer_rsrc_t rs, int lane)
    {
        a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * kBytes, 0,
                                                                            kLoadStreamPolicy));
    }
    __device__ __forceinline__ void add_sel(float s[kN], bool on) const
    {
        const float e[kN] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < kN; ++k)
            s[k] = on ? s[k] + e[k] : s[k];
    }
    template <bool FIRST>
    __device__ __forceinline__ void add_to(float s[kN]) const
    {
        const float e[kN] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < kN; ++k)
            s[k] = FIRST ? e[k] : s[k] + e[k];
    }
};
struct Bf16Oct {
    static constexpr int kN = 8, kBytes = 16;
    u32x4 r;
    // element offset of the lane's k-th value from the wave's first element
    static __device__ __forceinline__ int elem(int lane, int k) { return 8 * lane + k; }
    __device__ __forceinline__ void load(const void *base, int64_t i)
    {
        r = ld_stream(reinterpret_cast<const u32x4 *>(base) + i);
    }
    __device__ __forceinline__ void load_span(__amdgpu_buffer_rsrc_t rs, int lane)
    {
        r = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * kBytes, 0,
                                                                            kLoadStreamPolicy));
    }
    __device__ __forceinline__ void add_sel(float s[kN], bool on) const
    {
        const float e[kN] = {bf_lo(r.x), bf_hi(r.x), bf_lo(r.y), bf_hi(r.y),
                             bf_lo(r.z), bf_hi(r.z), bf_lo(r.w), bf_hi(r.w)};
#pragma unroll
        for (int k = 0; k < kN; ++k)
            s[k] = on ? s[k] + e[k] : s[k];
    }
    template <bool FIRST>
    __device__ __forceinline__ void add_to(float s[kN]) const
    {
        const float e[kN] = {bf_lo(r.x), bf_hi(r.x), bf_lo(r.y), bf_hi(r.y),
                             bf_lo(r.z), bf_hi(r.z), bf_lo(r.w), bf_hi(r.w)};
#pragma unroll
        for (int k = 0; k < kN; ++k)
            s[k] = FIRST ? e[k] : s[k] + e[k];
    }
};
struct F32Oct {
    static constexpr int kN = 8, kBytes = 32;
    f32x4 a, b;
    // element offset of the lane's k-th value from the wave's first element
    static __device__ __forceinline__ int elem(int lane, int k)
    {
        return k < 4 ? 4 * lane + k : 4 * kWave + 4 * lane + (k - 4);
    }
    __device__ __forceinline__ void load(const void *base, int64_t i)
    {
        const int64_t lane = threadIdx.x & (kWave - 1);
        const f32x4 *p = reinterpret_cast<const f32x4 *>(base) + (2 * i - lane);
        a = ld_stream(p);
        b = ld_stream(p + kWave);
    }
    __device__ __forceinline__ void load_span(__amdgpu_buffer_rsrc_t rs, int lane)
    {
        a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, 0,
                                                                            kLoadStreamPolicy));
        b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                          rs, kWave * 16 + lane * 16, 0, kLoadStreamPolicy));
    }
    __device__ __forceinline__ void add_sel(float s[kN], bool on) const
    {
        const float e[kN] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int k = 0; k < kN; ++k)
            s[k] = on ? s[k] + e[k] : s[k];
    }
    template <bool FIRST>
    __device__ __forceinline__ void add_to(float s[kN]) const
    {
        const float e[kN] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int k = 0; k < kN; ++k)
            s[k] = FIRST ? e[k] : s[k] + e[k];
    }
};

// s[k] = G_0[k] + G_1[k] + ... + G_{n-1}[k] over group i, left to right in
// rank order.  Loads are issued in batches ahead of the adds (at most 16
// ranks in flight per lane, to bound register use at large N); the adds keep
// rank order.
template <int NR, int CAP, typename QD>
__device__ __forceinline__ void rank_sum(const GradSet<CAP> &gs, int n, int64_t i, float s[QD::kN])
{
    if constexpr (NR > 0) {
        constexpr int B = NR < 16 ? NR : 16;
#pragma unroll
        for (int q0 = 0; q0 < NR; q0 += B) {
            const int nb = NR - q0 < B ? NR - q0 : B;  // known once unrolled
            QD c[B];
#pragma unroll
            for (int b = 0; b < B; ++b)
                if (b < nb)
                    c[b].load(gs.p[q0 + b], i);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (b >= nb)
                    break;
                if (q0 + b == 0)
                    c[b].template add_to<true>(s);
                else
                    c[b].template add_to<false>(s);
            }
        }
    } else {
        // Runtime rank count: ceil(n / B) batches of B ranks (128 bytes of
        // loads per lane), the last one partial, software-pipelined -- batch
        // k + 1's loads are issued before batch k is added -- so two batches
        // stay in flight.  Full batches use plain loads.  The partial batch
        // loads each slot through a buffer resource confined to the wave's
        // span of its rank's gradient; a slot past the rank count gets an
        // empty resource, so its load is dropped by the range check (no
        // memory access, zero returned) and its add is masked off.  It thus
        // goes out at once like a full batch, with no branch around any load.
        // (Loaded one at a time, the ranks past the last full batch each
        // cost a memory round trip: N = 17 to 31 ran at 27-49 % of the HBM
        // peak.  Building a resource for every rank of the full batches too
        // cost 1 to 4 points at 128 and 256 ranks.)  The adds keep rank
        // order, rank 0 starting the sum.  Every call site gives lane l of a
        // wave group i = i0 + l with i0 the same over the wave.
        constexpr int B = 128 / (int)sizeof(QD) < 4 ? 4 : 128 / (int)sizeof(QD);
        constexpr int W = QD::kBytes;
        const int lane = (int)(threadIdx.x & (kWave - 1));
        const uint64_t i0 = (uint64_t)(i - lane);
        const int64_t base = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(i0 >> 32)) << 32) |
                                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)i0)) * W;
        auto rsrc = [&](int q) {
            const bool on = q < n;
            const char *p = static_cast<const char *>(gs.p[on ? q : 0]) + base;
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), 0, on ? kWave * W : 0,
                                                     kRawBufferWord3);
        };
        const int nfull = n / B, nbat = (n + B - 1) / B;
        // batch k's loads into x: plain loads for a full batch, the
        // range-checked ones for the partial last batch (a uniform branch
        // per batch)
        auto load_batch = [&](QD (&x)[B], int k) {
            const int q0 = k * B;
            if (k < nfull) {
#pragma unroll
                for (int b = 0; b < B; ++b)
                    x[b].load(gs.p[q0 + b], i);
            } else {
#pragma unroll
                for (int b = 0; b < B; ++b)
                    x[b].load_span(rsrc(q0 + b), lane);
            }
        };
        QD cur[B], nxt[B];
        load_batch(cur, 0);
        for (int k = 0; k < nbat; ++k) {
            const int q0 = k * B;
            if (k + 1 < nbat)
                load_batch(nxt, k + 1);
            if (k == 0)
                cur[0].template add_to<true>(s);
            else
                cur[0].template add_to<false>(s);
            if (k < nfull) {
#pragma unroll
                for (int b = 1; b < B; ++b)
                    cur[b].template add_to<false>(s);
            } else {
#pragma unroll
                for (int b = 1; b < B; ++b)
                    cur[b].add_sel(s, q0 + b < n);
            }
            if (k + 1 < nbat) {
#pragma unroll
                for (int b = 0; b < B; ++b)
                    cur[b] = nxt[b];
            }
        }
    }
}

// One element's gradient, scalar path.
template <typename GT>
__device__ __forceinline__ float grad_at(const void *base, int64_t i);
template <>
__device__ __forceinline__ float grad_at<uint16_t>(const void *base, int64_t i)
{
    return __uint_as_float((unsigned)reinterpret_cast<const uint16_t *>(base)[i] << 16);
}
template <>
__device__ __forceinline__ float grad_at<float>(const void *base, int64_t i)
{
    return reinterpret_cast<const float *>(base)[i];
}

// The average s / divisor.  For a power-of-two divisor, s * (1/divisor) is
// the same correctly rounded value (both round the same real number), and
// costs one multiply instead of a division sequence.
template <bool POW2>
__device__ __forceinline__ float average(float s, const StepConsts &c)
{
    if constexpr (POW2)
        return s * c.inv_divisor;
    else
        return s / c.divisor;
}

// AdamW on one element ("ZeRO and FSDP sharding", Code), one rounding per
// operation in this order:
//   m = b1*m + (1-b1)*g
//   v = b2*v + ((1-b2)*g)*g
//   w = w*decay - (step_size*m) / (sqrt(v)/bc2 + eps)
__device__ __forceinline__ void adamw(float g, float &w, float &m, float &v, const StepConsts &c)
{
    const float m_dec = c.b1 * m;
    const float m_inc = c.omb1 * g;
    m = m_dec + m_inc;
    const float v_dec = c.b2 * v;
    const float v_inc = (c.omb2 * g) * g;
    v = v_dec + v_inc;
    const float den = sqrtf(v) / c.bc2 + c.eps;
    const float upd = (c.step_size * m) / den;
    const float w_dec = w * c.decay;
    w = w_dec - upd;
}

// Round-to-nearest-even bf16 of a pair, packed low-first (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi)
{
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16(float x)
{
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Sum of a double over one wave64 in a fixed order (butterfly); every lane
// ends with the same bits.
__device__ __forceinline__ double wave_sum(double x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x = x + __shfl_xor(x, off, 64);
    return x;
}

// Sum of a double over a kBlock-thread workgroup in a fixed order; valid in
// thread 0.  Wave butterflies, then the wave totals in wave order.
__device__ __forceinline__ double block_sum(double x)
{
    x = wave_sum(x);
    __shared__ double wave_tot[kBlock / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
        wave_tot[wave] = x;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0) {
        t = wave_tot[0];
#pragma unroll
        for (int w = 1; w < kBlock / 64; ++w)
            t = t + wave_tot[w];
    }
    return t;
}

}  // namespace dev
}  // namespace zero
