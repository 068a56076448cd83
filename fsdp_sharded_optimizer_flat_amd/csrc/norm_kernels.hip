// norm_kernels.hip -- two-stage sum of squares for global grad-norm clipping.
//
// "ZeRO and FSDP sharding", Implementation notes: clipping needs the global
// norm, i.e. the summed squared norms of the shards (then all-reduced across
// ranks).  "ZeRO: Three Ledgers", section 2: a norm is a decomposable
// reduction costing O(1) scalars per rank.
//
// Stage 1 fuses the reduction half of the reduce-scatter with the sum of
// squares: each lane forms g = (rank-ordered sum) / divisor for its eight
// consecutive elements, optionally writes g (fp32) so the step can read one
// reduced gradient instead of N, and accumulates g^2 in binary64.  Each wave
// reduces its lanes in a fixed order to one partial per 512-element tile.
// Stage 2 sums the partials in a fixed-order tree of 1024-way workgroups.
// The partition (segments, grid size, element groups) depends only on the
// layout, the rank and the index spaces -- never on the device, the
// pointers' alignment or whether g is written -- so the result is bitwise
// reproducible.
#include <algorithm>
#include <mutex>
#include <vector>

#include <utility>

#include "device_common.h"

// Partials of zero_gradnorm_async_noalloc: device memory that belongs to the
// library's code object, one copy per GPU, so that call allocates nothing.
// Host code never passes this name to a kernel (on the host it is only a
// stand-in for the symbol); it uses the per-device address that
// noalloc_scratch() looks up.
static __device__ __align__(256) double scratch[ZERO_NOALLOC_SCRATCH_BYTES / sizeof(double)];

namespace zero {
namespace {

using namespace dev;

// Stage 1 over one segment of `len` elements, cut into tiles of kNormSpan =
// 512 elements that start `phase` elements before the segment (0 to 56, a
// whole number of octs: the segment's first gradient element modulo a
// 128-byte line, so that the tiles' gradient spans start on lines when the
// gradient bases do).  Workgroup b (one wave64) owns tile b and lane l an
// oct of it: elements 8l .. 8l+7 for bf16 gradients, 4l .. 4l+3 and
// 256+4l .. +3 for fp32 (the loaders' layouts, OD::elem).  The lane adds its
// oct's squares in that order, the wave sums its lanes by a fixed butterfly,
// and lane 0 writes the tile's partial.  Elements before the segment or
// past `len` contribute +0.0, which leaves a binary64 sum unchanged.
//
// VEC: every gradient is 16-byte aligned at the segment start (and g_out
// too), so whole tiles load each rank's oct as whole 1 KiB spans per wave
// instruction (one for bf16, the access width that streams N = 64 ranks best
// on MI355X, two for fp32), and the wave stores g as two contiguous 1 KiB
// spans, quads l and 64 + l of the tile (bf16's octs go through LDS to get
// there; fp32's already are).  In the first tile the lanes before the
// segment load in-bounds data (the phase never exceeds the segment's offset
// in its buffers) and discard it, and their quads of g are not stored.  The
// last, partial tile of a segment, and every tile without VEC, reads the same
// elements one by one.  Either way every value and every addition happen in
// the same order, so the result depends on neither pointer alignment nor on
// whether g_out is written.  One tile per workgroup (a non-persistent grid)
// keeps the tiles in flight in one compact window, as in the step kernel.
// Tile `tile` of a segment whose gradient elements start g8 octs (8 * g8
// elements) past every rank's gradient base; G (may be null) is the
// segment's g_out.

// A vector tile's g to G + t0 (quads l and 64 + l from lane l); in a phased
// first tile (PHASED, t0 < 0) the first store only where quad l lies in the
// segment.
template <typename OD, bool PHASED>
__device__ __forceinline__ void store_tile_g(const float g[kOct], float *Gt, int64_t t0,
                                             int lane, f32x4 *xg)
{
    f32x4 q0 = f32x4{g[0], g[1], g[2], g[3]}, q1 = f32x4{g[4], g[5], g[6], g[7]};
    if constexpr (OD::kBytes != 32) {  // bf16: lane l holds quads 2l and 2l + 1
        xg[2 * lane] = q0;
        xg[2 * lane + 1] = q1;
        __syncthreads();
        q0 = xg[lane];
        q1 = xg[kWave + lane];
    }
    f32x4 *t4 = reinterpret_cast<f32x4 *>(Gt);
    if (!PHASED || t0 + 4 * (int64_t)lane >= 0)
        st_span(q0, t4, lane);
    st_span(q1, t4 + kWave, lane);  // quads 64.. lie in the segment (phase < 256)
}

template <int NR, int CAP, typename GT, typename OD, bool POW2, bool VEC>
__device__ __forceinline__ void norm_tile(const GradSet<CAP> &gs, int n, float *__restrict__ G,
                                          int64_t len, int64_t g8, int phase, int64_t tile,
                                          int lane, const StepConsts &c,
                                          double *__restrict__ partial, f32x4 *xg)
{
    static_assert(OD::kN == kOct, "one oct per lane");
    const int64_t t0 = tile * kNormSpan - phase;  // the tile's first element
    float g[kOct];
    if (VEC && t0 >= 0 && t0 + kNormSpan <= len) {  // a whole tile (uniform over the workgroup)
        float s[kOct];
        rank_sum<NR, CAP, OD>(gs, n, g8 + t0 / kOct + lane, s);
#pragma unroll
        for (int k = 0; k < kOct; ++k)
            g[k] = average<POW2>(s[k], c);
        if (G)
            store_tile_g<OD, false>(g, G + t0, t0, lane, xg);
    } else if (VEC && t0 < 0 && t0 + kNormSpan <= len) {  // a phased first tile
        float s[kOct];
        rank_sum<NR, CAP, OD>(gs, n, g8 + t0 / kOct + lane, s);
#pragma unroll
        for (int k = 0; k < kOct; ++k)
            g[k] = t0 + OD::elem(lane, k) >= 0 ? average<POW2>(s[k], c) : 0.0f;
        if (G)
            store_tile_g<OD, true>(g, G + t0, t0, lane, xg);
    } else {
        const int64_t gb = g8 * kOct;
#pragma unroll
        for (int k = 0; k < kOct; ++k) {
            const int64_t e = t0 + OD::elem(lane, k);
            g[k] = 0.0f;
            if (e >= 0 && e < len) {
                float s = grad_at<GT>(gs.p[0], gb + e);
                for (int q = 1; q < n; ++q)
                    s = s + grad_at<GT>(gs.p[q], gb + e);
                g[k] = average<POW2>(s, c);
                if (G)
                    G[e] = g[k];
            }
        }
    }
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kOct; ++k) {
        const double x = (double)g[k];
        acc = acc + x * x;
    }
    const double t = wave_sum(acc);
    if (lane == 0)
        *partial = t;
}

template <int NR, int CAP, typename GT, typename OD, bool POW2, bool VEC>
__global__ __launch_bounds__(kWave) void norm_kernel(GradSet<CAP> gs, int n,
                                                    float *__restrict__ G, int64_t len,
                                                    int phase, StepConsts c,
                                                    double *__restrict__ partials)
{
    __shared__ f32x4 xg[2 * kWave];  // the tile's g in element order
    const int64_t tile = blockIdx.x;
    norm_tile<NR, CAP, GT, OD, POW2, VEC>(gs, n, G, len, 0, phase, tile, threadIdx.x, c,
                                          partials + tile, xg);
}

// Several aligned segments in one launch -- one rank's slice of every unit --
// instead of a launch per segment (each launch's drain and refill is worth
// tens of MB of streaming: one rank's GPT-2 Large norm pass, 36 segments,
// ran at 36-40 % of the HBM peak).  Each segment keeps its own tiles and
// partial slots, so the partition -- and the sum's bits -- are those of the
// launch per segment.  A workgroup finds its segment as the step's shared
// launches do: a byte per group of 512 tiles naming the segment that holds
// the group's first tile (bit 7: the whole group lies in it), a walk over
// segment ends only in a group that holds a boundary.
constexpr int kNormPieces = 48;
constexpr int kNormGroups = 512;
constexpr int kNormGroupShift = 9;
constexpr int64_t kNormBatchTiles = int64_t(kNormGroups) << kNormGroupShift;

struct NormPiece {
    int64_t g8;     // octs from every gradient base to the segment's first element
    int64_t s;      // g_out elements to the segment's first g
    int64_t len;    // elements
    int64_t pbase;  // the segment's first partial
    uint32_t first; // the launch's first tile of this segment
    int32_t phase;  // elements the segment's first tile starts before it
};

struct NormBatch {
    NormPiece p[kNormPieces];
    uint32_t end[kNormPieces];        // segment i covers tiles [p[i].first, end[i])
    uint32_t group[kNormGroups / 4];  // byte per group, as described above
    int32_t n_pieces, pad;
};
static_assert(sizeof(NormBatch) + sizeof(GradSet<64>) + sizeof(StepConsts) + 64 <= 4096,
              "kernel arguments are limited to 4 KB");

template <int NR, int CAP, typename GT, typename OD, bool POW2>
__global__ __launch_bounds__(kWave) void norm_batch_kernel(GradSet<CAP> gs, int n,
                                                          float *__restrict__ G, const NormBatch b,
                                                          StepConsts c,
                                                          double *__restrict__ partials)
{
    __shared__ f32x4 xg[2 * kWave];
    const uint32_t blk = blockIdx.x;
    const uint32_t g = blk >> kNormGroupShift;
    const uint32_t entry = (b.group[g >> 2] >> ((g & 3u) * 8u)) & 0xffu;
    int i = (int)(entry & 0x7fu);
    if (!(entry & 0x80u))
        while (blk >= b.end[i])  // the last segment ends at the grid size: the walk stops there
            ++i;
    const NormPiece pc = b.p[i];
    const int64_t tile = blk - pc.first;
    norm_tile<NR, CAP, GT, OD, POW2, true>(gs, n, G ? G + pc.s : nullptr, pc.len, pc.g8, pc.phase,
                                           tile, threadIdx.x, c, partials + pc.pbase + tile, xg);
}

// One level of the fixed-order reduction of the partials: workgroup b sums
// in[b * kNormFanIn .. min(n, (b + 1) * kNormFanIn)) -- thread t takes the
// four consecutive values at b * kNormFanIn + 4t, in order, then the
// workgroup sums its threads in a fixed order -- and writes out[b].
__global__ __launch_bounds__(kBlock) void norm_level_kernel(const double *__restrict__ in,
                                                           int64_t n, double *__restrict__ out)
{
    const int64_t base = (int64_t)blockIdx.x * kNormFanIn + 4 * (int64_t)threadIdx.x;
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (base + k < n)
            acc = acc + in[base + k];
    const double t = block_sum(acc);
    if (threadIdx.x == 0)
        out[blockIdx.x] = t;
}

// The clip coefficient on the device, with the host formula: the n sums of
// squares added in order (binary64; n is 1 for one shard's sum, N for the
// ranks' sums of a sharded norm), norm = sqrt(sum), c = max_norm / (norm +
// 1e-6) with correctly rounded sqrt and division, capped at 1, rounded once
// to binary32 -- the same bits as zero_clip_coef computes on the host.  A
// total that is negative, NaN or infinite (a non-finite gradient; the host
// function refuses it) gives a NaN coefficient, which makes the device-clip
// step leave the state unchanged.  One thread.
__global__ void clip_coef_kernel(const double *__restrict__ sums, int n, double max_norm,
                                 float *__restrict__ coef, double *__restrict__ total)
{
    if (threadIdx.x != 0 || blockIdx.x != 0)
        return;
    double t = sums[0];
    for (int r = 1; r < n; ++r)
        t = t + sums[r];
    double c = __builtin_nan("");
    if (t >= 0.0 && t <= 1.7976931348623157e308) {
        const double norm = sqrt(t);
        c = max_norm / (norm + 1e-6);
        if (c > 1.0)
            c = 1.0;
    }
    *coef = (float)c;
    if (total)
        *total = t;
}

template <int NR, typename GT, typename OD, bool POW2, bool VEC>
hipError_t launch_nr(const void *const *grads, int n, float *G, int64_t len, int phase,
                     const StepConsts &c, double *partials, int64_t blocks, hipStream_t st)
{
    constexpr int CAP = NR > 0 ? NR : ZERO_MAX_RANKS;
    GradSet<CAP> gs{};
    for (int q = 0; q < n; ++q)
        gs.p[q] = grads[q];
    const size_t lds = occupancy_cap_lds(norm_waves_per_cu(n, NR == 0, (int)sizeof(GT)),
                                         2 * kWave * sizeof(f32x4));
    hipLaunchKernelGGL((norm_kernel<NR, CAP, GT, OD, POW2, VEC>), dim3((unsigned)blocks),
                       dim3(kWave), lds, st, gs, n, G, len, phase, c, partials);
    return hipGetLastError();
}

template <bool POW2, int... Ks>
hipError_t bf16_vec_compiled(std::integer_sequence<int, Ks...>, const void *const *grads, int n,
                             float *G, int64_t len, int phase, const StepConsts &c,
                             double *partials, int64_t blocks, hipStream_t st)
{
    using T = uint16_t;
    using QD = Bf16Oct;
    hipError_t r = hipSuccess;
    const bool hit =
        ((n == Ks + 1
              ? (r = launch_nr<Ks + 1, T, QD, POW2, true>(grads, n, G, len, phase, c, partials,
                                                          blocks, st),
                 true)
              : false) ||
         ...);
    if (hit)
        return r;
    if (n == 64)
        return launch_nr<64, T, QD, POW2, true>(grads, n, G, len, phase, c, partials, blocks, st);
    return launch_nr<0, T, QD, POW2, true>(grads, n, G, len, phase, c, partials, blocks, st);
}

// bf16 gradients, aligned: a kernel compiled for each rank count up to
// kMaxCompiledRanks and for 64, the run-time kernel for any other N.
template <bool POW2>
hipError_t launch_bf16_vec(const void *const *grads, int n, float *G, int64_t len, int phase,
                           const StepConsts &c, double *partials, int64_t blocks, hipStream_t st)
{
    return bf16_vec_compiled<POW2>(std::make_integer_sequence<int, kMaxCompiledRanks>{}, grads, n,
                                   G, len, phase, c, partials, blocks, st);
}

// ---- several segments per launch ---------------------------------------

void fill_norm_groups(NormBatch &b, uint32_t total)
{
    int first_piece = 0, last_piece = 0;
    for (uint32_t g = 0; g < (uint32_t)kNormGroups; ++g) {
        const uint32_t a = g << kNormGroupShift;
        if (a >= total)
            break;
        const uint32_t z =
            std::min<uint64_t>((uint64_t)a + (1u << kNormGroupShift) - 1u, total - 1u);
        while (b.end[first_piece] <= a)
            ++first_piece;
        if (last_piece < first_piece)
            last_piece = first_piece;
        while (b.end[last_piece] <= z)
            ++last_piece;
        const uint32_t entry = (uint32_t)first_piece | (first_piece == last_piece ? 0x80u : 0u);
        b.group[g >> 2] |= entry << ((g & 3u) * 8u);
    }
}

// Batches of the segments, in order: at most kNormPieces segments and
// kNormBatchTiles tiles each, a longer segment cut at a whole tile (its
// later tiles keep their elements and partial slots; the part after a cut
// starts on a tile boundary, with no phase).
std::vector<std::pair<NormBatch, uint32_t>> norm_batches(const NormSegment *segs, int count)
{
    std::vector<std::pair<NormBatch, uint32_t>> out;
    NormBatch b{};
    uint32_t tiles = 0;
    auto flush = [&]() {
        if (b.n_pieces == 0)
            return;
        fill_norm_groups(b, tiles);
        out.emplace_back(b, tiles);
        b = NormBatch{};
        tiles = 0;
    };
    for (int k = 0; k < count; ++k) {
        int64_t g8 = segs[k].g_off / kOct, sg = segs[k].g_out_off, len = segs[k].len,
                pbase = segs[k].partial;
        int phase = segs[k].phase;
        while (len > 0) {
            const int64_t nt =
                std::min((len + phase + kNormSpan - 1) / kNormSpan, kNormBatchTiles);
            const int64_t part = std::min(len, nt * kNormSpan - phase);  // elements covered
            if (b.n_pieces == kNormPieces || (int64_t)tiles + nt > kNormBatchTiles)
                flush();
            NormPiece &q = b.p[b.n_pieces];
            q.g8 = g8;
            q.s = sg;
            q.len = part;
            q.pbase = pbase;
            q.first = tiles;
            q.phase = phase;
            tiles += (uint32_t)nt;
            b.end[b.n_pieces] = tiles;
            ++b.n_pieces;
            g8 += part / kOct;  // a cut part is whole tiles less the phase: whole octs
            sg += part;
            pbase += nt;
            len -= part;
            phase = 0;
        }
    }
    flush();
    return out;
}

template <int NR, bool POW2>
hipError_t launch_norm_batch_nr(const NormSegment *segs, int count, const void *const *grads, int n,
                                float *G, const StepConsts &c, double *partials, hipStream_t st)
{
    GradSet<NR> gs{};
    for (int q = 0; q < n; ++q)
        gs.p[q] = grads[q];
    const size_t lds = occupancy_cap_lds(norm_waves_per_cu(n, false, 2), 2 * kWave * sizeof(f32x4));
    for (const auto &bb : norm_batches(segs, count)) {
        hipLaunchKernelGGL((norm_batch_kernel<NR, NR, uint16_t, Bf16Oct, POW2>), dim3(bb.second),
                           dim3(kWave), lds, st, gs, n, G, bb.first, c, partials);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <bool POW2, int... Ks>
hipError_t norm_batch_compiled(std::integer_sequence<int, Ks...>, const NormSegment *segs,
                               int count, const void *const *grads, int n, float *G,
                               const StepConsts &c, double *partials, hipStream_t st)
{
    hipError_t r = hipErrorNotSupported;
    const bool hit =
        ((n == Ks + 1
              ? (r = launch_norm_batch_nr<Ks + 1, POW2>(segs, count, grads, n, G, c, partials, st),
                 true)
              : false) ||
         ...);
    if (!hit && n == 64)
        r = launch_norm_batch_nr<64, POW2>(segs, count, grads, n, G, c, partials, st);
    return r;
}

}  // namespace

int64_t norm_segment_blocks(int64_t len, int phase)
{
    return len > 0 ? (len + phase + kNormSpan - 1) / kNormSpan : 0;
}

int norm_segment_phase(int64_t g_off, int grad_bytes)
{
    // the segment's first gradient element modulo a 128-byte line, in whole
    // octs (never more than g_off, so the first tile stays in the buffers)
    const int64_t line = 128 / grad_bytes;
    return (int)(g_off % line) / kOct * kOct;
}

int launch_norm_segment(int64_t len, int phase, bool vec, const void *const *grads, int n_grads,
                        int grad_dtype, float *g_out, const StepConsts &c, double *partials,
                        void *stream)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t blocks = norm_segment_blocks(len, phase);
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0xffffffffLL / kWave)
        return hipErrorInvalidValue;  // larger than one dispatch can address
    const bool bf = grad_dtype == ZERO_BF16;
    const bool p2 = c.div_pow2 != 0;
    const int ph = phase;
    if (bf && vec)
        return p2 ? launch_bf16_vec<true>(grads, n_grads, g_out, len, ph, c, partials, blocks, st)
                  : launch_bf16_vec<false>(grads, n_grads, g_out, len, ph, c, partials, blocks, st);
    if (bf)
        return p2 ? launch_nr<0, uint16_t, Bf16Oct, true, false>(grads, n_grads, g_out, len, ph, c,
                                                                  partials, blocks, st)
                  : launch_nr<0, uint16_t, Bf16Oct, false, false>(grads, n_grads, g_out, len, ph, c,
                                                                   partials, blocks, st);
    if (vec)
        return p2 ? launch_nr<0, float, F32Oct, true, true>(grads, n_grads, g_out, len, ph, c,
                                                             partials, blocks, st)
                  : launch_nr<0, float, F32Oct, false, true>(grads, n_grads, g_out, len, ph, c,
                                                              partials, blocks, st);
    return p2 ? launch_nr<0, float, F32Oct, true, false>(grads, n_grads, g_out, len, ph, c, partials,
                                                          blocks, st)
              : launch_nr<0, float, F32Oct, false, false>(grads, n_grads, g_out, len, ph, c, partials,
                                                           blocks, st);
}

int launch_norm_batch(const NormSegment *segs, int count, const void *const *grads, int n_grads,
                      int grad_dtype, float *g_out, const StepConsts &c, double *partials,
                      void *stream)
{
    if (grad_dtype != ZERO_BF16)
        return hipErrorNotSupported;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const auto seq = std::make_integer_sequence<int, kMaxCompiledRanks>{};
    return c.div_pow2 ? norm_batch_compiled<true>(seq, segs, count, grads, n_grads, g_out, c,
                                                  partials, st)
                      : norm_batch_compiled<false>(seq, segs, count, grads, n_grads, g_out, c,
                                                   partials, st);
}

int noalloc_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0)
        return hipErrorInvalidDevice;
    static std::mutex mu;
    static std::vector<void *> addr;  // per device, looked up once
    std::lock_guard<std::mutex> lock(mu);
    if ((size_t)dev >= addr.size())
        addr.resize((size_t)dev + 1, nullptr);
    if (!addr[(size_t)dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        addr[(size_t)dev] = p;
    }
    *ptr = addr[(size_t)dev];
    return hipSuccess;
}

int launch_clip_coef(const double *sums, int n, double max_norm, float *coef, double *total,
                     void *stream)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(clip_coef_kernel, dim3(1), dim3(kWave), 0, st, sums, n, max_norm, coef,
                       total);
    return hipGetLastError();
}

int launch_norm_tree(const double *partials, int64_t n_partials, double *scratch, double *result,
                     void *stream)
{
    // Levels of kNormFanIn-way sums until one value remains; the last level
    // writes *result.  A single partial still passes through one level, so the
    // result is always produced the same way.
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const double *in = partials;
    int64_t n = n_partials;
    double *out = scratch;
    do {
        const int64_t blocks = (n + kNormFanIn - 1) / kNormFanIn;
        double *dst = blocks == 1 ? result : out;
        hipLaunchKernelGGL(norm_level_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, in, n,
                           dst);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        in = dst;
        n = blocks;
        out += blocks;
    } while (n > 1);
    return hipSuccess;
}

}  // namespace zero
