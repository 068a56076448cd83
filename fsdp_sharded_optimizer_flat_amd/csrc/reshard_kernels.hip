// reshard_kernels.hip -- the device side of a checkpoint reshard: copy the
// runs of a reshard plan from the old shards into the new one and zero-fill
// its padding ("ZeRO and FSDP sharding", Implementation notes: a sharded
// checkpoint is resharded to a new N when it is loaded).
//
// Pure data movement, bound by HBM bandwidth.  A plan has one run per (unit,
// source rank) pair: hundreds of runs of a few KB to a few hundred MB.  Up to
// kCopyPieces runs travel by value in one launch's kernel arguments, so a
// whole plan takes a handful of launches.
//
// Finding its run is the only work a workgroup does before its load, and it
// lengthens the life of every 1 KB workgroup: a binary search over the runs'
// block prefix sums (seven dependent scalar loads) cost 3 to 6 points of the
// 8 TB/s peak against a plain copy.  So the launch also carries a group table:
// the grid's blocks in 512 equal groups, and for each the run that holds the
// group's first block, with a flag when the whole group lies in that run.  A
// workgroup reads its group's entry (one scalar load, its address known from
// blockIdx alone), steps forward over run ends only when its group is
// flagged as holding a run boundary, then loads its run.
//
// Each workgroup is one wave64 and each lane moves one 16-byte block: 1 KB
// per workgroup.  Measured on MI355X, spans that small stream best (a plain
// 1 GiB copy reaches 84% of 8 TB/s this way against 76-78% with 4 KB per
// wave in four passes).
//
// Within a run every store is a 16-byte vector store aligned in the
// destination, issued as one wave's whole-span store (st_span).  Shard boundaries fall anywhere, so the source is usually at
// another 16-byte phase; then each lane reads the two aligned 16-byte blocks
// its bytes straddle and funnel-shifts them together (both blocks hold bytes
// of the run, so no read leaves the source buffer's 16-byte-aligned extent).
// The few elements before the destination's first aligned block and after
// its last are copied one by one by the run's first workgroup.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"

namespace zero {
namespace {

using dev::st_span;
using dev::u32x4;

constexpr int kCopyPieces = 96;     // runs per launch
constexpr int kCopyThreads = kWave; // one wave64 per workgroup
constexpr int64_t kCopyPerBlock = kCopyThreads;  // 16-byte blocks per workgroup (1 KB)
constexpr int kGroups = 512;        // group-table entries per launch
constexpr int kMinGroupShift = 9;   // blocks per group: 2^9 .. 2^17
constexpr int kMaxGroupShift = 17;
constexpr int64_t kMaxBlocksPerLaunch = int64_t(kGroups) << kMaxGroupShift;  // 2^26
constexpr int64_t kMaxPieceBytes = int64_t(1) << 31;  // element count fits 32 bits

struct CopyPiece {
    const unsigned char *src;  // null: zero-fill
    unsigned char *dst;
    uint32_t n;                // elements
    uint32_t first;            // the launch's first block of this piece
};

// Kernel arguments of one launch: 3,208 bytes.
struct CopyBatch {
    CopyPiece p[kCopyPieces];
    uint32_t end[kCopyPieces];   // piece i covers blocks [p[i].first, end[i])
    uint32_t group[kGroups / 4]; // byte g: the piece holding group g's first
                                 // block; bit 7 set when the group lies in it whole
    int32_t n_pieces;
    int32_t elem;                // bytes per element: 2 or 4
};
static_assert(sizeof(CopyBatch) <= 4096, "kernel arguments are limited to 4 KB");

// Split of a run: `head` elements before dst's first 16-byte boundary, then
// `blocks` whole 16-byte blocks, then `tail` elements.
struct Split {
    int64_t head, blocks, tail;
};

__host__ __device__ inline Split split_of(const unsigned char *dst, int64_t n, int elem)
{
    Split s;
    s.head = (int64_t)((16u - (unsigned)((uintptr_t)dst % 16u)) % 16u) / elem;
    if (s.head > n)
        s.head = n;
    s.blocks = (n - s.head) * elem / 16;
    s.tail = n - s.head - s.blocks * (16 / elem);
    return s;
}

__device__ __forceinline__ void copy_elem(const unsigned char *s, unsigned char *d, int64_t i,
                                          int elem)
{
    if (elem == 4)
        reinterpret_cast<uint32_t *>(d)[i] = s ? reinterpret_cast<const uint32_t *>(s)[i] : 0u;
    else
        reinterpret_cast<uint16_t *>(d)[i] = s ? reinterpret_cast<const uint16_t *>(s)[i] : 0u;
}

// Bytes [delta, delta + 16) of the 32-byte concatenation lo:hi (delta even,
// 0 < delta < 16).
__device__ __forceinline__ u32x4 funnel(u32x4 lo, u32x4 hi, unsigned delta)
{
    unsigned a0, a1, a2, a3, a4;
    switch (delta >> 2) {  // uniform across the workgroup
    case 0: a0 = lo.x; a1 = lo.y; a2 = lo.z; a3 = lo.w; a4 = hi.x; break;
    case 1: a0 = lo.y; a1 = lo.z; a2 = lo.w; a3 = hi.x; a4 = hi.y; break;
    case 2: a0 = lo.z; a1 = lo.w; a2 = hi.x; a3 = hi.y; a4 = hi.z; break;
    default: a0 = lo.w; a1 = hi.x; a2 = hi.y; a3 = hi.z; a4 = hi.w; break;
    }
    const unsigned b = delta & 3u;  // 0 or 2
    u32x4 r;
    r.x = __builtin_amdgcn_alignbyte(a1, a0, b);
    r.y = __builtin_amdgcn_alignbyte(a2, a1, b);
    r.z = __builtin_amdgcn_alignbyte(a3, a2, b);
    r.w = __builtin_amdgcn_alignbyte(a4, a3, b);
    return r;
}

// SHIFT: log2 of the blocks per group, fixed per launch so that the group
// index needs no argument.
template <int SHIFT>
__global__ __launch_bounds__(kCopyThreads) void copy_batch_kernel(const CopyBatch b)
{
    const uint32_t blk = blockIdx.x;
    const uint32_t g = blk >> SHIFT;
    const uint32_t entry = (b.group[g >> 2] >> ((g & 3u) * 8u)) & 0xffu;
    int i = (int)(entry & 0x7fu);
    if (!(entry & 0x80u))
        while (blk >= b.end[i])  // the last piece ends at the grid size: the walk stops there
            ++i;
    const uint32_t first = b.p[i].first;
    const unsigned char *s = b.p[i].src;
    unsigned char *d = b.p[i].dst;
    const int e = b.elem;
    const Split sp = split_of(d, b.p[i].n, e);
    const int64_t lb = blk - first;
    const int t = threadIdx.x;
    if (lb == 0) {  // head and tail elements (at most 7 each)
        if (t < sp.head)
            copy_elem(s, d, t, e);
        else if (t >= 32 && t < 32 + sp.tail)
            copy_elem(s, d, sp.head + sp.blocks * (16 / e) + (t - 32), e);
    }
    u32x4 *db = reinterpret_cast<u32x4 *>(d + sp.head * e);
    u32x4 *span = db + lb * kCopyPerBlock;  // this workgroup's 1 KB of the destination
    const int64_t j = lb * kCopyPerBlock + t;
    if (j >= sp.blocks)
        return;
    if (!s) {
        st_span(u32x4{0u, 0u, 0u, 0u}, span, t);
        return;
    }
    const unsigned char *sb = s + sp.head * e;
    const unsigned delta = (unsigned)((uintptr_t)sb % 16u);
    const u32x4 *sa = reinterpret_cast<const u32x4 *>(sb - delta);  // aligned
    if (delta == 0) {
        st_span(__builtin_nontemporal_load(sa + j), span, t);
    } else {
        // block j + 1 holds bytes of block j's span (delta > 0); the
        // neighbouring lane has just fetched it, so the second load is
        // served from cache
        const u32x4 lo = __builtin_nontemporal_load(sa + j), hi = sa[j + 1];
        st_span(funnel(lo, hi, delta), span, t);
    }
}

// The group table of a launch of `total` blocks in pieces ending at end[0..n).
void fill_groups(CopyBatch &b, uint32_t total, int shift)
{
    int first_piece = 0, last_piece = 0;
    for (uint32_t g = 0; g < (uint32_t)kGroups; ++g) {
        const uint32_t a = g << shift;
        if (a >= total)
            break;
        const uint32_t z = std::min<uint64_t>((uint64_t)a + (1u << shift) - 1u, total - 1u);
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

template <int SHIFT>
void launch_copy(const CopyBatch &b, uint32_t blocks, hipStream_t stream)
{
    hipLaunchKernelGGL(copy_batch_kernel<SHIFT>, dim3(blocks), dim3(kCopyThreads), 0, stream, b);
}

struct Batcher {
    CopyBatch b{};
    int64_t blocks = 0;
    hipStream_t stream;
    int err = hipSuccess;

    void flush()
    {
        if (b.n_pieces == 0 || err != hipSuccess)
            return;
        const uint32_t total = (uint32_t)blocks;
        int shift = kMinGroupShift;
        while (((total - 1u) >> shift) >= (uint32_t)kGroups)
            ++shift;
        fill_groups(b, total, shift);
        switch (shift) {
        case 9: launch_copy<9>(b, total, stream); break;
        case 10: launch_copy<10>(b, total, stream); break;
        case 11: launch_copy<11>(b, total, stream); break;
        case 12: launch_copy<12>(b, total, stream); break;
        case 13: launch_copy<13>(b, total, stream); break;
        case 14: launch_copy<14>(b, total, stream); break;
        case 15: launch_copy<15>(b, total, stream); break;
        case 16: launch_copy<16>(b, total, stream); break;
        default: launch_copy<kMaxGroupShift>(b, total, stream); break;
        }
        err = hipGetLastError();
        const int32_t elem = b.elem;
        b = CopyBatch{};
        b.elem = elem;
        blocks = 0;
    }

    void add(const unsigned char *src, unsigned char *dst, int64_t n)
    {
        const int e = b.elem;
        while (n > 0 && err == hipSuccess) {
            const int64_t take = std::min(n, kMaxPieceBytes / e);
            const Split sp = split_of(dst, take, e);
            const int64_t nb = std::max<int64_t>(1, (sp.blocks + kCopyPerBlock - 1) / kCopyPerBlock);
            if (b.n_pieces == kCopyPieces || blocks + nb > kMaxBlocksPerLaunch)
                flush();
            CopyPiece &pc = b.p[b.n_pieces];
            pc.src = src;
            pc.dst = dst;
            pc.n = (uint32_t)take;
            pc.first = (uint32_t)blocks;
            blocks += nb;
            b.end[b.n_pieces] = (uint32_t)blocks;
            ++b.n_pieces;
            if (src)
                src += take * e;
            dst += take * e;
            n -= take;
        }
    }
};

}  // namespace

int launch_reshard(const std::vector<ReshardRun> &runs, const void *const *src, void *dst,
                   int elem, void *stream)
{
    Batcher bt;
    bt.b.elem = elem;
    bt.stream = reinterpret_cast<hipStream_t>(stream);
    for (const ReshardRun &r : runs) {
        const unsigned char *s =
            r.src_rank < 0 ? nullptr
                           : static_cast<const unsigned char *>(src[r.src_rank]) + r.src_k * elem;
        bt.add(s, static_cast<unsigned char *>(dst) + r.dst_k * elem, r.len);
    }
    bt.flush();
    return bt.err;
}

}  // namespace zero
