// layout.cpp -- the flat-buffer packer's host side: unit padding, shard
// ownership, the local <-> global index maps, the element runs ("pieces")
// that the kernels stream over, and the copy plan of a reshard.
//
// "ZeRO and FSDP sharding", How it works: each unit's parameters are flattened
// into one buffer padded to a multiple of N, and rank r owns slice r.  Same
// page, Pitfalls: without the padding the last rank's slice is corrupted.
// "Learn: ZeRO & FSDP", section 5 (FSDP1 vs FSDP2): FSDP2 shards each
// parameter on its own along dim 0; a unit with granule g (its row length)
// pads to a multiple of N g, so each rank's slice is whole rows.
#include <algorithm>
#include <climits>
#include <cstring>

#include "zero_internal.h"

namespace zero {

bool layout_ok(const zero_layout *L)
{
    if (!L || L->magic != ZERO_LAYOUT_MAGIC || L->n_ranks < 1 || L->n_units < 0 ||
        L->n_units > ZERO_MAX_UNITS)
        return false;
    int64_t off = 0, loff = 0, numel = 0;
    for (int32_t u = 0; u < L->n_units; ++u) {
        const zero_unit &x = L->unit[u];
        // padded is the least multiple of N g at or above numel:
        // padded - numel < N g, i.e. (padded - numel) / N < g in integers
        if (x.numel < 0 || x.shard < 0 || x.granule < 1 || x.numel % x.granule != 0 ||
            x.shard % x.granule != 0 || x.padded != x.shard * L->n_ranks || x.padded < x.numel ||
            (x.padded - x.numel) / L->n_ranks >= x.granule || x.offset != off ||
            x.local_offset != loff)
            return false;
        off += x.padded;
        loff += x.shard;
        numel += x.numel;
    }
    return off == L->padded && loff == L->shard && numel == L->numel;
}

int64_t unit_start(const zero_layout *L, int32_t u, int32_t index)
{
    if (u >= L->n_units)
        return index == ZERO_GLOBAL ? L->padded : L->shard;
    return index == ZERO_GLOBAL ? L->unit[u].offset : L->unit[u].local_offset;
}

std::vector<Segment> build_segments(const zero_layout *L, int32_t rank, int32_t grad_index,
                                    int32_t state_index, int32_t out_index, int32_t u0,
                                    int32_t u1, bool grads_from_range)
{
    std::vector<Segment> segs;
    if (u1 < 0 || u1 > L->n_units)
        u1 = L->n_units;
    if (u0 < 0)
        u0 = 0;
    if (u0 >= u1)
        return segs;
    const int64_t gbase = grads_from_range ? unit_start(L, u0, grad_index) : 0;
    if (rank < 0) {  // every rank's slices of the units: one identity-mapped run
        const int64_t a = unit_start(L, u0, ZERO_GLOBAL), b = unit_start(L, u1, ZERO_GLOBAL);
        if (b > a)
            segs.push_back({a - gbase, a, a, b - a});
        return segs;
    }
    for (int32_t u = u0; u < u1; ++u) {
        const zero_unit &x = L->unit[u];
        if (x.shard == 0)
            continue;
        const int64_t j0 = x.offset + (int64_t)rank * x.shard;  // global start
        const int64_t k0 = x.local_offset;                      // local start
        Segment s;
        s.g_off = (grad_index == ZERO_GLOBAL ? j0 : k0) - gbase;
        s.s_off = state_index == ZERO_GLOBAL ? j0 : k0;
        s.o_off = out_index == ZERO_GLOBAL ? j0 : k0;
        s.len = x.shard;
        if (!segs.empty()) {
            Segment &p = segs.back();
            if (p.g_off + p.len == s.g_off && p.s_off + p.len == s.s_off &&
                p.o_off + p.len == s.o_off) {
                p.len += s.len;
                continue;
            }
        }
        segs.push_back(s);
    }
    return segs;
}

int64_t selected_elements(const zero_layout *L, int32_t rank)
{
    return rank < 0 ? L->padded : L->shard;
}

// Residue that makes (addr / elem + off + h) a multiple of `mult`, as a
// constraint on h modulo `mult`.
static inline int64_t need_mod(const void *p, int elem, int64_t off, int mult)
{
    int64_t e = (int64_t)((uintptr_t)p / (uintptr_t)elem) + off;
    int64_t r = e % mult;
    return (mult - r) % mult;
}

// Quad accesses need 16 bytes of alignment for fp32 buffers and 8 bytes for
// bf16 buffers; either way a multiple of kQuad elements from a suitably
// aligned address.
static inline int64_t quad_need(const void *p, int elem, int64_t off)
{
    const int bytes = elem == 4 ? 16 : 8;
    const int mult = bytes / elem;  // elements per aligned unit: 4 in both cases
    return need_mod(p, elem, off, mult);
}

// The wave grid's phase for a vector body that starts at element offsets
// (g, s, o): the p in 0..15 quads that puts the most streamed bytes at a
// 128-byte line when each wave's span starts, counting each gradient's read,
// each state array's read and write, and the bf16 output's write, writes
// twice (a store covering part of a line costs more than a load).  A wave
// span is 64 quads, a whole number of lines for every element size, so only
// the span starts matter; any p keeps quad alignment.
static int line_phase(const Request &rq, int gsize, int64_t g, int64_t s, int64_t o)
{
    auto at_line = [](const void *base, int elem, int64_t off, int p, int shift_elems) {
        const uintptr_t a = (uintptr_t)base + (uintptr_t)(off * elem);
        return (a - (uintptr_t)(shift_elems * p) * (uintptr_t)elem) % 128u == 0;
    };
    int best = 0, best_score = -1;
    for (int p = 0; p < 16; ++p) {
        int score = 0;
        for (int q = 0; q < rq.n_grads; ++q)
            if (at_line(rq.grads[q], gsize, g, p, kQuad))
                score += gsize;
        for (int i = 0; i < rq.n_state_ptrs; ++i)
            if (rq.state_ptrs[i] && at_line(rq.state_ptrs[i], 4, s, p, kQuad))
                score += 4 + 2 * 4;
        if (rq.out_ptr && at_line(rq.out_ptr, 2, o, p, kQuad))
            score += 2 * 2;
        if (score > best_score) {
            best_score = score;
            best = p;
        }
    }
    return best;
}

std::vector<Piece> build_pieces(const std::vector<Segment> &segs, const Request &rq)
{
    std::vector<Piece> pieces;
    const int gsize = rq.grad_dtype == ZERO_BF16 ? 2 : 4;
    for (const Segment &s : segs) {
        // The head h in [0, kQuad) after which every buffer is quad-aligned;
        // none exists when the buffers' phases disagree.
        int64_t head = -1;
        for (int64_t h = 0; h < kQuad && head < 0; ++h) {
            bool ok = true;
            for (int q = 0; q < rq.n_grads && ok; ++q)
                ok = quad_need(rq.grads[q], gsize, s.g_off) == h;
            for (int i = 0; i < rq.n_state_ptrs && ok; ++i)
                if (rq.state_ptrs[i])
                    ok = quad_need(rq.state_ptrs[i], 4, s.s_off) == h;
            if (ok && rq.out_ptr)
                ok = quad_need(rq.out_ptr, 2, s.o_off) == h;
            if (ok)
                head = h;
        }
        if (head < 0 || head >= s.len) {
            pieces.push_back({s.g_off, s.s_off, s.o_off, s.len, false});
            continue;
        }
        const int64_t body = (s.len - head) / kQuad * kQuad;
        if (head > 0)
            pieces.push_back({s.g_off, s.s_off, s.o_off, head, false});
        if (body > 0) {
            Piece pc{s.g_off + head, s.s_off + head, s.o_off + head, body, true};
            pc.phase = line_phase(rq, gsize, pc.g_off, pc.s_off, pc.o_off);
            pieces.push_back(pc);
        }
        const int64_t tail_at = head + body;
        if (tail_at < s.len)
            pieces.push_back({s.g_off + tail_at, s.s_off + tail_at, s.o_off + tail_at,
                              s.len - tail_at, false});
    }
    return pieces;
}

bool segment_vec_aligned(const Segment &s, const Request &rq)
{
    // 16 bytes at the segment start for every gradient (8 bf16 / 4 fp32
    // elements) and for g_out.
    const int gsize = rq.grad_dtype == ZERO_BF16 ? 2 : 4;
    for (int q = 0; q < rq.n_grads; ++q)
        if (need_mod(rq.grads[q], gsize, s.g_off, 16 / gsize) != 0)
            return false;
    for (int i = 0; i < rq.n_state_ptrs; ++i)
        if (rq.state_ptrs[i] && need_mod(rq.state_ptrs[i], 4, s.s_off, 4) != 0)
            return false;
    return true;
}

int64_t norm_partials_bound(const zero_layout *L, int32_t rank)
{
    // One partial per kNormSpan-element tile of each segment, whose first
    // tile starts up to 56 elements before it: ceil((len + phase) / 512) <=
    // len / 512 + 2 per segment; at most one segment per unit (one in total
    // for rank < 0).
    const int64_t segs = rank < 0 ? 1 : (L->n_units > 0 ? L->n_units : 1);
    return selected_elements(L, rank) / kNormSpan + 2 * segs;
}

bool layouts_match(const zero_layout *from, const zero_layout *to)
{
    return layout_ok(from) && layout_ok(to) && from->numel == to->numel;
}

std::vector<ReshardRun> build_reshard_runs(const zero_layout *from, const zero_layout *to,
                                           int32_t dst_rank)
{
    std::vector<ReshardRun> runs;
    auto add = [&runs](const ReshardRun &r) {
        if (r.len <= 0)
            return;
        if (!runs.empty()) {
            ReshardRun &p = runs.back();
            const bool src_next = r.src_rank < 0 ? p.src_rank < 0
                                                 : p.src_rank == r.src_rank && p.src_k + p.len == r.src_k;
            if (src_next && p.dst_k + p.len == r.dst_k) {
                p.len += r.len;
                return;
            }
        }
        runs.push_back(r);
    };
    // An element is identified by its stream position: its index in the
    // concatenation of every unit's unpadded elements, in unit order.  The
    // destination's stream positions only increase, so one forward walk over
    // the source units finds every owner.
    int32_t a = 0;
    int64_t a_start = 0, b_start = 0;
    for (int32_t u = 0; u < to->n_units; ++u) {
        const zero_unit &y = to->unit[u];
        if (y.shard > 0) {
            // positions within unit u that dst_rank's slice covers
            const int64_t p0 = (int64_t)dst_rank * y.shard, p1 = p0 + y.shard;
            const int64_t live = std::min(p1, y.numel);
            for (int64_t s = b_start + p0, s_end = b_start + live; s < s_end;) {
                while (a + 1 < from->n_units && s >= a_start + from->unit[a].numel)
                    a_start += from->unit[a++].numel;  // equal totals: s lies in some unit
                const zero_unit &x = from->unit[a];
                const int64_t pos = s - a_start;
                const int64_t q = pos / x.shard;  // x.shard > 0: the unit holds s
                const int64_t end =
                    std::min(s_end, a_start + std::min((q + 1) * x.shard, x.numel));
                add({(int32_t)q, x.local_offset + (pos - q * x.shard),
                     y.local_offset + (s - b_start - p0), end - s});
                s = end;
            }
            const int64_t z0 = std::max(p0, live);
            add({-1, 0, y.local_offset + (z0 - p0), p1 - z0});
        }
        b_start += y.numel;
    }
    return runs;
}

int64_t norm_tree_scratch(int64_t n)
{
    // sum over the levels of ceil(n / kNormFanIn^k), k >= 1, until one value
    int64_t total = 0;
    while (n > 1) {
        n = (n + kNormFanIn - 1) / kNormFanIn;
        total += n;
    }
    return total;
}

}  // namespace zero

using namespace zero;

extern "C" size_t zero_layout_bytes(int32_t n_units)
{
    if (n_units < 0)
        n_units = 0;
    return sizeof(zero_layout) + sizeof(zero_unit) * (size_t)n_units;
}

// The packer proper: unit u pads to a multiple of N g_u (g_u = 1 when
// `granule` is null).
static zero_status pack_impl(int32_t n_ranks, int32_t n_units, const int64_t *unit_numel,
                             const int64_t *granule, zero_layout *layout, size_t layout_bytes,
                             size_t *bytes_needed)
{
    if (n_ranks < 1 || n_units < 0 || n_units > ZERO_MAX_UNITS ||
        (n_units > 0 && !unit_numel))
        return ZERO_EINVAL;
    const size_t need = zero_layout_bytes(n_units);
    if (bytes_needed)
        *bytes_needed = need;
    int64_t off = 0, numel = 0;
    for (int32_t u = 0; u < n_units; ++u) {  // validate and check the totals first
        const int64_t p = unit_numel[u], g = granule ? granule[u] : 1;
        if (p < 0 || g < 1 || p % g != 0)
            return ZERO_EINVAL;
        int64_t ng, padded;
        if (__builtin_mul_overflow((int64_t)n_ranks, g, &ng) || p > INT64_MAX - (ng - 1))
            return ZERO_ERANGE;
        padded = (p + ng - 1) / ng * ng;
        if (off > INT64_MAX - padded || numel > INT64_MAX - p)
            return ZERO_ERANGE;
        off += padded;
        numel += p;
    }
    if (!layout)
        return ZERO_OK;  // size query
    if (layout_bytes < need)
        return ZERO_ENOSPC;
    layout->magic = ZERO_LAYOUT_MAGIC;
    layout->n_ranks = n_ranks;
    layout->n_units = n_units;
    layout->reserved = 0;
    int64_t loff = 0;
    off = 0;
    for (int32_t u = 0; u < n_units; ++u) {
        zero_unit &x = layout->unit[u];
        x.numel = unit_numel[u];
        x.granule = granule ? granule[u] : 1;
        const int64_t rows = x.numel / x.granule;
        x.shard = (rows + n_ranks - 1) / n_ranks * x.granule;  // ceil(rows / N) rows
        x.padded = x.shard * n_ranks;
        x.offset = off;
        x.local_offset = loff;
        off += x.padded;
        loff += x.shard;
    }
    layout->numel = numel;
    layout->padded = off;
    layout->shard = loff;
    return ZERO_OK;
}

extern "C" zero_status zero_pack(int32_t n_ranks, int32_t n_units, const int64_t *unit_numel,
                                 zero_layout *layout, size_t layout_bytes, size_t *bytes_needed)
{
    return pack_impl(n_ranks, n_units, unit_numel, nullptr, layout, layout_bytes, bytes_needed);
}

extern "C" zero_status zero_pack_rows(int32_t n_ranks, int32_t n_units, const int64_t *unit_numel,
                                      const int64_t *unit_granule, zero_layout *layout,
                                      size_t layout_bytes, size_t *bytes_needed)
{
    if (n_units > 0 && !unit_granule)
        return ZERO_EINVAL;
    return pack_impl(n_ranks, n_units, unit_numel, unit_granule, layout, layout_bytes,
                     bytes_needed);
}

extern "C" zero_status zero_global_index(const zero_layout *L, int32_t rank, int64_t k, int64_t *j)
{
    if (!layout_ok(L) || !j || rank < 0 || rank >= L->n_ranks || k < 0 || k >= L->shard)
        return ZERO_EINVAL;
    // binary search for the unit whose local range holds k
    int32_t lo = 0, hi = L->n_units - 1;
    while (lo < hi) {
        int32_t mid = lo + (hi - lo + 1) / 2;
        if (L->unit[mid].local_offset <= k)
            lo = mid;
        else
            hi = mid - 1;
    }
    while (L->unit[lo].shard == 0 || k >= L->unit[lo].local_offset + L->unit[lo].shard)
        ++lo;  // skip empty units sharing the same local offset
    const zero_unit &x = L->unit[lo];
    *j = x.offset + (int64_t)rank * x.shard + (k - x.local_offset);
    return ZERO_OK;
}

extern "C" zero_status zero_owner(const zero_layout *L, int64_t j, int32_t *rank, int64_t *k)
{
    if (!layout_ok(L) || !rank || !k || j < 0 || j >= L->padded)
        return ZERO_EINVAL;
    int32_t lo = 0, hi = L->n_units - 1;
    while (lo < hi) {
        int32_t mid = lo + (hi - lo + 1) / 2;
        if (L->unit[mid].offset <= j)
            lo = mid;
        else
            hi = mid - 1;
    }
    while (L->unit[lo].padded == 0 || j >= L->unit[lo].offset + L->unit[lo].padded)
        ++lo;
    const zero_unit &x = L->unit[lo];
    const int64_t within = j - x.offset;
    *rank = (int32_t)(within / x.shard);
    *k = x.local_offset + within % x.shard;
    return ZERO_OK;
}

// Placement of n buffers in one allocation: buffer i starts at the first
// byte at or after the previous buffer's end whose offset modulo 2 MiB is
// (i * 256 KiB) mod 2 MiB.  Device memory is mapped in 2 MiB pages, so the
// phase of a buffer inside its page is the same physically as virtually;
// staggering the phases keeps buffers that are streamed side by side off the
// same HBM channels at the same moment.  One exception, measured: in a run
// of more than 32 buffers of one size (the gradients of a staged step) whose
// bases would lie a multiple of 2 MiB plus 32 MiB apart modulo 64 MiB (beyond
// the stagger), each buffer after the first starts one page later; at the
// rank counts that spacing falls on, the staged step ran 1.2 to 7.2 points
// faster with it (bf16 96 and 160 ranks, fp32 64 and 192), and those runs
// are the only ones it changes.
extern "C" zero_status zero_arena_plan(int32_t n_buffers, const int64_t *bytes, int64_t *offsets,
                                       int64_t *total_bytes)
{
    constexpr int64_t kPage = int64_t(2) << 20;
    constexpr int64_t kStagger = int64_t(256) << 10;
    constexpr int32_t kManyBuffers = 32;
    constexpr int64_t kAliasPages = 32;  // 64 MiB
    if (n_buffers < 0 || !total_bytes || (n_buffers > 0 && (!bytes || !offsets)))
        return ZERO_EINVAL;
    int64_t end = 0;
    for (int32_t i = 0; i < n_buffers; ++i)
        if (bytes[i] < 0)
            return ZERO_EINVAL;
    int32_t run_begin = 0, run_end = 0;  // the maximal run of equal sizes holding buffer i
    for (int32_t i = 0; i < n_buffers; ++i) {
        if (i >= run_end) {
            run_begin = i;
            run_end = i + 1;
            while (run_end < n_buffers && bytes[run_end] == bytes[i])
                ++run_end;
        }
        const int64_t phase = ((int64_t)i * kStagger) % kPage;
        // smallest start >= end with start % kPage == phase
        const int64_t base = end / kPage * kPage;
        int64_t start = base + phase;
        if (start < end)
            start += kPage;
        if (i > run_begin && run_end - run_begin > kManyBuffers &&
            ((start - offsets[i - 1]) / kPage) % kAliasPages == kAliasPages / 2) {
            if (start > INT64_MAX - kPage)
                return ZERO_ERANGE;
            start += kPage;
        }
        if (start > INT64_MAX - bytes[i])
            return ZERO_ERANGE;
        offsets[i] = start;
        end = start + bytes[i];
    }
    *total_bytes = end;
    return ZERO_OK;
}
