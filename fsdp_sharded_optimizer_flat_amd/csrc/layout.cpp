// layout.cpp -- the flat-buffer packer's host side: unit padding, shard
// ownership, the local <-> global index maps, and the element runs ("pieces")
// that the kernels stream over.
//
// "ZeRO and FSDP sharding", How it works: each unit's parameters are flattened
// into one buffer padded to a multiple of N, and rank r owns slice r.  Same
// page, Pitfalls: without the padding the last rank's slice is corrupted.
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
        if (x.numel < 0 || x.shard < 0 || x.padded != x.shard * L->n_ranks || x.padded < x.numel ||
            x.padded - x.numel >= L->n_ranks || x.offset != off || x.local_offset != loff)
            return false;
        off += x.padded;
        loff += x.shard;
        numel += x.numel;
    }
    return off == L->padded && loff == L->shard && numel == L->numel;
}

std::vector<Segment> build_segments(const zero_layout *L, int32_t rank, int32_t grad_index,
                                    int32_t state_index, int32_t out_index)
{
    std::vector<Segment> segs;
    if (rank < 0) {  // every rank's slices: the whole flat buffer, identity map
        if (L->padded > 0)
            segs.push_back({0, 0, 0, L->padded});
        return segs;
    }
    for (int32_t u = 0; u < L->n_units; ++u) {
        const zero_unit &x = L->unit[u];
        if (x.shard == 0)
            continue;
        const int64_t j0 = x.offset + (int64_t)rank * x.shard;  // global start
        const int64_t k0 = x.local_offset;                      // local start
        Segment s;
        s.g_off = grad_index == ZERO_GLOBAL ? j0 : k0;
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
        if (body > 0)
            pieces.push_back({s.g_off + head, s.s_off + head, s.o_off + head, body, true});
        const int64_t tail_at = head + body;
        if (tail_at < s.len)
            pieces.push_back({s.g_off + tail_at, s.s_off + tail_at, s.o_off + tail_at,
                              s.len - tail_at, false});
    }
    return pieces;
}

bool segment_vec_aligned(const Segment &s, const Request &rq)
{
    const int gsize = rq.grad_dtype == ZERO_BF16 ? 2 : 4;
    for (int q = 0; q < rq.n_grads; ++q)
        if (quad_need(rq.grads[q], gsize, s.g_off) != 0)
            return false;
    for (int i = 0; i < rq.n_state_ptrs; ++i)
        if (rq.state_ptrs[i] && quad_need(rq.state_ptrs[i], 4, s.s_off) != 0)
            return false;
    return true;
}

int64_t norm_partials_bound(const zero_layout *L, int32_t rank)
{
    // One partial per started kNormSpan elements of each segment; at most one
    // segment per unit (one in total for rank < 0).
    const int64_t segs = rank < 0 ? 1 : (L->n_units > 0 ? L->n_units : 1);
    return selected_elements(L, rank) / kNormSpan + segs;
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

extern "C" zero_status zero_pack(int32_t n_ranks, int32_t n_units, const int64_t *unit_numel,
                                 zero_layout *layout, size_t layout_bytes, size_t *bytes_needed)
{
    if (n_ranks < 1 || n_units < 0 || n_units > ZERO_MAX_UNITS ||
        (n_units > 0 && !unit_numel))
        return ZERO_EINVAL;
    const size_t need = zero_layout_bytes(n_units);
    if (bytes_needed)
        *bytes_needed = need;
    if (!layout)
        return ZERO_OK;  // size query
    if (layout_bytes < need)
        return ZERO_ENOSPC;
    int64_t off = 0, loff = 0, numel = 0;
    for (int32_t u = 0; u < n_units; ++u) {
        const int64_t p = unit_numel[u];
        if (p < 0)
            return ZERO_EINVAL;
        if (p > INT64_MAX - n_ranks)
            return ZERO_ERANGE;
        const int64_t shard = (p + n_ranks - 1) / n_ranks;  // ceil(p / N)
        const int64_t padded = shard * n_ranks;
        if (off > INT64_MAX - padded || numel > INT64_MAX - p)
            return ZERO_ERANGE;
        off += padded;
        loff += shard;
        numel += p;
    }
    layout->magic = ZERO_LAYOUT_MAGIC;
    layout->n_ranks = n_ranks;
    layout->n_units = n_units;
    layout->reserved = 0;
    off = loff = 0;
    for (int32_t u = 0; u < n_units; ++u) {
        zero_unit &x = layout->unit[u];
        x.numel = unit_numel[u];
        x.shard = (x.numel + n_ranks - 1) / n_ranks;
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
