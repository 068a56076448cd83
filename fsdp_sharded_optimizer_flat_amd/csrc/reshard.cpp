// reshard.cpp -- resharding a sharded checkpoint to a new layout.
//
// "ZeRO and FSDP sharding", Implementation notes: each rank saves only its own
// shard, and loading under a different N reshards.  "Learn: ZeRO & FSDP",
// section 5 (FSDP1 vs FSDP2): FSDP2's per-parameter, dim-0 shards are another
// layout of the same elements.  Both are one map: element p of unit u sits at rank
// p / S_u, local index L_u + p mod S_u, in any layout; a reshard copies every
// element of the destination shard from where the source layout keeps it and
// zero-fills positions at or past P_u.
#include <hip/hip_runtime.h>

#include <cstring>

#include "zero_internal.h"

using namespace zero;

namespace {

zero_status check_reshard(const zero_layout *from, const void *const *src, const zero_layout *to,
                          int32_t dst_rank, const void *dst, int32_t dtype, int *elem)
{
    if (!layouts_match(from, to) || dst_rank < 0 || dst_rank >= to->n_ranks || !src ||
        (!dst && to->shard > 0) || (dtype != ZERO_F32 && dtype != ZERO_BF16))
        return ZERO_EINVAL;
    const int e = dtype == ZERO_F32 ? 4 : 2;
    if ((uintptr_t)dst % (uintptr_t)e != 0)
        return ZERO_EALIGN;
    const uintptr_t d0 = (uintptr_t)dst, d1 = d0 + (uintptr_t)to->shard * e;
    for (int32_t q = 0; q < from->n_ranks; ++q) {
        if (from->shard > 0 && !src[q])
            return ZERO_EINVAL;
        if ((uintptr_t)src[q] % (uintptr_t)e != 0)
            return ZERO_EALIGN;
        const uintptr_t s0 = (uintptr_t)src[q], s1 = s0 + (uintptr_t)from->shard * e;
        if (s0 < d1 && d0 < s1 && from->shard > 0 && to->shard > 0)
            return ZERO_EINVAL;  // the destination would overwrite a source
    }
    *elem = e;
    return ZERO_OK;
}

}  // namespace

extern "C" zero_status zero_reshard(const zero_layout *from, const void *const *src,
                                    const zero_layout *to, int32_t dst_rank, void *dst,
                                    int32_t dtype, void *stream)
{
    int elem = 0;
    zero_status st = check_reshard(from, src, to, dst_rank, dst, dtype, &elem);
    if (st != ZERO_OK)
        return st;
    const std::vector<ReshardRun> runs = build_reshard_runs(from, to, dst_rank);
    const int err = launch_reshard(runs, src, dst, elem, stream);
    return err == hipSuccess ? ZERO_OK : hip_fail(err, "zero_reshard");
}

extern "C" zero_status zero_reshard_host(const zero_layout *from, const void *const *src,
                                         const zero_layout *to, int32_t dst_rank, void *dst,
                                         int32_t dtype)
{
    int elem = 0;
    zero_status st = check_reshard(from, src, to, dst_rank, dst, dtype, &elem);
    if (st != ZERO_OK)
        return st;
    char *d = static_cast<char *>(dst);
    for (const ReshardRun &r : build_reshard_runs(from, to, dst_rank)) {
        if (r.src_rank < 0)
            std::memset(d + r.dst_k * elem, 0, (size_t)r.len * elem);
        else
            std::memcpy(d + r.dst_k * elem,
                        static_cast<const char *>(src[r.src_rank]) + r.src_k * elem,
                        (size_t)r.len * elem);
    }
    return ZERO_OK;
}

extern "C" zero_status zero_reshard_traffic(const zero_layout *from, const zero_layout *to,
                                            int32_t dst_rank, int32_t dtype, double *bytes,
                                            int64_t *elements)
{
    if (!layouts_match(from, to) || dst_rank < 0 || dst_rank >= to->n_ranks || !bytes ||
        !elements || (dtype != ZERO_F32 && dtype != ZERO_BF16))
        return ZERO_EINVAL;
    const int elem = dtype == ZERO_F32 ? 4 : 2;
    int64_t copied = 0;
    for (const ReshardRun &r : build_reshard_runs(from, to, dst_rank))
        if (r.src_rank >= 0)
            copied += r.len;
    *elements = to->shard;
    *bytes = (double)elem * (double)(copied + to->shard);  // read what is copied, write it all
    return ZERO_OK;
}
