// offload.cpp -- the ZeRO-Offload step with its PCIe transfers, pipelined.
//
// "Learn: ZeRO & FSDP", section 6: ZeRO-Offload keeps the optimizer state and
// the fp32 step on the CPU; the reduced gradient comes down over PCIe, the
// CPU runs AdamW, the updated parameters go back up -- the single PCIe link
// is the bottleneck.  Here one rank's shard is cut into chunks that flow
// through two pinned staging slots: the device-to-host copy of chunk c + 1,
// the host step on chunk c and the host-to-device copy of chunk c - 1
// proceed at the same time (two caller streams, one per PCIe direction).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "zero_internal.h"

using namespace zero;

namespace {

struct Events {
    hipEvent_t down[2] = {nullptr, nullptr}, up[2] = {nullptr, nullptr};
    ~Events()
    {
        for (int i = 0; i < 2; ++i) {
            if (down[i])
                (void)hipEventDestroy(down[i]);
            if (up[i])
                (void)hipEventDestroy(up[i]);
        }
    }
};

}  // namespace

extern "C" zero_status zero_offload_step(const zero_layout *L, int32_t rank,
                                         const float *d_grad, float *h_grad_stage,
                                         float *master, float *exp_avg, float *exp_avg_sq,
                                         uint16_t *h_out_stage, uint16_t *d_out,
                                         int64_t chunk, const zero_adamw_scalars *sc,
                                         int32_t n_threads, void *stream_down, void *stream_up)
{
    if (!layout_ok(L) || rank < 0 || rank >= L->n_ranks || !d_grad || !h_grad_stage || !master ||
        !exp_avg || !exp_avg_sq || !h_out_stage || !d_out || !sc || sc->t < 1 || chunk < 1)
        return ZERO_EINVAL;
    if (((uintptr_t)d_grad | (uintptr_t)h_grad_stage | (uintptr_t)master | (uintptr_t)exp_avg |
         (uintptr_t)exp_avg_sq) % 4 != 0 ||
        ((uintptr_t)h_out_stage | (uintptr_t)d_out) % 2 != 0)
        return ZERO_EALIGN;
    const int64_t S = L->shard;
    if (S == 0)
        return ZERO_OK;
    hipStream_t sd = reinterpret_cast<hipStream_t>(stream_down);
    hipStream_t su = reinterpret_cast<hipStream_t>(stream_up);
    Events ev;
    for (int i = 0; i < 2; ++i) {
        int e = hipEventCreateWithFlags(&ev.down[i], hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&ev.up[i], hipEventDisableTiming);
        if (e != hipSuccess)
            return hip_fail(e, "zero_offload_step events");
    }
    const int64_t nchunks = (S + chunk - 1) / chunk;
    auto span = [&](int64_t c, int64_t &k0, int64_t &len) {
        k0 = c * chunk;
        len = std::min<int64_t>(chunk, S - k0);
    };
    auto down = [&](int64_t c) -> int {
        int64_t k0, len;
        span(c, k0, len);
        const int slot = (int)(c & 1);
        int e = hipMemcpyAsync(h_grad_stage + slot * chunk, d_grad + k0, (size_t)len * 4,
                               hipMemcpyDeviceToHost, sd);
        if (e == hipSuccess)
            e = hipEventRecord(ev.down[slot], sd);
        return e;
    };
    // one-unit, one-rank layout of a chunk: every buffer is indexed 0..len-1
    alignas(8) unsigned char lbuf[sizeof(zero_layout) + sizeof(zero_unit)];
    zero_layout *CL = reinterpret_cast<zero_layout *>(lbuf);

    int e = down(0);
    if (e != hipSuccess)
        return hip_fail(e, "zero_offload_step copy down");
    for (int64_t c = 0; c < nchunks; ++c) {
        const int slot = (int)(c & 1);
        int64_t k0, len;
        span(c, k0, len);
        if (c + 1 < nchunks) {  // the next chunk comes down while this one is stepped
            e = down(c + 1);
            if (e != hipSuccess)
                return hip_fail(e, "zero_offload_step copy down");
        }
        e = hipEventSynchronize(ev.down[slot]);
        if (e == hipSuccess && c >= 2)  // the up copy that last read this out slot is done
            e = hipEventSynchronize(ev.up[slot]);
        if (e != hipSuccess)
            return hip_fail(e, "zero_offload_step wait");
        zero_status st = zero_pack(1, 1, &len, CL, sizeof lbuf, nullptr);
        if (st != ZERO_OK)
            return st;
        const void *g = h_grad_stage + slot * chunk;
        st = zero_step_host(CL, 0, &g, 1, ZERO_F32, ZERO_LOCAL, 1.0f, master + k0, exp_avg + k0,
                            exp_avg_sq + k0, ZERO_LOCAL, h_out_stage + slot * chunk, ZERO_LOCAL,
                            sc, n_threads);
        if (st != ZERO_OK)
            return st;
        e = hipMemcpyAsync(d_out + k0, h_out_stage + slot * chunk, (size_t)len * 2,
                           hipMemcpyHostToDevice, su);
        if (e == hipSuccess)
            e = hipEventRecord(ev.up[slot], su);
        if (e != hipSuccess)
            return hip_fail(e, "zero_offload_step copy up");
    }
    e = hipStreamSynchronize(su);
    if (e == hipSuccess)
        e = hipStreamSynchronize(sd);
    return e == hipSuccess ? ZERO_OK : hip_fail(e, "zero_offload_step synchronize");
}
