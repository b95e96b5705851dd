// ZeRO-3 / FSDP prefetch: the host-side scheduler of the per-unit parameter
// gathers.
//
// ZeRO-3 keeps only a shard of every weight on each rank; right before a
// unit (a layer) runs, its full weights are all-gathered, the next unit's
// gather starts while the current one computes, and a unit's full weights
// are dropped once it is done (podcast summary of "Training at thousands of
// GPUs", section "ZeRO optimizer"; CS336 lecture 8 notes, "Code example:
// FSDP").
//
// The object owns no device memory: the caller gives it a ring of unit
// buffers and a gather stream.  issue() gathers a flat range into the next
// buffer with zs_gather on the gather stream, after the compute that last
// released that buffer; acquire() makes a compute stream wait for that
// gather; release() marks the compute stream's use of the buffer done.  A
// buffer goes free -> issued -> acquired -> free, and calls out of that
// order are refused, so the host cannot race a gather against a compute
// that still reads the buffer.  HIP events are the only resources it
// creates.

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <new>
#include <vector>

#include "zs_internal.h"

struct zs_prefetch {
    const zs_layout* L = nullptr;
    std::vector<const uint16_t*> shards;
    std::vector<uint16_t*> buffers;
    int64_t buffer_elems = 0;
    hipStream_t gs = nullptr;
    std::vector<hipEvent_t> ready;      // per buffer: its gather is done
    std::vector<hipEvent_t> released;   // per buffer: its compute is done
    std::vector<char> state;            // per buffer: kFree/kIssued/kAcquired
    std::vector<char> ever_released;
    int32_t cursor = 0;
};

namespace {

using zs::fail;

constexpr char kFree = 0, kIssued = 1, kAcquired = 2;

int hip_fail(hipError_t e, const char* what)
{
    return fail(ZS_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

void destroy(zs_prefetch* P)
{
    for (hipEvent_t e : P->ready)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : P->released)
        if (e) (void)hipEventDestroy(e);
    delete P;
}

int check_slot(const zs_prefetch* P, int32_t slot)
{
    if (!P) return fail(ZS_EINVAL, "prefetch is NULL");
    if (slot < 0 || slot >= (int32_t)P->buffers.size())
        return fail(ZS_ERANGE, "slot %d outside [0, %d)", slot,
                    (int)P->buffers.size());
    return ZS_OK;
}

}  // namespace

extern "C" int zs_prefetch_create(const zs_layout* L,
                                  const uint16_t* const* shards,
                                  uint16_t* const* buffers,
                                  int32_t n_buffers, int64_t buffer_elems,
                                  void* gather_stream, zs_prefetch** out)
{
    zs::clear_error();
    if (!out) return fail(ZS_EINVAL, "out is NULL");
    *out = nullptr;
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    if (L->world > ZS_GATHER_MAX_WORLD)
        return fail(ZS_EINVAL, "world %d above %d", L->world,
                    ZS_GATHER_MAX_WORLD);
    if (!shards || !buffers)
        return fail(ZS_EINVAL, "shards and buffers must be non-NULL");
    if (n_buffers < 1 || n_buffers > 64)
        return fail(ZS_EINVAL, "n_buffers %d outside [1, 64]", n_buffers);
    if (buffer_elems < 0)
        return fail(ZS_EINVAL, "buffer_elems %lld < 0",
                    (long long)buffer_elems);
    for (int32_t r = 0; r < L->world; ++r)
        if (!shards[r]) return fail(ZS_EINVAL, "shards[%d] is NULL", r);
    for (int32_t k = 0; k < n_buffers; ++k) {
        if (!buffers[k]) return fail(ZS_EINVAL, "buffers[%d] is NULL", k);
        if (reinterpret_cast<uintptr_t>(buffers[k]) & 15u)
            return fail(ZS_EALIGN, "buffers[%d] not 16-byte aligned", k);
    }
    zs_prefetch* P = new (std::nothrow) zs_prefetch;
    if (!P) return fail(ZS_ENOMEM, "host allocation");
    try {
        P->L = L;
        P->shards.assign(shards, shards + L->world);
        P->buffers.assign(buffers, buffers + n_buffers);
        P->buffer_elems = buffer_elems;
        P->gs = static_cast<hipStream_t>(gather_stream);
        P->ready.assign(n_buffers, nullptr);
        P->released.assign(n_buffers, nullptr);
        P->state.assign(n_buffers, kFree);
        P->ever_released.assign(n_buffers, 0);
    } catch (const std::bad_alloc&) {
        delete P;
        return fail(ZS_ENOMEM, "host allocation");
    }
    hipError_t e = hipSuccess;
    for (int32_t k = 0; e == hipSuccess && k < n_buffers; ++k) {
        e = hipEventCreateWithFlags(&P->ready[k], hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&P->released[k],
                                        hipEventDisableTiming);
    }
    if (e != hipSuccess) {
        destroy(P);
        return hip_fail(e, "hipEventCreateWithFlags");
    }
    *out = P;
    return ZS_OK;
}

extern "C" int zs_prefetch_issue(zs_prefetch* P, int64_t flat_lo,
                                 int64_t flat_hi, int32_t* slot)
{
    zs::clear_error();
    if (!P) return fail(ZS_EINVAL, "prefetch is NULL");
    if (!slot) return fail(ZS_EINVAL, "slot is NULL");
    if (flat_lo < 0 || flat_hi < flat_lo || flat_hi > P->L->flat_numel)
        return fail(ZS_ERANGE, "range [%lld, %lld) outside [0, %lld]",
                    (long long)flat_lo, (long long)flat_hi,
                    (long long)P->L->flat_numel);
    if (flat_hi - flat_lo > P->buffer_elems)
        return fail(ZS_ERANGE, "range of %lld elements above the buffers' "
                    "%lld", (long long)(flat_hi - flat_lo),
                    (long long)P->buffer_elems);
    const int32_t k = P->cursor;
    if (P->state[k] != kFree)
        return fail(ZS_EINVAL, "the next buffer (%d) is still in use: "
                    "release it first", k);
    if (P->ever_released[k]) {
        const hipError_t e = hipStreamWaitEvent(P->gs, P->released[k], 0);
        if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    }
    const int rc = zs_gather(P->L, P->shards.data(), flat_lo, flat_hi,
                             P->buffers[k], P->gs);
    if (rc) return rc;
    const hipError_t e = hipEventRecord(P->ready[k], P->gs);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    P->state[k] = kIssued;
    P->cursor = (P->cursor + 1) % (int32_t)P->buffers.size();
    *slot = k;
    return ZS_OK;
}

extern "C" int zs_prefetch_acquire(zs_prefetch* P, int32_t slot,
                                   void* compute_stream, uint16_t** buffer)
{
    zs::clear_error();
    int rc = check_slot(P, slot);
    if (rc) return rc;
    if (P->state[slot] != kIssued)
        return fail(ZS_EINVAL, "buffer %d was not issued", slot);
    const hipError_t e = hipStreamWaitEvent(
        static_cast<hipStream_t>(compute_stream), P->ready[slot], 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    P->state[slot] = kAcquired;
    if (buffer) *buffer = P->buffers[slot];
    return ZS_OK;
}

extern "C" int zs_prefetch_release(zs_prefetch* P, int32_t slot,
                                   void* compute_stream)
{
    zs::clear_error();
    int rc = check_slot(P, slot);
    if (rc) return rc;
    if (P->state[slot] != kAcquired)
        return fail(ZS_EINVAL, "buffer %d was not acquired", slot);
    const hipError_t e = hipEventRecord(P->released[slot],
                                        static_cast<hipStream_t>(
                                            compute_stream));
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    P->state[slot] = kFree;
    P->ever_released[slot] = 1;
    return ZS_OK;
}

extern "C" void zs_prefetch_free(zs_prefetch* P)
{
    if (P) destroy(P);
}
