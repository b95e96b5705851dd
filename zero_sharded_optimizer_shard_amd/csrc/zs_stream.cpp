// ZeRO-2 streaming engine: the host-side scheduler that steps each bucket
// as soon as its gradients have arrived.
//
// ZeRO-2 keeps only this rank's share of the gradients: the reduce-scatter
// runs per bucket while backward is still producing the next buckets, and
// the optimizer work of a bucket can start once its slices are here
// (podcast summary of "Training at thousands of GPUs", sections "Data
// parallelism" and "ZeRO optimizer": buckets of bucket_cap_mb, overlap of
// communication and computation; DDP-to-ZeRO blog 3.3: overlap_comm).
//
// The engine owns no device memory.  The caller gives it a ring of staging
// slots (device buffers), one or more upload streams and one or more step
// streams.  Each arriving bucket (its W tiled gradient slices, in device or
// pinned host memory) is copied into the next slot on the next upload
// stream in turn, after the step that last read that slot; every `group`
// arrivals become one zs_buckets_step launch on the next step stream in
// turn, ordered after the group's copies by one event per upload stream
// they used.  Several upload streams are for hosts where one stream's copies
// leave the host link idle; on MI355X one stream of 25 MiB pinned copies
// already filled it (56 GB/s in a 70B-shaped host-fed step, within 1 % of
// four streams).  Spreading groups over several step streams lets one
// launch's tail overlap the next launch (groups touch disjoint buckets).
// HIP events are the only resources it creates, and it enqueues few stream
// packets: an event record after each group's copies and after each launch,
// and one wait on the upload stream per launch whose slots are reused (one
// record and one wait per bucket slowed a 70B-shaped step by a third on
// MI355X).
//
// Consecutive steps update the same state.  A bucket's launch in step t+1
// may land on another step stream than its launch in step t, and its slot
// may be one no launch has read yet, so nothing above orders the two.  Each
// step_begin after the first therefore makes every step stream wait for
// the work already queued on every other one (at most 8 x 7 waits per
// step), so the caller may queue steps back to back with no host sync.

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <new>
#include <vector>

#include "zs_internal.h"

struct zs_stream {
    const zs_layout* L = nullptr;
    int32_t group = 1;
    std::vector<uint16_t*> slots;
    int64_t slot_elems = 0;
    std::vector<hipStream_t> ups;     // upload streams, used in turn
    std::vector<hipStream_t> steps;
    // Events.  One per upload stream marks the pending group's copies on it
    // (each wait takes the event's latest record, so one event per stream
    // serves every group); a ring marks the group launches.  A slot is
    // reused n_slots arrivals after its last use, so at most n_slots
    // launches later: a ring of n_slots + 1 launch events still holds the
    // record of the launch that read it.
    std::vector<hipEvent_t> landed;   // per upload stream
    std::vector<hipEvent_t> fence;    // per step stream: its tail at the
                                      // start of a step
    std::vector<hipEvent_t> done;     // launch g at g % done.size()
    std::vector<int64_t> reader;      // per slot: last launch that read it
    std::vector<int64_t> waited;      // per (upload stream, step stream):
                                      // the last launch of that step stream
                                      // the upload stream waited on
    // the step in progress
    bool open = false;
    bool failed = false;              // a launch or a copy of it failed
    float* state = nullptr;
    uint16_t* pshard = nullptr;
    uint16_t* flat = nullptr;
    zs_adamw hp{};
    int64_t t = 0;
    std::vector<char> arrived;        // per bucket
    int32_t cursor = 0;               // next slot of the ring
    int64_t arrivals = 0;             // arrivals so far (all steps)
    uint32_t pend_ups = 0;            // upload streams the pending group used
    int64_t launches = 0;             // group launches so far (all steps)
    int32_t stepped = 0;              // buckets stepped in this step
    std::vector<int32_t> pend_ids, pend_slots;
};

namespace {

using zs::fail;

int64_t bucket_elems(const zs_layout* L, int32_t b)
{
    const int64_t tiles = (L->buckets[b].slice_numel + ZS_TILE - 1) / ZS_TILE;
    return tiles * L->world * ZS_TILE;
}

int hip_fail(hipError_t e, const char* what)
{
    return fail(ZS_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// A device call of the step failed: the step is abandoned (its pending group
// dropped) and later arrivals are refused until step_end closes it.  No
// launch reads the dropped group's slots, so no launch event orders their
// copies before the next copy into the same slot, which may run on another
// upload stream: the host waits for the upload streams the group used.
int abandon(zs_stream* S, int rc)
{
    for (size_t u = 0; u < S->ups.size(); ++u)
        if (S->pend_ups & (1u << u))
            (void)hipStreamSynchronize(S->ups[u]);
    S->failed = true;
    S->pend_ids.clear();
    S->pend_slots.clear();
    S->pend_ups = 0;
    return rc;
}

void destroy(zs_stream* S)
{
    for (hipEvent_t e : S->landed)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : S->fence)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : S->done)
        if (e) (void)hipEventDestroy(e);
    delete S;
}

// One zs_buckets_step over the pending arrivals, on the next step stream.
int launch_pending(zs_stream* S)
{
    const int32_t cnt = (int32_t)S->pend_ids.size();
    if (cnt == 0)
        return ZS_OK;
    if (cnt > ZS_MAX_GROUP)
        return abandon(S, fail(ZS_EINVAL, "%d pending buckets above %d", cnt,
                               ZS_MAX_GROUP));
    const int64_t g = S->launches;
    hipStream_t s = S->steps[g % (int64_t)S->steps.size()];
    // each upload stream is in order: one record after its last copy of the
    // group covers all of the group's copies on it
    hipError_t e = hipSuccess;
    for (size_t u = 0; u < S->ups.size(); ++u) {
        if (!(S->pend_ups & (1u << u)))
            continue;
        e = hipEventRecord(S->landed[u], S->ups[u]);
        if (e != hipSuccess)
            return abandon(S, hip_fail(e, "hipEventRecord"));
        e = hipStreamWaitEvent(s, S->landed[u], 0);
        if (e != hipSuccess)
            return abandon(S, hip_fail(e, "hipStreamWaitEvent"));
    }
    const uint16_t* grads[ZS_MAX_GROUP];
    for (int32_t i = 0; i < cnt; ++i)
        grads[i] = S->slots[S->pend_slots[i]];
    const int rc = zs_buckets_step(S->L, cnt, S->pend_ids.data(), grads,
                                   ZS_GRADS_TILED, 0, S->state, S->pshard,
                                   S->flat, &S->hp, S->t, s);
    if (rc) return abandon(S, rc);
    e = hipEventRecord(S->done[g % (int64_t)S->done.size()], s);
    if (e != hipSuccess) {
        // the launch is queued but no event marks its end, so no later copy
        // could wait for it before overwriting its slots: wait here
        (void)hipStreamSynchronize(s);
        return abandon(S, hip_fail(e, "hipEventRecord"));
    }
    for (int32_t k : S->pend_slots)
        S->reader[k] = g;
    ++S->launches;
    S->stepped += cnt;
    S->pend_ids.clear();
    S->pend_slots.clear();
    S->pend_ups = 0;
    return ZS_OK;
}

}  // namespace

extern "C" int zs_stream_create_multi(const zs_layout* L, int32_t group,
                                      uint16_t* const* slots, int32_t n_slots,
                                      int64_t slot_elems,
                                      void* const* upload_streams,
                                      int32_t n_upload_streams,
                                      void* const* step_streams,
                                      int32_t n_step_streams, zs_stream** out)
{
    zs::clear_error();
    if (!out) return fail(ZS_EINVAL, "out is NULL");
    *out = nullptr;
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    if (group < 1 || group > ZS_MAX_GROUP)
        return fail(ZS_EINVAL, "group %d outside [1, %d]", group,
                    ZS_MAX_GROUP);
    if (n_slots < group)
        return fail(ZS_EINVAL, "n_slots %d < group %d", n_slots, group);
    if (!slots) return fail(ZS_EINVAL, "slots is NULL");
    for (int32_t k = 0; k < n_slots; ++k) {
        if (!slots[k]) return fail(ZS_EINVAL, "slots[%d] is NULL", k);
        if (reinterpret_cast<uintptr_t>(slots[k]) & 15u)
            return fail(ZS_EALIGN, "slots[%d] not 16-byte aligned", k);
    }
    if (n_upload_streams < 1 || n_upload_streams > 8)
        return fail(ZS_EINVAL, "n_upload_streams %d outside [1, 8]",
                    n_upload_streams);
    if (!upload_streams) return fail(ZS_EINVAL, "upload_streams is NULL");
    if (n_step_streams < 1 || n_step_streams > 8)
        return fail(ZS_EINVAL, "n_step_streams %d outside [1, 8]",
                    n_step_streams);
    if (!step_streams) return fail(ZS_EINVAL, "step_streams is NULL");
    const int32_t nb = (int32_t)L->buckets.size();
    for (int32_t b = 0; b < nb; ++b)
        if (bucket_elems(L, b) > slot_elems)
            return fail(ZS_ERANGE, "slot_elems %lld < %lld elements of "
                        "bucket %d's tiled gradients", (long long)slot_elems,
                        (long long)bucket_elems(L, b), b);
    zs_stream* S = new (std::nothrow) zs_stream;
    if (!S) return fail(ZS_ENOMEM, "host allocation");
    try {
        S->L = L;
        S->group = group;
        S->slots.assign(slots, slots + n_slots);
        S->slot_elems = slot_elems;
        for (int32_t i = 0; i < n_upload_streams; ++i)
            S->ups.push_back(static_cast<hipStream_t>(upload_streams[i]));
        for (int32_t i = 0; i < n_step_streams; ++i)
            S->steps.push_back(static_cast<hipStream_t>(step_streams[i]));
        S->landed.assign((size_t)n_upload_streams, nullptr);
        S->fence.assign((size_t)n_step_streams, nullptr);
        S->done.assign((size_t)n_slots + 1, nullptr);
        S->reader.assign(n_slots, -1);
        S->waited.assign((size_t)n_upload_streams * n_step_streams, -1);
        S->arrived.assign(nb, 0);
        S->pend_ids.reserve(group);
        S->pend_slots.reserve(group);
    } catch (const std::bad_alloc&) {
        delete S;
        return fail(ZS_ENOMEM, "host allocation");
    }
    hipError_t e = hipSuccess;
    for (size_t j = 0; e == hipSuccess && j < S->landed.size(); ++j)
        e = hipEventCreateWithFlags(&S->landed[j], hipEventDisableTiming);
    for (size_t j = 0; e == hipSuccess && j < S->fence.size(); ++j)
        e = hipEventCreateWithFlags(&S->fence[j], hipEventDisableTiming);
    for (size_t j = 0; e == hipSuccess && j < S->done.size(); ++j)
        e = hipEventCreateWithFlags(&S->done[j], hipEventDisableTiming);
    if (e != hipSuccess) {
        destroy(S);
        return hip_fail(e, "hipEventCreateWithFlags");
    }
    *out = S;
    return ZS_OK;
}

extern "C" int zs_stream_create(const zs_layout* L, int32_t group,
                                uint16_t* const* slots, int32_t n_slots,
                                int64_t slot_elems, void* upload_stream,
                                void* const* step_streams,
                                int32_t n_step_streams, zs_stream** out)
{
    return zs_stream_create_multi(L, group, slots, n_slots, slot_elems,
                                  &upload_stream, 1, step_streams,
                                  n_step_streams, out);
}

extern "C" int zs_stream_step_begin(zs_stream* S, float* state,
                                    uint16_t* param_shard,
                                    uint16_t* full_flat, const zs_adamw* hp,
                                    int64_t step)
{
    zs::clear_error();
    if (!S) return fail(ZS_EINVAL, "stream is NULL");
    if (S->open) return fail(ZS_EINVAL, "a step is already open");
    if (!hp) return fail(ZS_EINVAL, "hp is NULL");
    if (step < 1) return fail(ZS_EINVAL, "step %lld < 1", (long long)step);
    if (!state) return fail(ZS_EINVAL, "state is NULL");
    if (!param_shard && !full_flat)
        return fail(ZS_EINVAL, "need param_shard or full_flat");
    if (!aligned16(state) || (param_shard && !aligned16(param_shard)) ||
        (full_flat && !aligned16(full_flat)))
        return fail(ZS_EALIGN, "device pointers must be 16-byte aligned");
    // order this step's launches after the previous steps' launches on
    // every other step stream (see the file header)
    const size_t ns = S->steps.size();
    if (S->launches > 0 && ns > 1) {
        hipError_t e = hipSuccess;
        for (size_t j = 0; e == hipSuccess && j < ns; ++j)
            e = hipEventRecord(S->fence[j], S->steps[j]);
        for (size_t i = 0; e == hipSuccess && i < ns; ++i)
            for (size_t j = 0; e == hipSuccess && j < ns; ++j)
                if (i != j)
                    e = hipStreamWaitEvent(S->steps[i], S->fence[j], 0);
        if (e != hipSuccess)
            return hip_fail(e, "ordering the step streams");
    }
    S->state = state;
    S->pshard = param_shard;
    S->flat = full_flat;
    S->hp = *hp;
    S->t = step;
    S->stepped = 0;
    S->pend_ids.clear();
    S->pend_slots.clear();
    S->pend_ups = 0;
    for (char& a : S->arrived) a = 0;
    S->failed = false;
    S->open = true;
    return ZS_OK;
}

extern "C" int zs_stream_arrive(zs_stream* S, int32_t bucket_id,
                                const uint16_t* src)
{
    zs::clear_error();
    if (!S) return fail(ZS_EINVAL, "stream is NULL");
    if (!S->open) return fail(ZS_EINVAL, "no step is open");
    if (S->failed)
        return fail(ZS_EINVAL, "an earlier call of this step failed: end "
                    "the step");
    const int32_t nb = (int32_t)S->L->buckets.size();
    if (bucket_id < 0 || bucket_id >= nb)
        return fail(ZS_ERANGE, "bucket_id %d outside [0, %d)", bucket_id,
                    nb);
    if (S->arrived[bucket_id])
        return fail(ZS_EINVAL, "bucket %d arrived twice in one step",
                    bucket_id);
    if (!src) return fail(ZS_EINVAL, "src is NULL");
    const int32_t k = S->cursor;
    S->cursor = (S->cursor + 1) % (int32_t)S->slots.size();
    const size_t u = (size_t)(S->arrivals % (int64_t)S->ups.size());
    hipStream_t up = S->ups[u];
    hipError_t e = hipSuccess;
    const int64_t r = S->reader[k];
    if (r >= 0) {
        // the copy overwrites what launch r read; launches complete in
        // order on each step stream, so one wait per upload stream, step
        // stream and launch
        const size_t j = (size_t)(r % (int64_t)S->steps.size());
        int64_t& w = S->waited[u * S->steps.size() + j];
        if (w < r) {
            e = hipStreamWaitEvent(up, S->done[r % (int64_t)S->done.size()],
                                   0);
            if (e != hipSuccess)
                return abandon(S, hip_fail(e, "hipStreamWaitEvent"));
            w = r;
        }
    }
    e = hipMemcpyAsync(S->slots[k], src,
                       (size_t)bucket_elems(S->L, bucket_id) * 2,
                       hipMemcpyDefault, up);
    if (e != hipSuccess) return abandon(S, hip_fail(e, "hipMemcpyAsync"));
    ++S->arrivals;
    S->arrived[bucket_id] = 1;
    S->pend_ids.push_back(bucket_id);
    S->pend_slots.push_back(k);
    S->pend_ups |= 1u << u;
    if ((int32_t)S->pend_ids.size() == S->group)
        return launch_pending(S);
    return ZS_OK;
}

extern "C" int zs_stream_step_end(zs_stream* S)
{
    zs::clear_error();
    if (!S) return fail(ZS_EINVAL, "stream is NULL");
    if (!S->open) return fail(ZS_EINVAL, "no step is open");
    S->open = false;
    if (S->failed)
        return fail(ZS_EINVAL, "the step was abandoned after an earlier "
                    "error; it is now closed");
    const int rc = launch_pending(S);
    if (rc) return rc;
    return S->stepped;
}

extern "C" void zs_stream_free(zs_stream* S)
{
    if (S) destroy(S);
}
