// ZeRO-3 / FSDP parameter gather: materialise a flat range of the bf16
// parameters (one layer, or any window) from the shards of all W ranks.
//
// ZeRO-3 keeps only a shard of every weight on each rank; right before a
// layer is used its full weight is all-gathered, the next layer's gather is
// started while the current one computes, and the full weight is dropped
// after use (podcast summary of "Training at thousands of GPUs", section
// "ZeRO optimizer"; CS336 lecture 8 notes, "Code example: FSDP").  The
// all-gather concatenates the ranks' slices in rank order, so position x of
// the flat buffer, inside bucket q at offset k, comes from rank
// r = k / slice_q, element q*S + k - r*slice_q of its shard.
//
// The kernel pulls: each workgroup, a single wave64, copies one
// 512-element chunk of one (bucket, rank) slice, clipped to the requested
// range, from that rank's shard to the output: 1 KiB per workgroup, one
// 16-byte access per thread, the stores streamed on to HBM with system
// scope (zsdev::stream_store); a launch covers only the (bucket, rank) rows
// that meet the range.  Measured on MI355X over the 34 gathers of a
// Llama-3-8B-shaped forward (stand-alone, three interleaved rounds): 85.2-
// 85.3 % of peak HBM bandwidth, against 82.6-82.8 % when every row of the
// first and last buckets is launched (5.2 % of the workgroups then find
// nothing to copy, at the start and end of each launch).  With all rows
// launched, in the benchmark, two interleaved rounds: one access per
// thread with streamed stores 82.6-82.7 % and 27.75 ms per forward
// pipelined beside the stand-in GEMMs, against 82.1 % and 28.0-28.2 ms for
// two accesses per thread with plain non-temporal stores; one access with
// plain stores 81.9-82.0 %, two with streamed stores 82.2 %.  Gathering
// the whole flat buffer in one launch: 84.6-84.8 % against 71 %.  Earlier, with two accesses per thread: 81.7 % with
// 128-thread workgroups, 79.1 % with 256 and 76.0 % with 512; four
// accesses per thread and larger chunks were slower.  On one GPU the W
// shards are W resident buffers; on a node they would be peer-mapped shards
// of the other GPUs read over xGMI.  2 B read + 2 B written per element,
// 16-byte non-temporal accesses except at a ragged end; bounded by HBM
// bandwidth.  Whole-tensor layouts take each tensor whole from its owner
// (gather_tensors below).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "zs_device.h"
#include "zs_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 64;                     // one wave per workgroup
constexpr int kVec = 8;                         // bf16 per 16-byte access
constexpr int kPerThread = 1;                   // accesses per thread
constexpr int64_t kChunk = (int64_t)kThreads * kVec * kPerThread;  // 512
// the largest slice the layouts allow (kMaxLaunchTiles tiles) fits one
// launch: fewer than 2^32 work-items along x
static_assert((kMaxLaunchTiles * ZS_TILE + kChunk - 1) / kChunk * kThreads <
                  (int64_t(1) << 32),
              "a slice's chunks fit one launch");
constexpr int kMaxGatherWorld = ZS_GATHER_MAX_WORLD;
constexpr int64_t kMaxGridY = 65535;

struct GatherArgs {
    const uint16_t* shards[kMaxGatherWorld];
    uint16_t* out;              // out[0] is flat position lo
    int64_t lo, hi;
    int64_t q0;                 // first bucket of this launch
    int64_t B, S, S_last;       // full bucket numel and slice; last slice
    int64_t nb;                 // buckets in the layout
    int32_t W;
    int32_t r_skip;             // rows of bucket q0 before the first launched
};

// blockIdx.y runs over the (bucket, rank) rows q0 * W + r_skip, ...: the
// host launches only rows that meet [lo, hi)
__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs a)
{
    const int64_t y = (int64_t)blockIdx.y + a.r_skip;
    const int64_t q = a.q0 + y / a.W;
    const int r = (int)(y % a.W);
    const int64_t S_q = q == a.nb - 1 ? a.S_last : a.S;
    const int64_t f = q * a.B + (int64_t)r * S_q;     // slice start (flat)
    const int64_t c0 = f + (int64_t)blockIdx.x * kChunk;
    int64_t s = c0 > a.lo ? c0 : a.lo;
    int64_t e = c0 + kChunk;
    if (e > f + S_q) e = f + S_q;
    if (e > a.hi) e = a.hi;
    if (s >= e)
        return;
    // s is a multiple of 8 (lo is; chunk and slice starts are)
    const uint16_t* src = a.shards[r] + q * a.S + (s - f);
    uint16_t* dst = a.out + (s - a.lo);
    const int64_t n = e - s;
    const int64_t nvec = n / kVec;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int64_t v = (int64_t)k * kThreads + threadIdx.x;
        if (v < nvec)
            zsdev::stream_store(
                dst, (uint32_t)(n * (int64_t)sizeof(uint16_t)),
                (uint32_t)(v * (int64_t)sizeof(u32x4)),
                __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(src) + v));
    }
    // ragged end (only where hi cuts a 16-byte group)
    const int64_t t = nvec * kVec + threadIdx.x;
    if (t < n)
        dst[t] = src[t];
}

// Whole-tensor layouts: every tensor comes whole from its owner's shard
// (a broadcast from the owner in place of an all-gather of slices); the
// padded tensors partition the flat buffer, so [lo, hi) is a list of
// contiguous copies, up to kMaxSegs per launch, in the flat gather's chunks
// and copies.  Over the 34 gathers of the same forward with the
// Llama-3-8B-shaped list assigned whole (two interleaved rounds): 4.750 ms
// per forward, 84.5 % of peak, against 4.865-4.868 ms (82.5 %) for two
// plain non-temporal copies per thread in 1024-element chunks.
constexpr int kMaxSegs = 16;
// chunks per launch: kThreads work-items each stay below 2^32
constexpr int64_t kMaxLaunchChunks = ((int64_t(1) << 32) - 1) / kThreads;

struct CopySeg {
    const uint16_t* src;
    uint16_t* dst;
    int64_t n;
};

struct CopyArgs {
    CopySeg s[kMaxSegs];
    int64_t start[kMaxSegs + 1];    // prefix of the segments' chunk counts
    int count;
};

__global__ __launch_bounds__(kThreads) void copy_segments_kernel(CopyArgs a)
{
    // blockIdx.x runs over the segments' chunks, in segment order
    const int64_t t = blockIdx.x;
    int i = 0;
    while (i + 1 < a.count && a.start[i + 1] <= t)
        ++i;
    const CopySeg& sg = a.s[i];
    const int64_t c0 = (t - a.start[i]) * kChunk;
    if (c0 >= sg.n)
        return;
    const int64_t n = sg.n - c0 < kChunk ? sg.n - c0 : kChunk;
    const uint16_t* src = sg.src + c0;     // both 16-byte aligned
    uint16_t* dst = sg.dst + c0;
    const int64_t nvec = n / kVec;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int64_t v = (int64_t)k * kThreads + threadIdx.x;
        if (v < nvec)
            zsdev::stream_store(
                dst, (uint32_t)(n * (int64_t)sizeof(uint16_t)),
                (uint32_t)(v * (int64_t)sizeof(u32x4)),
                __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(src) + v));
    }
    const int64_t j = nvec * kVec + threadIdx.x;
    if (j < n)
        dst[j] = src[j];
}

int gather_tensors(const zs_layout* L, const uint16_t* const* shards,
                   int64_t lo, int64_t hi, uint16_t* out, hipStream_t s)
{
    const int64_t A = L->align_elems;
    const int32_t nt = (int32_t)L->tensor_numel.size();
    CopyArgs a;
    int cnt = 0;
    a.start[0] = 0;
    auto flush = [&]() -> int {
        if (cnt == 0) return ZS_OK;
        a.count = cnt;
        hipLaunchKernelGGL(copy_segments_kernel,
                           dim3((unsigned)a.start[cnt], 1), dim3(kThreads),
                           0, s, a);
        cnt = 0;
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return zs::fail(ZS_EDEVICE, "gather kernel: %s",
                            hipGetErrorString(err));
        return ZS_OK;
    };
    for (int32_t t = 0; t < nt; ++t) {
        const int64_t n = L->tensor_numel[t];
        if (n == 0) continue;
        const int64_t t0 = L->tensor_off[t];
        const int64_t t1 = t0 + (n + A - 1) / A * A;     // padded extent
        const int64_t x0 = t0 > lo ? t0 : lo, x1 = t1 < hi ? t1 : hi;
        if (x1 <= x0) continue;
        const int64_t nc = (x1 - x0 + kChunk - 1) / kChunk;
        if (cnt > 0 && a.start[cnt] + nc > kMaxLaunchChunks) {
            const int rc = flush();
            if (rc) return rc;
        }
        a.s[cnt].src = shards[L->owner[t]] + L->owner_shard_off[t] +
                       (x0 - t0);
        a.s[cnt].dst = out + (x0 - lo);
        a.s[cnt].n = x1 - x0;
        a.start[cnt + 1] = a.start[cnt] + nc;
        if (++cnt == kMaxSegs) {
            const int rc = flush();
            if (rc) return rc;
        }
    }
    return flush();
}

}  // namespace

extern "C" int zs_gather(const zs_layout* L, const uint16_t* const* shards,
                         int64_t flat_lo, int64_t flat_hi, uint16_t* out,
                         void* hip_stream)
{
    using zs::fail;
    zs::clear_error();
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    const int32_t W = L->world;
    if (W > kMaxGatherWorld)
        return fail(ZS_EINVAL, "world %d above %d", W, kMaxGatherWorld);
    if (flat_lo < 0 || flat_hi < flat_lo || flat_hi > L->flat_numel)
        return fail(ZS_ERANGE, "range [%lld, %lld) outside [0, %lld]",
                    (long long)flat_lo, (long long)flat_hi,
                    (long long)L->flat_numel);
    if (flat_lo % kVec)
        return fail(ZS_EALIGN, "flat_lo %lld is not a multiple of 8",
                    (long long)flat_lo);
    if (flat_hi == flat_lo)
        return ZS_OK;
    if (!shards || !out)
        return fail(ZS_EINVAL, "shards and out must be non-NULL");
    GatherArgs a;
    for (int32_t r = 0; r < W; ++r) {
        if (!shards[r])
            return fail(ZS_EINVAL, "shards[%d] is NULL", r);
        if (reinterpret_cast<uintptr_t>(shards[r]) & 15u)
            return fail(ZS_EALIGN, "shards[%d] not 16-byte aligned", r);
        a.shards[r] = shards[r];
    }
    if (reinterpret_cast<uintptr_t>(out) & 15u)
        return fail(ZS_EALIGN, "out not 16-byte aligned");
    if (L->whole_tensors)
        return gather_tensors(L, shards, flat_lo, flat_hi, out,
                              static_cast<hipStream_t>(hip_stream));
    const int64_t nb = (int64_t)L->buckets.size();
    a.out = out;
    a.lo = flat_lo;
    a.hi = flat_hi;
    a.B = L->buckets[0].numel;
    a.S = L->buckets[0].slice_numel;
    a.S_last = L->buckets.back().slice_numel;
    a.nb = nb;
    a.W = W;
    // buckets overlapping [lo, hi): every bucket before the last is full
    int64_t q_first = flat_lo / a.B, q_last = (flat_hi - 1) / a.B;
    if (q_first > nb - 1) q_first = nb - 1;
    if (q_last > nb - 1) q_last = nb - 1;
    const unsigned gx = (unsigned)((a.S + kChunk - 1) / kChunk);
    const int64_t per_launch = kMaxGridY / W;           // buckets per launch
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    // rank rows of the first and last buckets that hold lo and hi - 1; the
    // rows before the first and after the last are not launched (their
    // workgroups would find nothing to copy)
    auto slice_of = [&](int64_t q) { return q == nb - 1 ? a.S_last : a.S; };
    int64_t r_first = (flat_lo - q_first * a.B) / slice_of(q_first);
    int64_t r_last = (flat_hi - 1 - q_last * a.B) / slice_of(q_last);
    if (r_first > W - 1) r_first = W - 1;
    if (r_last > W - 1) r_last = W - 1;
    for (int64_t q = q_first; q <= q_last; q += per_launch) {
        const int64_t nq = q_last + 1 - q < per_launch ? q_last + 1 - q
                                                       : per_launch;
        a.q0 = q;
        a.r_skip = q == q_first ? (int32_t)r_first : 0;
        const int64_t r_trim = q + nq - 1 == q_last ? W - 1 - r_last : 0;
        const int64_t rows = nq * W - a.r_skip - r_trim;
        hipLaunchKernelGGL(gather_kernel, dim3(gx, (unsigned)rows),
                           dim3(kThreads), 0, s, a);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return fail(ZS_EDEVICE, "gather kernel: %s",
                        hipGetErrorString(err));
    }
    return ZS_OK;
}
