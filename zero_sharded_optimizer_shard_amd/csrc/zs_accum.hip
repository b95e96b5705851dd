// Gradient accumulation into the local gradient bucket, the step just before
// the reduce-scatter.
//
// The global batch is split into k micro-batches whose gradients are added
// up one after another, then a single optimizer step runs (podcast summary
// of "Training at thousands of GPUs", sections "Motivation" and the
// glossary; DDP-to-ZeRO blog 3.3, gradient_accumulation_steps).  Here the
// k bf16 micro-batch gradients of each element are summed in an fp32
// accumulator in micro-batch order, starting from the first, and the last
// call divides by k and rounds to bf16 (nearest even), giving the bf16
// bucket the reduce-scatter sends.  Three launches per element stream:
//   first  acc = f32(g)                    2 B read, 4 B written
//   add    acc = acc + f32(g)              6 B read, 4 B written
//   last   out = bf16((acc + f32(g)) / k)  6 B read, 2 B written (acc is
//                                          not written back)
// Elementwise and HBM-bound: one-wave workgroups over 256-element chunks,
// one four-element unit per thread, every wave instruction one contiguous
// run, non-temporal accesses.  (Measured on MI355X over the 8B flat
// gradient buffer with two micro-batches, six interleaved rounds: 64-thread
// workgroups 83.0 % of peak on average, 128-thread 81.7 %, 512-thread
// 81.1 %; at 512 threads two units per thread 76-78 %, four 71 %: many
// small workgroups keep more of this short stream in flight.)

#include <hip/hip_runtime.h>

#include <cstdint>

#include "zs_internal.h"

namespace {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 64;                      // one wave per workgroup
constexpr int kUnits = 1;                         // 4-element units/thread
constexpr int64_t kChunk = (int64_t)kThreads * kUnits * 4;   // 256

__device__ __forceinline__ float lo16(uint32_t u)
{
    return __uint_as_float(u << 16);
}

__device__ __forceinline__ float hi16(uint32_t u)
{
    return __uint_as_float(u & 0xffff0000u);
}

__device__ __forceinline__ uint32_t to_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

struct AccArgs {
    float* acc;
    const uint16_t* grad;
    uint16_t* out;
    int64_t n;                  // elements, a multiple of 4
    float fk, invk;             // k and 1/k
    int pow2;                   // k is a power of two (1/k exact)
};

template <int MODE>
__global__ __launch_bounds__(kThreads) void accum_kernel(AccArgs a)
{
    const int64_t c0 = (int64_t)blockIdx.x * kChunk;
#pragma unroll
    for (int k = 0; k < kUnits; ++k) {
        const int64_t i = c0 + 4 * ((int64_t)k * kThreads + threadIdx.x);
        if (i >= a.n)
            continue;
        const u32x2 g = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2*>(a.grad + i));
        const float gx[4] = {lo16(g.x), hi16(g.x), lo16(g.y), hi16(g.y)};
        if constexpr (MODE == ZS_ACC_FIRST) {
            __builtin_nontemporal_store(
                f32x4{gx[0], gx[1], gx[2], gx[3]},
                reinterpret_cast<f32x4*>(a.acc + i));
        } else {
            const f32x4 c = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(a.acc + i));
            const float s[4] = {c.x + gx[0], c.y + gx[1], c.z + gx[2],
                                c.w + gx[3]};
            if constexpr (MODE == ZS_ACC_ADD) {
                __builtin_nontemporal_store(
                    f32x4{s[0], s[1], s[2], s[3]},
                    reinterpret_cast<f32x4*>(a.acc + i));
            } else {
                uint32_t b[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    b[e] = to_bf16(a.pow2 ? s[e] * a.invk : s[e] / a.fk);
                __builtin_nontemporal_store(
                    u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)},
                    reinterpret_cast<u32x2*>(a.out + i));
            }
        }
    }
}

}  // namespace

extern "C" int zs_accumulate(int32_t mode, float* acc, const uint16_t* grad,
                             uint16_t* out, int64_t n, int32_t k,
                             void* hip_stream)
{
    using zs::fail;
    zs::clear_error();
    if (mode != ZS_ACC_FIRST && mode != ZS_ACC_ADD && mode != ZS_ACC_LAST)
        return fail(ZS_EINVAL, "unknown mode %d", mode);
    if (n < 0) return fail(ZS_EINVAL, "n %lld < 0", (long long)n);
    if (n % 4) return fail(ZS_EALIGN, "n %lld is not a multiple of 4",
                           (long long)n);
    if (mode == ZS_ACC_LAST && k < 2)
        return fail(ZS_EINVAL, "k %d < 2 for the last micro-batch", k);
    if (n == 0) return ZS_OK;
    if (!acc || !grad || (mode == ZS_ACC_LAST && !out))
        return fail(ZS_EINVAL, "NULL pointer");
    // acc is read and written 16 bytes at a time, grad and out 8
    if ((reinterpret_cast<uintptr_t>(acc) & 15u) ||
        ((reinterpret_cast<uintptr_t>(grad) |
          reinterpret_cast<uintptr_t>(mode == ZS_ACC_LAST ? out : grad)) &
         7u))
        return fail(ZS_EALIGN, "acc must be 16-byte aligned, grad and out "
                    "8-byte aligned");
    AccArgs a;
    a.acc = acc;
    a.grad = grad;
    a.out = out;
    a.n = n;
    a.fk = (float)k;
    a.invk = k > 0 ? (float)(1.0 / (double)k) : 0.f;
    a.pow2 = k > 0 && (k & (k - 1)) == 0;
    const int64_t blocks = n / kChunk + (n % kChunk != 0);
    // one launch: fewer than 2^32 work-items along x
    if (blocks > (((int64_t)1 << 32) - 1) / kThreads)
        return fail(ZS_ERANGE, "n %lld too large for one launch",
                    (long long)n);
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    switch (mode) {
    case ZS_ACC_FIRST:
        hipLaunchKernelGGL(accum_kernel<ZS_ACC_FIRST>, dim3((unsigned)blocks),
                           dim3(kThreads), 0, s, a);
        break;
    case ZS_ACC_ADD:
        hipLaunchKernelGGL(accum_kernel<ZS_ACC_ADD>, dim3((unsigned)blocks),
                           dim3(kThreads), 0, s, a);
        break;
    default:
        hipLaunchKernelGGL(accum_kernel<ZS_ACC_LAST>, dim3((unsigned)blocks),
                           dim3(kThreads), 0, s, a);
        break;
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return fail(ZS_EDEVICE, "accumulate kernel: %s",
                    hipGetErrorString(err));
    return ZS_OK;
}
