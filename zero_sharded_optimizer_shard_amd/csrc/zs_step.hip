// Device side of libzs: the fused shard step and the all-gather pack, with
// their host launchers and argument checks.  Written for gfx950 (CDNA4,
// wave64).
//
// The step is one pass over the rank's shard.  Per 8-element group a thread
// reads W x 16 B of bf16 gradient (one 16-byte load per source rank, in rank
// order), 3 x 32 B of fp32 state, and writes 3 x 32 B of fp32 state plus
// 16 B of bf16 parameter: 2W + 26 bytes per element, nothing else.  The
// reduced gradient lives only in registers.  No LDS, no MFMA: the work is an
// elementwise stream bounded by HBM bandwidth.
//
// Arithmetic (CS336 lecture 8 notes, "Code example: ZeRO-1": reduce-scatter
// with SUM, then the rank-local AdamW update; DDP-to-ZeRO blog 2.1: the
// gradients are averaged), one IEEE fp32 rounding per operation, no
// contraction (built with -ffp-contract=off), correctly rounded divide and
// square root (hipcc's default for fp32):
//   g   = (((G0 + G1) + G2) + ... + G_{W-1}) / W
//   m   = b1*m + (1-b1)*g
//   v   = b2*v + (1-b2)*(g*g)
//   th  = th*(1-lr*wd) - (lr/bc1) * (m / (sqrt(v)/sqrt(bc2) + eps))
//   p   = bf16 of th, round to nearest even
//
// Grid shape: blockIdx.y is the bucket, blockIdx.x the 2048-element tile of
// that bucket's slice, so no thread divides to find its bucket and the
// all-gather position of each element is one multiply-add away.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "zs_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;              // 4 waves of 64
constexpr int kGroup = 8;                  // elements per thread (16 B bf16)
constexpr int64_t kTile = kThreads * kGroup;
constexpr int64_t kMaxGridY = 65535;

struct Consts {
    float b1, b2, omb1, omb2;   // beta1, beta2, 1-beta1, 1-beta2
    float ss;                   // lr / (1 - beta1^t)
    float bc2s;                 // sqrt(1 - beta2^t)
    float dec;                  // 1 - lr*wd
    float eps;
    float fw;                   // (float)W
    float invw;                 // 1/W (exact when W is a power of two)
    int pow2;                   // W is a power of two
};

struct StepArgs {
    const uint16_t* grads;      // [W][gstride], element 0 = launch start
    int64_t gstride;
    float* master;              // shard arrays, element 0 = launch start
    float* m;
    float* v;
    uint16_t* pshard;           // nullable
    uint16_t* flat;             // flat buffer at the launch's first bucket
    int64_t S;                  // slice numel of a full bucket
    int64_t S_last;             // slice numel of bucket q_last
    int64_t B;                  // numel of a full bucket
    int32_t q_last;             // launch-relative index of the last bucket
    int32_t rank;
    int32_t W;
    Consts c;
};

__device__ __forceinline__ float bf16_lo(uint32_t u)
{
    return __uint_as_float(u << 16);
}

__device__ __forceinline__ float bf16_hi(uint32_t u)
{
    return __uint_as_float(u & 0xffff0000u);
}

// fp32 -> bf16 bits, nearest even; NaN -> quiet NaN keeping sign and the
// top payload bits.
__device__ __forceinline__ uint32_t to_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void accumulate(float (&acc)[kGroup], u32x4 x)
{
    acc[0] = acc[0] + bf16_lo(x.x);
    acc[1] = acc[1] + bf16_hi(x.x);
    acc[2] = acc[2] + bf16_lo(x.y);
    acc[3] = acc[3] + bf16_hi(x.y);
    acc[4] = acc[4] + bf16_lo(x.z);
    acc[5] = acc[5] + bf16_hi(x.z);
    acc[6] = acc[6] + bf16_lo(x.w);
    acc[7] = acc[7] + bf16_hi(x.w);
}

__device__ __forceinline__ u32x4 ld_nt(const uint16_t* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f32x4 ld_nt(const float* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

__device__ __forceinline__ void st_nt(float* p, f32x4 x)
{
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

__device__ __forceinline__ void st_nt(uint16_t* p, u32x4 x)
{
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}

// Sum of the W gradient slices for 8 consecutive elements, rank order.
// WT > 0: W known at compile time; WT == 0: runtime W.
template <int WT>
__device__ __forceinline__ void reduce_group(const uint16_t* __restrict__ g,
                                             int64_t stride, int W,
                                             float (&acc)[kGroup])
{
    const u32x4 x0 = ld_nt(g);
    acc[0] = bf16_lo(x0.x);
    acc[1] = bf16_hi(x0.x);
    acc[2] = bf16_lo(x0.y);
    acc[3] = bf16_hi(x0.y);
    acc[4] = bf16_lo(x0.z);
    acc[5] = bf16_hi(x0.z);
    acc[6] = bf16_lo(x0.w);
    acc[7] = bf16_hi(x0.w);
    if constexpr (WT > 0 && WT <= 16) {
        // all loads in flight at once, then the ordered adds
        u32x4 x[WT > 1 ? WT - 1 : 1];
#pragma unroll
        for (int s = 1; s < WT; ++s)
            x[s - 1] = ld_nt(g + (int64_t)s * stride);
#pragma unroll
        for (int s = 1; s < WT; ++s)
            accumulate(acc, x[s - 1]);
    } else {
        // batches of 16 slices keep 64 VGPRs of loads in flight
        constexpr int kBatch = 16;
        int s = 1;
#pragma unroll 1
        for (; s + kBatch <= W; s += kBatch) {
            u32x4 x[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                x[u] = ld_nt(g + (int64_t)(s + u) * stride);
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                accumulate(acc, x[u]);
        }
#pragma unroll 1
        for (; s < W; ++s)
            accumulate(acc, ld_nt(g + (int64_t)s * stride));
    }
}

template <int WT>
__global__ __launch_bounds__(kThreads) void step_kernel(StepArgs a)
{
    const int32_t q = blockIdx.y;
    const int64_t slice = (q == a.q_last) ? a.S_last : a.S;
    const int64_t j = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kGroup;
    if (j >= slice)
        return;
    const int64_t e = (int64_t)q * a.S + j;

    // fp32 state first: its loads do not depend on the gradients
    const f32x4 th0 = ld_nt(a.master + e), th1 = ld_nt(a.master + e + 4);
    const f32x4 m0 = ld_nt(a.m + e), m1 = ld_nt(a.m + e + 4);
    const f32x4 v0 = ld_nt(a.v + e), v1 = ld_nt(a.v + e + 4);

    float g[kGroup];
    reduce_group<WT>(a.grads + e, a.gstride, WT > 0 ? WT : a.W, g);

    const Consts c = a.c;
    const bool pow2 = WT > 0 ? ((WT & (WT - 1)) == 0) : (c.pow2 != 0);
#pragma unroll
    for (int k = 0; k < kGroup; ++k)
        g[k] = pow2 ? g[k] * c.invw : g[k] / c.fw;

    float th[kGroup] = {th0.x, th0.y, th0.z, th0.w, th1.x, th1.y, th1.z, th1.w};
    float mm[kGroup] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    float vv[kGroup] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t pb[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
        const float mi = (c.b1 * mm[k]) + (c.omb1 * g[k]);
        const float g2 = g[k] * g[k];
        const float vi = (c.b2 * vv[k]) + (c.omb2 * g2);
        const float root = sqrtf(vi);
        const float den = (root / c.bc2s) + c.eps;
        const float upd = mi / den;
        const float t = (th[k] * c.dec) - (c.ss * upd);
        mm[k] = mi;
        vv[k] = vi;
        th[k] = t;
        pb[k] = to_bf16(t);
    }

    st_nt(a.master + e, f32x4{th[0], th[1], th[2], th[3]});
    st_nt(a.master + e + 4, f32x4{th[4], th[5], th[6], th[7]});
    st_nt(a.m + e, f32x4{mm[0], mm[1], mm[2], mm[3]});
    st_nt(a.m + e + 4, f32x4{mm[4], mm[5], mm[6], mm[7]});
    st_nt(a.v + e, f32x4{vv[0], vv[1], vv[2], vv[3]});
    st_nt(a.v + e + 4, f32x4{vv[4], vv[5], vv[6], vv[7]});
    const u32x4 p = {pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16),
                     pb[4] | (pb[5] << 16), pb[6] | (pb[7] << 16)};
    if (a.pshard)
        st_nt(a.pshard + e, p);
    if (a.flat)
        st_nt(a.flat + (int64_t)q * a.B + (int64_t)a.rank * slice + j, p);
}

// ---- pack: shard -> flat all-gather buffer ---------------------------------

struct PackFlatArgs {
    const uint16_t* shard;      // at the launch's first bucket
    uint16_t* flat;             // at the launch's first bucket
    int64_t S, S_last, B;
    int32_t q_last;
    int32_t rank;
};

__global__ __launch_bounds__(kThreads) void pack_flat_kernel(PackFlatArgs a)
{
    const int32_t q = blockIdx.y;
    const int64_t slice = (q == a.q_last) ? a.S_last : a.S;
    const int64_t j = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kGroup;
    if (j >= slice)
        return;
    const u32x4 x = ld_nt(a.shard + (int64_t)q * a.S + j);
    st_nt(a.flat + (int64_t)q * a.B + (int64_t)a.rank * slice + j, x);
}

// ---- pack: shard -> per-tensor storage through the chunk table -------------

__global__ __launch_bounds__(kThreads) void pack_chunks_kernel(
    const uint16_t* __restrict__ shard, const zs_chunk* __restrict__ chunks,
    int32_t c0, uint16_t* const* __restrict__ tensors)
{
    // one chunk per blockIdx.y; the chunk record and tensor pointer are the
    // same for the whole workgroup
    const zs_chunk ch = chunks[c0 + (int32_t)blockIdx.y];
    uint16_t* dst = tensors[ch.tensor_id] + ch.tensor_off;
    const uint16_t* src = shard + ch.shard_off;
    const int64_t n = ch.numel;
    const int64_t step = (int64_t)gridDim.x * kTile;
    const bool vec = ((reinterpret_cast<uintptr_t>(dst) |
                       reinterpret_cast<uintptr_t>(src)) & 15u) == 0;
    for (int64_t j = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kGroup;
         j < n; j += step) {
        if (vec && j + kGroup <= n) {
            st_nt(dst + j, ld_nt(src + j));
        } else {
            const int64_t end = j + kGroup < n ? j + kGroup : n;
            for (int64_t k = j; k < end; ++k)
                dst[k] = src[k];
        }
    }
}

// ---- host side ---------------------------------------------------------------

Consts make_consts(const zs_adamw& hp, int64_t t, int32_t W)
{
    // double precision, each constant rounded to fp32 once
    const double b1 = hp.beta1, b2 = hp.beta2, lr = hp.lr, wd = hp.weight_decay;
    const double bc1 = 1.0 - std::pow(b1, (double)t);
    const double bc2 = 1.0 - std::pow(b2, (double)t);
    Consts c;
    c.b1 = (float)b1;
    c.b2 = (float)b2;
    c.omb1 = (float)(1.0 - b1);
    c.omb2 = (float)(1.0 - b2);
    c.ss = (float)(lr / bc1);
    c.bc2s = (float)std::sqrt(bc2);
    c.dec = (float)(1.0 - lr * wd);
    c.eps = hp.eps;
    c.fw = (float)W;
    c.pow2 = (W & (W - 1)) == 0;
    c.invw = (float)(1.0 / (double)W);
    return c;
}

bool aligned16(const void* p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

int check_launch(const char* what)
{
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return zs::fail(ZS_EDEVICE, "%s: %s", what, hipGetErrorString(err));
    return ZS_OK;
}

template <int WT>
void launch_step_w(const StepArgs& a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL(step_kernel<WT>, grid, dim3(kThreads), 0, s, a);
}

void launch_step(const StepArgs& a, dim3 grid, hipStream_t s)
{
    switch (a.W) {
    case 1: launch_step_w<1>(a, grid, s); break;
    case 2: launch_step_w<2>(a, grid, s); break;
    case 4: launch_step_w<4>(a, grid, s); break;
    case 8: launch_step_w<8>(a, grid, s); break;
    case 16: launch_step_w<16>(a, grid, s); break;
    case 32: launch_step_w<32>(a, grid, s); break;
    case 64: launch_step_w<64>(a, grid, s); break;
    default: launch_step_w<0>(a, grid, s); break;
    }
}

// Checks shared by zs_step and zs_bucket_step.  `n` is the number of shard
// elements the call covers; `len` the gradient elements per slice it reads.
int check_step_args(const zs_layout* L, const uint16_t* grads,
                    int64_t grad_stride, int64_t len, const float* master,
                    const float* m, const float* v, const uint16_t* pshard,
                    const uint16_t* flat, const zs_adamw* hp, int64_t step)
{
    using zs::fail;
    if (!hp) return fail(ZS_EINVAL, "hp is NULL");
    if (step < 1) return fail(ZS_EINVAL, "step %lld < 1", (long long)step);
    if (!grads || !master || !m || !v)
        return fail(ZS_EINVAL, "grads, master, m and v must be non-NULL");
    if (!pshard && !flat)
        return fail(ZS_EINVAL, "need param_shard or full_flat");
    if (!aligned16(grads) || !aligned16(master) || !aligned16(m) ||
        !aligned16(v) || (pshard && !aligned16(pshard)) ||
        (flat && !aligned16(flat)))
        return fail(ZS_EALIGN, "device pointers must be 16-byte aligned");
    if (grad_stride % kGroup)
        return fail(ZS_EALIGN, "grad_stride %lld is not a multiple of 8",
                    (long long)grad_stride);
    if (grad_stride < len)
        return fail(ZS_ERANGE, "grad_stride %lld < %lld elements per slice",
                    (long long)grad_stride, (long long)len);
    if (grad_stride > INT64_MAX / 2 / L->world)
        return fail(ZS_ERANGE, "W * grad_stride overflows");
    return ZS_OK;
}

}  // namespace

extern "C" int zs_step(const zs_layout* L, const uint16_t* grads,
                       int64_t grad_stride, float* master, float* m, float* v,
                       uint16_t* param_shard, uint16_t* full_flat,
                       const zs_adamw* hp, int64_t step, void* hip_stream)
{
    zs::clear_error();
    if (!L) return zs::fail(ZS_EINVAL, "layout is NULL");
    if (!hp) return zs::fail(ZS_EINVAL, "hp is NULL");
    if (step < 1) return zs::fail(ZS_EINVAL, "step %lld < 1", (long long)step);
    if (L->shard_numel == 0)
        return ZS_OK;
    int rc = check_step_args(L, grads, grad_stride, L->shard_numel, master, m,
                             v, param_shard, full_flat, hp, step);
    if (rc) return rc;

    const int64_t nb = (int64_t)L->buckets.size();
    const int32_t W = L->world;
    StepArgs a;
    a.gstride = grad_stride;
    a.S = nb > 1 ? L->bucket_elems / W : L->buckets[0].slice_numel;
    a.S_last = L->buckets.back().slice_numel;
    a.B = nb > 1 ? L->bucket_elems : L->buckets[0].numel;
    a.rank = L->rank;
    a.W = W;
    a.c = make_consts(*hp, step, W);
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const unsigned gx = (unsigned)((a.S + kTile - 1) / kTile);
    for (int64_t y0 = 0; y0 < nb; y0 += kMaxGridY) {
        const int64_t ny = nb - y0 < kMaxGridY ? nb - y0 : kMaxGridY;
        const int64_t e0 = L->buckets[y0].shard_off;   // == y0 * S
        a.grads = grads + e0;
        a.master = master + e0;
        a.m = m + e0;
        a.v = v + e0;
        a.pshard = param_shard ? param_shard + e0 : nullptr;
        a.flat = full_flat ? full_flat + L->buckets[y0].flat_off : nullptr;
        a.q_last = (nb - 1 - y0 < ny) ? (int32_t)(nb - 1 - y0) : -1;
        launch_step(a, dim3(gx, (unsigned)ny), s);
        rc = check_launch("step kernel");
        if (rc) return rc;
    }
    return ZS_OK;
}

extern "C" int zs_bucket_step(const zs_layout* L, int32_t bucket_id,
                              const uint16_t* grads, int64_t grad_stride,
                              float* master, float* m, float* v,
                              uint16_t* param_shard, uint16_t* full_flat,
                              const zs_adamw* hp, int64_t step,
                              void* hip_stream)
{
    zs::clear_error();
    if (!L) return zs::fail(ZS_EINVAL, "layout is NULL");
    if (bucket_id < 0 || bucket_id >= (int32_t)L->buckets.size())
        return zs::fail(ZS_ERANGE, "bucket_id %d outside [0, %d)", bucket_id,
                        (int)L->buckets.size());
    const zs_bucket& b = L->buckets[bucket_id];
    int rc = check_step_args(L, grads, grad_stride, b.slice_numel, master, m,
                             v, param_shard, full_flat, hp, step);
    if (rc) return rc;
    StepArgs a;
    a.grads = grads;
    a.gstride = grad_stride;
    a.master = master + b.shard_off;
    a.m = m + b.shard_off;
    a.v = v + b.shard_off;
    a.pshard = param_shard ? param_shard + b.shard_off : nullptr;
    a.flat = full_flat ? full_flat + b.flat_off : nullptr;
    a.S = b.slice_numel;
    a.S_last = b.slice_numel;
    a.B = b.numel;
    a.q_last = 0;
    a.rank = L->rank;
    a.W = L->world;
    a.c = make_consts(*hp, step, L->world);
    const unsigned gx = (unsigned)((b.slice_numel + kTile - 1) / kTile);
    launch_step(a, dim3(gx, 1), static_cast<hipStream_t>(hip_stream));
    return check_launch("bucket step kernel");
}

extern "C" int zs_pack(const zs_layout* L, const uint16_t* param_shard,
                       uint16_t* full_flat, const zs_chunk* dev_chunks,
                       int32_t n_chunks, uint16_t* const* dev_tensor_ptrs,
                       void* hip_stream)
{
    using zs::fail;
    zs::clear_error();
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    const bool chunk_mode = dev_chunks || dev_tensor_ptrs;
    if (chunk_mode && (!dev_chunks || !dev_tensor_ptrs))
        return fail(ZS_EINVAL, "dev_chunks and dev_tensor_ptrs go together");
    if (chunk_mode && n_chunks != (int32_t)L->chunks.size())
        return fail(ZS_EINVAL, "n_chunks %d != layout's %d", n_chunks,
                    (int)L->chunks.size());
    if (!full_flat && !chunk_mode)
        return fail(ZS_EINVAL, "no destination: full_flat or chunks");
    if (L->shard_numel == 0)
        return ZS_OK;
    if (!param_shard) return fail(ZS_EINVAL, "param_shard is NULL");
    if (!aligned16(param_shard) || (full_flat && !aligned16(full_flat)))
        return fail(ZS_EALIGN, "param_shard/full_flat not 16-byte aligned");
    if (chunk_mode && (!aligned16(dev_chunks) ||
                       (reinterpret_cast<uintptr_t>(dev_tensor_ptrs) & 7u)))
        return fail(ZS_EALIGN, "chunk table or pointer array misaligned");
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);

    if (full_flat) {
        const int64_t nb = (int64_t)L->buckets.size();
        PackFlatArgs a;
        a.S = nb > 1 ? L->bucket_elems / L->world : L->buckets[0].slice_numel;
        a.S_last = L->buckets.back().slice_numel;
        a.B = nb > 1 ? L->bucket_elems : L->buckets[0].numel;
        a.rank = L->rank;
        const unsigned gx = (unsigned)((a.S + kTile - 1) / kTile);
        for (int64_t y0 = 0; y0 < nb; y0 += kMaxGridY) {
            const int64_t ny = nb - y0 < kMaxGridY ? nb - y0 : kMaxGridY;
            a.shard = param_shard + L->buckets[y0].shard_off;
            a.flat = full_flat + L->buckets[y0].flat_off;
            a.q_last = (nb - 1 - y0 < ny) ? (int32_t)(nb - 1 - y0) : -1;
            hipLaunchKernelGGL(pack_flat_kernel, dim3(gx, (unsigned)ny),
                               dim3(kThreads), 0, s, a);
            const int rc = check_launch("pack flat kernel");
            if (rc) return rc;
        }
    }
    if (chunk_mode && n_chunks > 0) {
        int64_t longest = 0;
        for (const zs_chunk& c : L->chunks)
            longest = c.numel > longest ? c.numel : longest;
        int64_t gx = (longest + kTile - 1) / kTile;
        if (gx > 256) gx = 256;
        for (int32_t c0 = 0; c0 < n_chunks; c0 += (int32_t)kMaxGridY) {
            const int32_t ny = n_chunks - c0 < kMaxGridY ? n_chunks - c0
                                                         : (int32_t)kMaxGridY;
            hipLaunchKernelGGL(pack_chunks_kernel,
                               dim3((unsigned)gx, (unsigned)ny),
                               dim3(kThreads), 0, s, param_shard, dev_chunks,
                               c0, dev_tensor_ptrs);
            const int rc = check_launch("pack chunks kernel");
            if (rc) return rc;
        }
    }
    return ZS_OK;
}
