// Device side of libzs: the fused shard step, the all-gather pack, the
// layout conversions, and their host launchers.  Written for gfx950 (CDNA4,
// wave64).
//
// The step is one pass over the rank's shard.  Per element it reads W x 2 B
// of bf16 gradient, 12 B of fp32 state (master, m, v) and writes the 12 B of
// state back plus 2 B of bf16 parameter: 2W + 26 bytes, nothing else.  The
// reduced gradient lives only in registers.  No LDS and no MFMA: the work
// is an elementwise stream bounded by HBM bandwidth.
//
// Arithmetic (CS336 lecture 8 notes, "Code example: ZeRO-1": reduce-scatter
// with SUM, then the rank-local AdamW update; DDP-to-ZeRO blog 2.1: the
// gradients are averaged), one IEEE fp32 rounding per operation, no
// contraction (built with -ffp-contract=off), correctly rounded divide and
// square root:
//   g   = (((G0 + G1) + G2) + ... + G_{W-1}) / W
//   m   = b1*m + (1-b1)*g
//   v   = b2*v + (1-b2)*(g*g)
//   th  = th*(1-lr*wd) - (lr/bc1) * (m / (sqrt(v)/sqrt(bc2) + eps))
//   p   = bf16 of th, round to nearest even
//
// Work decomposition.  The shard is cut into tiles of ZS_TILE = 8192
// elements of one bucket's slice.  At a compiled W a tile is stepped by 32
// one-wave workgroups, one 4-element unit per thread, each thread loading
// its unit of all W gradient slices at once, and only a few of these
// workgroups may share a CU (the launch reserves LDS the kernel does not
// use); runtime W, plain slice rows at W >= 32 and large bucket groups take
// other shapes (listed with the launchers below).  Either way every load or
// store instruction of a wave covers one contiguous run (1 KiB of fp32,
// 512 B of bf16) and a tile's rows are swept in bursts.  With the tiled
// state the three 32 KiB rows of a tile are adjacent, and with tiled
// gradients so are the W 16 KiB slice rows; measured on MI355X, that lifts
// this 2:1 read/write stream from about 5.4 to about 6.4 TB/s with the
// earlier 512-thread shapes.  All loads of a unit are issued before its
// arithmetic (all W slices at a compiled W, batches of 4 or 8 otherwise),
// and every access is non-temporal: nothing is reused.  The step's stores
// also carry system scope (sc0 sc1 nt), so the L2 streams them on to HBM
// instead of holding them as dirty lines: measured on MI355X, 82.0-82.2 %
// of peak against 80.4 % with plain non-temporal stores on the 8B-shaped
// W = 8 shard (512-thread workgroups then).  The pack and the layout
// conversions, plain copies, store the same way; their workgroup shapes,
// measured one by one, are given with each kernel below.
//
// Grid of the whole-shard step: blockIdx.y = bucket, blockIdx.x = tile
// (times the workgroups per tile) of that bucket's slice, so no thread
// divides to find its bucket, and the all-gather position of each element
// is one multiply-add away.  Bucket groups (the streaming step, and the
// whole-tensor layout's owned tensors) run a 1-D grid over their members'
// tiles, the member found from a prefix table in the kernel arguments.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>
#include <type_traits>
#include <vector>

#include "zs_device.h"
#include "zs_internal.h"

namespace {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int64_t kTile = ZS_TILE;
// Each kernel states its own workgroup shape beside it: the step's work
// shapes (Shape below), kStWave / kStWide / kGtThreads / kPackNT for the
// layout conversions and the flat pack, kPackThreads for the per-tensor
// pack.
constexpr int64_t kMaxGridY = 65535;

// Work shape of the step kernels: NT threads per workgroup, U 4-element
// units per thread, gradient slices loaded NB at a time; P = ZS_TILE /
// (4 NT U) workgroups share one tile (consecutive blockIdx.x).
template <int NT_, int U_, int NB_>
struct Shape {
    static constexpr int NT = NT_;
    static constexpr int U = U_;
    static constexpr int NB = NB_;
    static constexpr int P = (int)(kTile / (4 * NT_ * U_));
    static_assert((int64_t)P * 4 * NT_ * U_ == kTile, "shape must tile");
};

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

// Where one launch's tiles sit.  Buckets are launch-relative: bucket q
// (q < q_last, or every q when q_last < 0) is a full bucket with slice S,
// numel B and TPB tiles; bucket q_last has slice S_last <= S.
struct Geom {
    int64_t S, S_last, B, TPB;
    int32_t q_last, rank;
};

struct TileRef {
    int64_t tile;       // launch-relative tile index
    int64_t e0;         // launch-relative shard element of the tile start
    int64_t nvalid;     // elements of the tile inside the slice
    int64_t fpos;       // launch-relative flat position of the tile start
};

// P workgroups per tile (blockIdx.x = tile * P + part); P = 1 for the
// conversions and the pack.
template <int P = 1>
__device__ __forceinline__ bool tile_of(const Geom& g, TileRef& r)
{
    const int32_t q = blockIdx.y;
    const int64_t slice = (q == g.q_last) ? g.S_last : g.S;
    const int64_t x = blockIdx.x / P;
    const int64_t j0 = x * kTile;
    if (j0 >= slice)
        return false;
    r.tile = (int64_t)q * g.TPB + x;
    r.e0 = (int64_t)q * g.S + j0;
    r.nvalid = slice - j0 < kTile ? slice - j0 : kTile;
    r.fpos = (int64_t)q * g.B + (int64_t)g.rank * slice + j0;
    return true;
}

// The same for an explicit tile x of bucket blockIdx.y (the gradient tiling
// conversion, whose workgroups are not in tile-major order).
__device__ __forceinline__ bool tile_at(const Geom& g, int64_t x, TileRef& r)
{
    const int32_t q = blockIdx.y;
    const int64_t slice = (q == g.q_last) ? g.S_last : g.S;
    const int64_t j0 = x * kTile;
    if (j0 >= slice)
        return false;
    r.tile = (int64_t)q * g.TPB + x;
    r.e0 = (int64_t)q * g.S + j0;
    r.nvalid = slice - j0 < kTile ? slice - j0 : kTile;
    r.fpos = (int64_t)q * g.B + (int64_t)g.rank * slice + j0;
    return true;
}

// element offset of unit k of this thread inside its tile, for a workgroup
// of NT threads that is part `blockIdx.x % P` of P on the tile
template <int P, int NT>
__device__ __forceinline__ int unit_off(int k)
{
    const int part = (int)(blockIdx.x % P);
    return part * (int)(kTile / P) + 4 * (k * NT + (int)threadIdx.x);
}

// Tile locators of the layout conversions and the flat pack.  GeomLoc:
// the regular buckets of the flat mode (blockIdx.y = bucket); SegLoc: up to
// kMaxMembers explicit segments (a 1-D grid over their tiles), e.g. the
// owned tensors of the whole-tensor mode; positions are then absolute.
//
// kMaxGroup: buckets per zs_buckets_step call (the public limit).
// kMaxMembers: members per launch, held in the kernel arguments; whole-shard
// steps of the whole-tensor mode pack up to this many owned tensors into one
// launch (the Llama-3-8B-shaped list gives a rank 22 of them at W = 8).
constexpr int kMaxGroup = ZS_MAX_GROUP;
constexpr int kMaxMembers = 32;
static_assert(kMaxMembers >= kMaxGroup, "a call's group fits one launch");

struct Seg {
    int64_t shard_off, tile_off, fpos, slice;
};

struct GeomLoc {
    Geom g;
    // P workgroups per tile (blockIdx.x = tile * P + part)
    template <int P>
    __device__ bool at(TileRef& r) const { return tile_of<P>(g, r); }
    // tile x of the launch's row of tiles
    __device__ bool at_tile(int64_t x, TileRef& r) const
    {
        return tile_at(g, x, r);
    }
};

// Member i of a group launch owns the launch's tiles [start[i], start[i+1])
// (blockIdx.x runs over the group's tiles, start[0] = 0); a binary search
// over the prefix table, wave-uniform scalar loads of the kernel arguments,
// finds it: the largest i < count with start[i] <= t.
__device__ __forceinline__ int member_of(const int64_t* start, int count,
                                         int64_t t)
{
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

struct SegLoc {
    Seg s[kMaxMembers];
    int64_t start[kMaxMembers + 1];
    int count;
    template <int P>
    __device__ bool at(TileRef& r) const
    {
        const int64_t t = blockIdx.x / P;
        const int i = member_of(start, count, t);
        const Seg& sg = s[i];
        const int64_t x = t - start[i];
        const int64_t j0 = x * kTile;
        if (j0 >= sg.slice)
            return false;
        r.tile = sg.tile_off + x;
        r.e0 = sg.shard_off + j0;
        r.nvalid = sg.slice - j0 < kTile ? sg.slice - j0 : kTile;
        r.fpos = sg.fpos + j0;
        return true;
    }
    // the same for an explicit tile t of the launch's members
    __device__ bool at_tile(int64_t t, TileRef& r) const
    {
        const int i = member_of(start, count, t);
        const Seg& sg = s[i];
        const int64_t x = t - start[i];
        const int64_t j0 = x * kTile;
        if (j0 >= sg.slice)
            return false;
        r.tile = sg.tile_off + x;
        r.e0 = sg.shard_off + j0;
        r.nvalid = sg.slice - j0 < kTile ? sg.slice - j0 : kTile;
        r.fpos = sg.fpos + j0;
        return true;
    }
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

__device__ __forceinline__ u32x2 ld2(const uint16_t* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

__device__ __forceinline__ f32x4 ld4(const float* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

// Stores of the step: element jj of a tile row at `row` (wave-uniform),
// streamed on to HBM (zsdev::stream_store); the region is the row's ZS_TILE
// elements, so the hardware drops any store outside the row.
__device__ __forceinline__ void st2_out(uint16_t* row, int jj, u32x2 x)
{
    zsdev::stream_store(row, (uint32_t)(kTile * sizeof(uint16_t)),
                        (uint32_t)jj * (uint32_t)sizeof(uint16_t), x);
}

__device__ __forceinline__ void st4_out(float* row, int jj, f32x4 x)
{
    zsdev::stream_store(row, (uint32_t)(kTile * sizeof(float)),
                        (uint32_t)jj * (uint32_t)sizeof(float), x);
}

struct StepArgs {
    const uint16_t* grads;      // launch base (see zs_step)
    int64_t gstride;            // slices layout: elements between slices
    float* state;               // tiled state at the launch's first tile
    uint16_t* pshard;           // nullable, at the launch's first element
    uint16_t* flat;             // nullable, at the launch's first bucket
    Geom g;
    int32_t W;
    Consts c;
};

// Slices s0 .. s0+n-1 (n <= NB) of every unit: all loads first, then the
// adds in rank order.  Slice 0 initialises the sum, so the sign of a zero
// sum is that of the first addend, as in a left-to-right sum.
template <int NB, class SH>
__device__ __forceinline__ void reduce_batch(const uint16_t* __restrict__ g0,
                                             int64_t gs, int s0, int n,
                                             bool full, int64_t nvalid,
                                             float (&acc)[SH::U][4])
{
    constexpr int U = SH::U;
    u32x2 x[U][NB];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int jj = unit_off<SH::P, SH::NT>(k);
        if (full || jj < nvalid) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                if (i < n)
                    x[k][i] = ld2(g0 + (int64_t)(s0 + i) * gs + jj);
        }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int jj = unit_off<SH::P, SH::NT>(k);
        if (!(full || jj < nvalid))
            continue;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (i >= n)
                continue;
            const u32x2 u = x[k][i];
            if (s0 + i == 0) {
                acc[k][0] = bf16_lo(u.x);
                acc[k][1] = bf16_hi(u.x);
                acc[k][2] = bf16_lo(u.y);
                acc[k][3] = bf16_hi(u.y);
            } else {
                acc[k][0] = acc[k][0] + bf16_lo(u.x);
                acc[k][1] = acc[k][1] + bf16_hi(u.x);
                acc[k][2] = acc[k][2] + bf16_lo(u.y);
                acc[k][3] = acc[k][3] + bf16_hi(u.y);
            }
        }
    }
}

// WT > 0: W known at compile time; WT == 0: runtime W.
template <int WT, class SH>
__device__ __forceinline__ void reduce(const uint16_t* __restrict__ g0,
                                       int64_t gs, int W, bool full,
                                       int64_t nvalid,
                                       float (&acc)[SH::U][4])
{
    constexpr int NB = SH::NB;
    if constexpr (WT > 0 && WT <= NB) {
        reduce_batch<WT, SH>(g0, gs, 0, WT, full, nvalid, acc);
    } else if constexpr (WT > 0) {
        static_assert(WT % NB == 0, "compiled W must be a multiple of the "
                      "batch");
#pragma unroll
        for (int s0 = 0; s0 < WT; s0 += NB)
            reduce_batch<NB, SH>(g0, gs, s0, NB, full, nvalid, acc);
    } else {
#pragma unroll 1
        for (int s0 = 0; s0 < W; s0 += NB) {
            const int n = W - s0 < NB ? W - s0 : NB;
            reduce_batch<NB, SH>(g0, gs, s0, n, full, nvalid, acc);
        }
    }
}

// Where a tile's fp32 state sits.  TileRows: one tile of the tiled state,
// rows master, m, v (or m, v for the pure-bf16 step) ZS_TILE floats apart.
// PlainRows: the tile's stretch of three plain arrays.
template <bool PURE>
struct TileRows {
    float* st;
    static constexpr int kM = PURE ? 0 : 1;     // row of m; v follows
    __device__ float* th() const { return st; }
    __device__ float* m() const { return st + kM * kTile; }
    __device__ float* v() const { return st + (kM + 1) * kTile; }
};

struct PlainRows {
    float* th_;
    float* m_;
    float* v_;
    __device__ float* th() const { return th_; }
    __device__ float* m() const { return m_; }
    __device__ float* v() const { return v_; }
};

// One tile of the step, with every pointer already at the tile: g0 the
// first gradient value of slice 0 (tiled: the tile's W rows, gs = ZS_TILE;
// slices: gs = the slice stride), rows the tile's fp32 state (TileRows or
// PlainRows), ps / fl the tile's first bf16 output (each nullable).  This
// workgroup is part blockIdx.x % P of SH::P on the tile.
//
// PURE (the pure-bf16 variant, no fp32 master): the state holds only m and
// v, and the parameter is the bf16 value itself, read from and written back
// to ps if it is given, else fl.
template <int WT, class SH, bool PURE = false, class Rows>
__device__ __forceinline__ void step_tile(const uint16_t* __restrict__ g0,
                                          int64_t gs, const Rows rows,
                                          uint16_t* __restrict__ ps,
                                          uint16_t* __restrict__ fl,
                                          int64_t nvalid, int W,
                                          const Consts& c)
{
    constexpr int U = SH::U;
    const bool full = nvalid == kTile;

    // state first: its loads do not depend on the gradients
    uint16_t* const pp = PURE ? (ps ? ps : fl) : nullptr;
    f32x4 th[U], mm[U], vv[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int jj = unit_off<SH::P, SH::NT>(k);
        if (full || jj < nvalid) {
            if constexpr (PURE) {
                const u32x2 q = ld2(pp + jj);
                th[k] = f32x4{bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y),
                              bf16_hi(q.y)};
            } else {
                th[k] = ld4(rows.th() + jj);
            }
            mm[k] = ld4(rows.m() + jj);
            vv[k] = ld4(rows.v() + jj);
        }
    }

    float g[U][4];
    reduce<WT, SH>(g0, gs, W, full, nvalid, g);

    const bool pow2 = WT > 0 ? ((WT & (WT - 1)) == 0) : (c.pow2 != 0);
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int jj = unit_off<SH::P, SH::NT>(k);
        if (!(full || jj < nvalid))
            continue;
        float t4[4] = {th[k].x, th[k].y, th[k].z, th[k].w};
        float m4[4] = {mm[k].x, mm[k].y, mm[k].z, mm[k].w};
        float v4[4] = {vv[k].x, vv[k].y, vv[k].z, vv[k].w};
        uint32_t pb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float gi = pow2 ? g[k][i] * c.invw : g[k][i] / c.fw;
            const float mi = (c.b1 * m4[i]) + (c.omb1 * gi);
            const float g2 = gi * gi;
            const float vi = (c.b2 * v4[i]) + (c.omb2 * g2);
            const float root = sqrtf(vi);
            const float den = (root / c.bc2s) + c.eps;
            const float upd = mi / den;
            const float t = (t4[i] * c.dec) - (c.ss * upd);
            m4[i] = mi;
            v4[i] = vi;
            t4[i] = t;
            pb[i] = to_bf16(t);
        }
        if constexpr (!PURE)
            st4_out(rows.th(), jj, f32x4{t4[0], t4[1], t4[2], t4[3]});
        st4_out(rows.m(), jj, f32x4{m4[0], m4[1], m4[2], m4[3]});
        st4_out(rows.v(), jj, f32x4{v4[0], v4[1], v4[2], v4[3]});
        const u32x2 p = {pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)};
        if constexpr (PURE) {
            st2_out(pp, jj, p);
        } else {
            if (ps)
                st2_out(ps, jj, p);
            if (fl)
                st2_out(fl, jj, p);
        }
    }
}

// Whole-shard step: blockIdx.y = bucket, blockIdx.x = tile * P + part.
template <int WT, bool TILED, class SH, bool PURE>
__global__ __launch_bounds__(SH::NT) void step_kernel(StepArgs a)
{
    TileRef r;
    if (!tile_of<SH::P>(a.g, r))
        return;
    const int W = WT > 0 ? WT : a.W;
    const uint16_t* g0 = TILED ? a.grads + r.tile * (int64_t)W * kTile
                               : a.grads + r.e0;
    step_tile<WT, SH, PURE>(g0, TILED ? kTile : a.gstride,
                      TileRows<PURE>{a.state + r.tile * ((PURE ? 2 : 3) *
                                                         kTile)},
                      a.pshard ? a.pshard + r.e0 : nullptr,
                      a.flat ? a.flat + r.fpos : nullptr, r.nvalid, W, a.c);
}

// The whole-shard step on three plain [shard_numel] fp32 arrays (master, m,
// v) instead of the tiled state: the tile's stretch of each array takes the
// place of its state row.
struct PlainArgs {
    const uint16_t* grads;      // launch base (see zs_step)
    int64_t gstride;            // slices layout: elements between slices
    float* master;              // plain arrays at the launch's first element
    float* m;
    float* v;
    uint16_t* pshard;           // nullable, at the launch's first element
    uint16_t* flat;             // nullable, at the launch's first bucket
    Geom g;
    int32_t W;
    Consts c;
};

template <int WT, bool TILED, class SH>
__global__ __launch_bounds__(SH::NT) void step_plain_kernel(PlainArgs a)
{
    TileRef r;
    if (!tile_of<SH::P>(a.g, r))
        return;
    const int W = WT > 0 ? WT : a.W;
    const uint16_t* g0 = TILED ? a.grads + r.tile * (int64_t)W * kTile
                               : a.grads + r.e0;
    step_tile<WT, SH, false>(g0, TILED ? kTile : a.gstride,
                             PlainRows{a.master + r.e0, a.m + r.e0,
                                       a.v + r.e0},
                             a.pshard ? a.pshard + r.e0 : nullptr,
                             a.flat ? a.flat + r.fpos : nullptr, r.nvalid, W,
                             a.c);
}

// A group of buckets, each from its own staging buffer: blockIdx.x runs
// over the members' tiles (times P), in member order.

struct GroupMember {
    const uint16_t* grads;      // this bucket's staging
    float* state;               // state at the bucket's first tile
    uint16_t* pshard;           // nullable, at the bucket's first element
    uint16_t* flat;             // nullable, at this rank's slice of it
                                // (pure: exactly one of pshard, flat)
    int64_t slice;              // slice_numel
};

struct GroupArgs {
    GroupMember mb[kMaxMembers];
    int64_t start[kMaxMembers + 1]; // prefix of the members' tile counts
    int32_t count;
    int64_t gstride;
    int32_t W;
    Consts c;
};
// kernel arguments are limited to 4 KiB
static_assert(sizeof(GroupArgs) <= 4096 && sizeof(SegLoc) <= 2048,
              "group tables must fit the kernel arguments");

template <int WT, bool TILED, class SH, bool PURE>
__global__ __launch_bounds__(SH::NT) void group_step_kernel(GroupArgs a)
{
    // blockIdx.x = (group tile) * P + part; the group tile belongs to one
    // member, as its tile x
    const int64_t t = blockIdx.x / SH::P;
    const int i = member_of(a.start, a.count, t);
    const GroupMember& mb = a.mb[i];
    const int64_t x = t - a.start[i];
    const int64_t j0 = x * kTile;
    if (j0 >= mb.slice)
        return;
    const int W = WT > 0 ? WT : a.W;
    const int64_t nvalid = mb.slice - j0 < kTile ? mb.slice - j0 : kTile;
    const uint16_t* g0 = TILED ? mb.grads + x * (int64_t)W * kTile
                               : mb.grads + j0;
    step_tile<WT, SH, PURE>(g0, TILED ? kTile : a.gstride,
                      TileRows<PURE>{mb.state + x * (PURE ? 2 : 3) * kTile},
                      mb.pshard ? mb.pshard + j0 : nullptr,
                      mb.flat ? mb.flat + j0 : nullptr, nvalid, W, a.c);
}

// ---- layout conversions ------------------------------------------------------

// Up to three plain fp32 arrays, one per row of a tiled state of ROWS rows
// (3: master, m, v; 2: m, v).
struct Rows {
    const float* in[3];         // pack: sources, NULL = zeros
    float* out[3];              // unpack: destinations, NULL = skipped
};

// One state row of one tile per 8192 / (4 NT) workgroups of NT threads, one
// 16-byte group per thread, the stores streamed on to HBM with system scope.
// Each conversion runs in the order of its output, so that consecutive
// workgroups write consecutive memory: the unpack with the row on the
// grid's z axis (the dispatcher advances z last, so the workgroups in
// flight write one plain array in order), the pack with blockIdx.x =
// ((x - x0) * ROWS + row) * P + part for tile x (each launch covers at most
// kOrderedLaunchTiles tiles, x0 its first).  Measured on MI355X over the
// 8B-shaped W = 8 shard's state, interleaved rounds:
//  - unpack (24 B per element): one-wave workgroups 3.56-3.57 ms, 84.4-84.6
//    % of peak, against 3.80 ms (79 %) for 256-thread ones with plain
//    non-temporal stores, 3.65 ms for one-wave ones with plain stores and
//    3.70 ms for 256-thread ones with streamed stores;
//  - pack of all three rows: one-wave workgroups 3.51-3.52 ms (85.5-85.8
//    %), 256-thread ones 3.73-3.74 ms; with the row on z instead (reading
//    one plain array in order), 3.63-3.65 ms one-wave, 3.84 ms (78.4 %)
//    256-thread with plain stores;
//  - pack of the master alone, m and v written as zeros (16 B per element,
//    three quarters of it writes): 256-thread workgroups 2.39-2.40 ms
//    (83.8-83.9 %), one-wave ones 2.50-2.51 ms; with the row on z, 2.48-
//    2.51 ms and 2.87-2.90 ms, and 2.61 ms with plain stores.
// So a pack that reads every row takes one-wave workgroups and a pack with
// a zero row 256-thread ones.  (Earlier forms: 4.57 and 4.44 ms, 66-68 %,
// with one 512-thread workgroup per tile walking all rows; 4.14 / 3.97 ms
// with 512-thread workgroups on z.)
constexpr int kStWave = 64, kStWide = 256;
constexpr int64_t kOrderedLaunchTiles = 4096;
template <int NT>
constexpr int st_parts() { return (int)(kTile / 4 / NT); }
static_assert(kMaxLaunchTiles * kTile / 4 < (int64_t(1) << 32),
              "one launch row of tiles fits the grid");

// offset of this thread's 4 floats inside its tile row
template <int NT>
__device__ __forceinline__ int state_off()
{
    constexpr int P = st_parts<NT>();
    return (int)(blockIdx.x % P) * (int)(kTile / P) + 4 * (int)threadIdx.x;
}

// plain rows -> tiled state; padding positions and rows without a source
// written as zero
template <int ROWS, class Loc, int NT>
__global__ __launch_bounds__(NT) void state_pack_kernel(
    Rows rw, float* __restrict__ state, int64_t x0, Loc loc)
{
    constexpr int P = st_parts<NT>();
    const int64_t rr = blockIdx.x / P;              // (x - x0) * ROWS + row
    const int64_t xr = rr / ROWS;
    const int row = (int)(rr - xr * ROWS);
    TileRef r;
    if (!loc.at_tile(x0 + xr, r))
        return;
    const int jj = state_off<NT>();
    const float* in = rw.in[row];
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (jj < r.nvalid && in)
        x = ld4(in + r.e0 + jj);
    st4_out(state + r.tile * (ROWS * kTile) + row * kTile, jj, x);
}

// tiled state -> plain rows (each nullable)
template <int ROWS, class Loc>
__global__ __launch_bounds__(kStWave) void state_unpack_kernel(
    const float* __restrict__ state, Rows rw, Loc loc)
{
    TileRef r;
    if (!loc.template at<st_parts<kStWave>()>(r))
        return;
    const int row = (int)blockIdx.z;
    const int jj = state_off<kStWave>();
    float* out = rw.out[row];
    if (jj < r.nvalid && out)
        zsdev::stream_store(
            out + r.e0, (uint32_t)(r.nvalid * (int64_t)sizeof(float)),
            (uint32_t)jj * (uint32_t)sizeof(float),
            ld4(state + r.tile * (ROWS * kTile) + row * kTile + jj));
}

// gradient slices [W][stride] -> tiled [tile][W][kTile]; padding zeroed.
// One tile row (tile, rank s) per kGtParts one-wave workgroups, one 16-byte
// group per thread (slice starts, strides and slice lengths are multiples
// of 8 elements; a partial group would be copied element-wise), in the
// order of the output: blockIdx.x = ((x - x0) * W + s) * kGtParts + part for
// tile x of the launch's row of tiles, so consecutive workgroups write
// consecutive memory, each reading its piece of slice s; the stores are
// streamed on to HBM with system scope.  A launch covers at most
// kGtLaunchTiles tiles (x0 is its first).  Measured on MI355X over the 8B
// shard at W = 8 (32 GB moved), three interleaved rounds: 4.72-4.74 ms,
// 84.7-85.1 % of peak, against 4.94-4.96 ms for 256-thread workgroups in
// this order and 5.09-5.10 ms (78.8 %) for the order it replaced, the rank
// row on the grid's z axis (workgroups in flight reading one slice front to
// back and writing 16 KiB rows W rows apart; 256 threads, streamed stores;
// 5.20 ms with plain stores; 64 to 1024 threads 5.48-6.02 ms).
constexpr int kGtThreads = 64;
constexpr int kGtParts = (int)(kTile / 8 / kGtThreads);   // 16 per row
constexpr int64_t kGtLaunchTiles = kOrderedLaunchTiles;

template <class Loc>
__global__ __launch_bounds__(kGtThreads) void grads_tile_kernel(
    const uint16_t* __restrict__ slices, int64_t stride,
    uint16_t* __restrict__ tiled, int32_t W, int64_t x0, Loc loc)
{
    const int64_t row = blockIdx.x / kGtParts;      // (x - x0) * W + s
    const int64_t xr = row / W;
    const int64_t s = row - xr * W;
    TileRef r;
    if (!loc.at_tile(x0 + xr, r))
        return;
    uint16_t* dst = tiled + (r.tile * (int64_t)W + s) * kTile;
    const uint16_t* src = slices + r.e0 + s * stride;
    const int g = (int)(blockIdx.x % kGtParts) * kGtThreads + (int)threadIdx.x;
    const int nv = (int)(r.nvalid / 8);                // whole valid groups
    const uint32_t row_bytes = (uint32_t)(kTile * sizeof(uint16_t));
    if (g < nv) {
        zsdev::stream_store(
            dst, row_bytes, (uint32_t)g * (uint32_t)sizeof(u32x4),
            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) +
                                       g));
    } else if (g > nv || r.nvalid % 8 == 0) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        zsdev::stream_store(dst, row_bytes,
                            (uint32_t)g * (uint32_t)sizeof(u32x4), z);
    } else {
        // the partial group (the layouts never produce one): its valid
        // elements and zeros
        for (int j = g * 8; j < g * 8 + 8; ++j)
            dst[j] = j < r.nvalid ? src[j] : (uint16_t)0;
    }
}

// ---- pack: shard -> flat all-gather buffer ---------------------------------

// Sixteen one-wave workgroups per tile, one 16-byte copy per thread, the
// stores streamed on to HBM with system scope (zsdev::stream_store): on the
// 8B-shaped shard 0.590-0.593 ms (84.7-85.0 % of peak) against 0.602-0.603
// ms (83.2-83.4 %) with plain non-temporal stores, 0.637-0.642 ms
// (78.2-78.8 %) for four 256-thread workgroups of one copy and 0.671 ms for
// eight 128-thread ones, interleaved in one process.  Reserving LDS to hold fewer of them per CU only slowed it
// (28 per CU 78.8 %, 16 per CU 69.5 %): a copy needs every load in flight
// the device takes.  Earlier trials of the same stream: eight one-wave
// workgroups of two copies per thread 0.652-0.665 ms, two 256-thread
// workgroups of two 0.660-0.673 ms, one 512-thread workgroup of 8-byte
// copies 5.89-5.93 TB/s.
// Slices and padded tensors are multiples of 8 elements, so a 16-byte group
// is either wholly inside the tile's valid part or wholly outside.
constexpr int kPackNT = 64;
constexpr int kPackV = 1;                         // 16-byte copies per thread
constexpr int kPackP = (int)(kTile / (kPackNT * kPackV * 8));  // 16 per tile
static_assert(kMaxLaunchTiles * kPackP * kPackNT < (int64_t(1) << 32),
              "one launch row of tiles fits the grid");

template <class Loc>
__global__ __launch_bounds__(kPackNT) void pack_flat_kernel(
    const uint16_t* __restrict__ shard, uint16_t* __restrict__ flat,
    Loc loc)
{
    TileRef r;
    if (!loc.template at<kPackP>(r))
        return;
    const int part = (int)(blockIdx.x % kPackP);
#pragma unroll
    for (int v = 0; v < kPackV; ++v) {
        const int jj = part * (int)(kTile / kPackP) +
                       8 * (v * kPackNT + (int)threadIdx.x);
        if (jj < r.nvalid)
            zsdev::stream_store(
                flat + r.fpos, (uint32_t)(r.nvalid * sizeof(uint16_t)),
                (uint32_t)jj * (uint32_t)sizeof(uint16_t),
                __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(shard + r.e0 + jj)));
    }
}

// ---- pack: shard -> per-tensor storage through the chunk table -------------
//
// One-wave workgroups, up to kPackGridX of them per chunk striding over it,
// 8 elements per thread and step, the 16-byte stores streamed on to HBM
// with system scope.  Measured on MI355X (the 8B-shaped W = 8 shard's 650
// chunks): 0.593-0.594 ms (84.5-84.6 % of peak) against 0.604 ms (83.1 %)
// with plain non-temporal stores, interleaved in one process; 0.65 ms with
// 256-thread workgroups and at most 256 per chunk (64 threads and 256 per
// chunk: 0.67-0.74 ms; 256 threads and 4096: 0.64 ms).

constexpr int kPackThreads = 64;
constexpr int64_t kPackGridX = 4096;
constexpr int kPackGroup = 8;
constexpr int64_t kPackTile = kPackThreads * kPackGroup;

__global__ __launch_bounds__(kPackThreads) void pack_chunks_kernel(
    const uint16_t* __restrict__ shard, const zs_chunk* __restrict__ chunks,
    int32_t c0, uint16_t* const* __restrict__ tensors)
{
    // one chunk per blockIdx.y; the chunk record and tensor pointer are the
    // same for the whole workgroup
    const zs_chunk ch = chunks[c0 + (int32_t)blockIdx.y];
    uint16_t* dst = tensors[ch.tensor_id] + ch.tensor_off;
    const uint16_t* src = shard + ch.shard_off;
    const int64_t n = ch.numel;
    const int64_t step = (int64_t)gridDim.x * kPackTile;
    const bool vec = ((reinterpret_cast<uintptr_t>(dst) |
                       reinterpret_cast<uintptr_t>(src)) & 15u) == 0;
    // jw: the wave's first element this step (wave-uniform), the base of
    // its store region
    for (int64_t jw = (int64_t)blockIdx.x * kPackTile; jw < n; jw += step) {
        const int64_t j = jw + (int64_t)threadIdx.x * kPackGroup;
        if (j >= n)
            continue;
        if (vec && j + kPackGroup <= n) {
            const int64_t left = n - jw;
            zsdev::stream_store(
                dst + jw,
                (uint32_t)((left < kPackTile ? left : kPackTile) *
                           (int64_t)sizeof(uint16_t)),
                (uint32_t)threadIdx.x * (uint32_t)(kPackGroup *
                                                   sizeof(uint16_t)),
                __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(src + j)));
        } else {
            const int64_t end = j + kPackGroup < n ? j + kPackGroup : n;
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

int64_t tiles_for(int64_t slice)
{
    return (slice + kTile - 1) / kTile;
}

// One launch range of the whole shard: buckets [y0, y0 + ny).  Every bucket
// before the last is full, so bucket y0 starts at element y0*S of the shard
// and at tile y0*TPB.
struct Range {
    int64_t y0, ny;
    Geom g;
};

// Calls fn(range) for each chunk of at most kMaxGridY buckets.
template <class Fn>
int for_shard_ranges(const zs_layout* L, Fn fn)
{
    const int64_t nb = (int64_t)L->buckets.size();
    Geom g;
    g.S = L->buckets[0].slice_numel;
    g.B = L->buckets[0].numel;
    g.S_last = L->buckets.back().slice_numel;
    g.TPB = tiles_for(g.S);
    g.rank = L->rank;
    for (int64_t y0 = 0; y0 < nb; y0 += kMaxGridY) {
        Range r;
        r.y0 = y0;
        r.ny = nb - y0 < kMaxGridY ? nb - y0 : kMaxGridY;
        r.g = g;
        r.g.q_last = (nb - 1 - y0 < r.ny) ? (int32_t)(nb - 1 - y0) : -1;
        const int rc = fn(r);
        if (rc) return rc;
    }
    return ZS_OK;
}

// Calls fn(loc, grid, shard_base, tile_base, flat_base) for every launch
// that covers the whole shard: regular bucket ranges in the flat mode
// (positions relative to the bases), groups of up to kMaxMembers owned
// tensors in the whole-tensor mode (absolute positions, zero bases, a 1-D
// grid over the group's tiles).
template <class Fn>
int for_launches(const zs_layout* L, Fn fn)
{
    if (!L->whole_tensors)
        return for_shard_ranges(L, [&](const Range& R) {
            const zs_bucket& b0 = L->buckets[R.y0];
            GeomLoc loc;
            loc.g = R.g;
            return fn(loc, dim3((unsigned)R.g.TPB, (unsigned)R.ny),
                      b0.shard_off, b0.tile_off, b0.flat_off);
        });
    const int64_t nb = (int64_t)L->buckets.size();
    for (int64_t g0 = 0; g0 < nb;) {
        SegLoc loc;
        int cnt = 0;
        loc.start[0] = 0;
        for (; cnt < kMaxMembers && g0 + cnt < nb; ++cnt) {
            const zs_bucket& b = L->buckets[g0 + cnt];
            const int64_t nt = tiles_for(b.slice_numel);
            if (cnt > 0 && loc.start[cnt] + nt > kMaxLaunchTiles)
                break;
            loc.s[cnt] = Seg{b.shard_off, b.tile_off, slice_flat_pos(L, b),
                             b.slice_numel};
            loc.start[cnt + 1] = loc.start[cnt] + nt;
        }
        loc.count = cnt;
        g0 += cnt;
        const int rc = fn(loc, dim3((unsigned)loc.start[cnt], 1), 0, 0, 0);
        if (rc) return rc;
    }
    return ZS_OK;
}

Geom bucket_geom(const zs_layout* L, const zs_bucket& b)
{
    Geom g;
    g.S = b.slice_numel;
    g.S_last = b.slice_numel;
    g.B = b.numel;
    g.TPB = tiles_for(b.slice_numel);
    g.q_last = 0;
    g.rank = L->rank;
    return g;
}

// Kernel choice: Args = StepArgs (whole shard) or GroupArgs (buckets).
// Residency cap.  Nothing in the step kernels uses LDS, so reserving LDS
// at launch is what sets how many of their small workgroups share a CU:
// LDS per CU / k (rounded down to 512 bytes) lets k of them in.  Measured
// on MI355X, the stream runs faster with far fewer workgroups in flight
// than would fit (32 one-wave workgroups per CU): the device then sweeps
// fewer tiles' rows at a time, as a wider active window of tiles measured
// slower (the device's achievable read/write mix rises from 82-83 % to
// 84-86 % of peak).  The right k depends on the work shape and W; see the
// shape table below.  Where the device's LDS size cannot be had the step
// launches uncapped.
constexpr int kCapDevices = 64;
std::atomic<int> g_lds_per_cu[kCapDevices];     // bytes; 0 = not known yet
std::atomic<int> g_cap_on{1};                   // zs_set_residency_cap

// LDS bytes to reserve per workgroup so that at most `wgs` share a CU, or 0
// (no cap) for wgs == 0 or when the device's LDS size cannot be had.
unsigned residency_cap_lds(int wgs)
{
    if (wgs <= 0 || !g_cap_on.load(std::memory_order_relaxed))
        return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kCapDevices)
        return 0;
    int lds = g_lds_per_cu[dev].load(std::memory_order_relaxed);
    if (lds == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(
                &v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                dev) != hipSuccess || v <= 0)
            v = -1;
        g_lds_per_cu[dev].store(v, std::memory_order_relaxed);
        lds = v;
    }
    if (lds <= 0)
        return 0;
    return (unsigned)(lds / wgs / 512 * 512);
}

// WGS: workgroups per CU (0 = uncapped).
template <int WT, bool TILED, class SH, bool PURE, int WGS, class Args>
void launch_kernel(const Args& a, dim3 grid, hipStream_t s)
{
    grid.x *= SH::P;
    const unsigned lds = residency_cap_lds(WGS);
    if constexpr (std::is_same<Args, StepArgs>::value)
        hipLaunchKernelGGL((step_kernel<WT, TILED, SH, PURE>), grid,
                           dim3(SH::NT), lds, s, a);
    else if constexpr (std::is_same<Args, PlainArgs>::value)
        hipLaunchKernelGGL((step_plain_kernel<WT, TILED, SH>), grid,
                           dim3(SH::NT), lds, s, a);
    else
        hipLaunchKernelGGL((group_step_kernel<WT, TILED, SH, PURE>), grid,
                           dim3(SH::NT), lds, s, a);
}

template <int WT, class SH, bool PURE, int WGS, class Args>
void launch_shape(const Args& a, bool tiled, dim3 grid, hipStream_t s)
{
    if (tiled)
        launch_kernel<WT, true, SH, PURE, WGS>(a, grid, s);
    else
        launch_kernel<WT, false, SH, PURE, WGS>(a, grid, s);
}

// Work shapes and residency, chosen by measurement on MI355X (8B-shaped
// shard at W = 4, 5, 8 and 16, 7B-shaped at W = 32, 64 and 100, 70B-shaped
// bucket groups at W = 16; three arenas per process, several processes):
//  - One (compiled W; on plain slices only below W = 32): one wave per
//    workgroup, one 4-element unit per thread, all W gradient slices
//    loaded in one batch (at least 4), 32 workgroups per tile, and few of
//    them per CU.  Launches of 4096 tiles or more (one_wgs):
//      W = 8:  12 per CU, 85.0 % in three processes (the same shape with 16
//              per CU 84.5-85.1 %, with 11 or 14 84.3-84.7 %; slices loaded
//              4 at a time, 16 per CU, 83.4-84.9 %; uncapped 80.5-83.3 %);
//              pure bf16 10 per CU, 86.0-86.6 % (12 per CU: 82.9-83.5 %);
//      W = 4:  12 per CU, 85.3-85.9 % (16: 83.6-84.0 %; uncapped 82.2 %);
//      W = 16: 7 per CU, 82.3-87.0 % (8: 80.9-84.2 %, 6: 75-76 %; slices 4
//              at a time with 16 per CU 82.9 %);
//      W = 32: 6 per CU, 84.5-85.7 % (5 or 7: 81.4-81.8 %); 512-thread
//              workgroups of 8-slice batches (the earlier Deep shape, 148
//              VGPRs, one per CU) 77.4-80.3 %;
//      W = 64: 5 per CU, 82.7-84.6 % (4: 82.9-84.1 %, 3: 67 %); pure bf16 6
//              per CU, 82.6-84.5 %; Deep 79.0-80.7 % (pure 80.4-81.2 %);
//      W = 1, 2: 16 per CU (not measured apart);
//      the step on three plain state arrays (plain_wgs), interleaved over
//      three placements of the arrays: W = 8 8 per CU, 85.4-85.7 % (12:
//      82.1-82.5 %, 7: 84.7-85.4 %, 9: 83.6-83.9 %, 10: 83.6-83.8 %, 6:
//      71 %, 16: 78 %); W = 4 10 per CU, 84.0-85.0 % (12: 82.3-82.5 %, 8:
//      82.8-83.9 %); at W = 16, 32 and 64 the mixed caps held (W = 16 6 per
//      CU 80.8-84.1 % against 80.3-82.0 %, too close to the drop at 5).
//    Launches of fewer tiles (small_wgs: bucket groups of a streaming
//    step, GPT-2-sized shards), in one process each, against Small:
//      W = 8:  16 per CU: GPT-2-shaped shard (1899 tiles) 82.8-82.9 % (12:
//              82.1 %, 20: 82.1 %, 8: 76.6 %; Small 81.8-81.9 %); 8B-shaped
//              groups of 16 buckets (3200 tiles) on two streams 83.6-83.8 %
//              (12: 82.5 %, 20: 83.2 %; Small 81.6-82.0 %);
//      W = 16: 7 per CU: 70B-shaped groups of 16 (1600 tiles) 37.06-37.15
//              ms per full step, 86.1-86.3 % (8: 85.6-85.8 %, 6: 72.5 %;
//              Small 38.7-38.8 ms, 82.4-82.6 %);
//      W = 64: 5 per CU: 7B-shaped groups of 16 (400 tiles) 81.7 % (4:
//              82.2 %, 6: 80.8 %; Small uncapped 77.6 %).
//    The cap and the batch depth act together (more slices per wave, fewer
//    waves), and the optimum is narrow at W = 16 and 32: one more or one
//    fewer workgroup per CU costs 3-10 points there.
//  - Runtime W, mixed precision, 4096 tiles or more (launch_runtime_one):
//    one-wave workgroups, slices in batches of 8 (W <= 8), 16 (W <= 16) or
//    32 (W <= 64) or 64, 12 / 12 / 8 (W <= 32) / 7 / 6 per CU; tiled
//    gradients, and plain slices at W <= 8.  Against the earlier Wave and
//    Wide shapes, interleaved in one process each: W = 3 85.9 % (80.9 %),
//    W = 5 85.7 % (81.3 %; plain slices 85.9 %, 82.7 %; plain state 83.0 %,
//    77.5 %), W = 12 84.4-84.6 % (82.7-82.8 %), W = 20 86.0-86.2 %
//    (78.8-79.4 %), W = 33 82.5-83.1 % (76.8-77.7 %), W = 48 83.0-83.1 %
//    (78.7-79.6 %; plain state 78.8 %, 74.2 %), W = 100 82.4-82.7 %
//    (78.9-81.0 %), W = 128 82.8-82.9 % (79.7 %).  The pure-bf16 step on
//    tiled gradients above W = 8, with 14 per CU at W <= 16: W = 12 84.9 %
//    (81.4 %), W = 20 80.0 % (76.2 %), W = 24 81.9 % (78.0 %), W = 48 79.9 %
//    (77.0 %), W = 100 81.8 % (80.9 %); at W = 5 it lost (76 % against
//    82 %).  Plain slices at W = 20 fell to 53 % with a 32-slice batch;
//  - Wave (runtime W < 32: the pure-bf16 step up to W = 8, plain slices
//    above W = 8, bucket groups): the same one-wave unit, slices 4 at a time,
//    uncapped (W = 5: the cap lost, 79-82 % against 82-84 %); and, 16 per
//    CU, large group launches at compiled W < 32 (the whole-tensor step's
//    owned tensors, 32 per launch: 84.7-85.0 % on the 8B-shaped W = 8
//    shard, where One at 12 per CU gave 79.7-82.6 %; interleaved in one
//    process, Wave 84.1 % against One at 12-24 per CU 83.3-84.0 %);
//  - Deep (512-thread workgroups of four units, slices 8 at a time, one
//    per CU by its 148 VGPRs), uncapped: plain slice rows at compiled
//    W >= 32 (7B-shaped W = 64: 73-77 %, One 66 %), also in large group
//    launches (on tiled gradients those take One: the 7B-shaped whole-tensor
//    step at W = 64 83.3-83.5 % at 4-5 per CU against Deep's 80.3 %);
//  - Wide / PureWide (runtime W >= 32 for plain slices and bucket groups): 512-thread workgroups of four units (256 for the
//    two-row pure state): 79-80 % at W = 100, against 75-78 % with uncapped
//    one-wave workgroups;
//  - Runtime W above 8, mixed precision on tiled gradients, launches of
//    fewer tiles too (bucket groups of 16 on two streams): W = 12 84.8 %
//    (Small 79.9 %), W = 24 85.0 % (78.3 %), W = 48 82.0 % (76.0 %), W = 100
//    80.1 % (75.7 %);
//  - Small (launches of fewer than kSmallLaunch tiles at runtime W up to 8
//    and for the pure-bf16 step, and on plain slices at W >= 32): one unit per thread and sixteen
//    128-thread workgroups per tile, so that a few hundred or thousand
//    tiles still spread evenly over the 256 CUs with a short tail,
//    uncapped (it ran the compiled-W small launches before One: GPT-2-
//    shaped W = 8 shard 81.4-81.5 % at 8 per CU, against 79.6-79.7 % for
//    four 512-thread workgroups per tile and 75 % for Wide).
template <int WT>
using ShapeOne = Shape<64, 1, (WT < 4 ? 4 : WT)>;
using ShapeWave = Shape<64, 1, 4>;
using ShapeDeep = Shape<512, 4, 8>;
using ShapeWide = Shape<512, 4, 4>;
using ShapeSmall = Shape<128, 1, 4>;
using ShapePureWide = Shape<256, 4, 4>;
constexpr int64_t kSmallLaunch = 4096;
constexpr int kWaveWgs = 16;

template <int WT, bool PURE>
constexpr int one_wgs()
{
    if constexpr (WT == 8)
        return PURE ? 10 : 12;
    else if constexpr (WT == 64)
        return PURE ? 6 : 5;
    else if constexpr (WT == 4)
        return 12;
    else if constexpr (WT == 16)
        return 7;
    else if constexpr (WT == 32)
        return 6;
    else
        return 16;
}

// the step on three plain state arrays (zs_step_plain), launches of
// kSmallLaunch tiles or more: its state rows lie in three separate arrays,
// and fewer workgroups per CU pay at W = 4 and 8
template <int WT>
constexpr int plain_wgs()
{
    return WT == 8 ? 8 : WT == 4 ? 10 : one_wgs<WT, false>();
}

// launches of fewer than kSmallLaunch tiles: more workgroups per CU at
// W <= 8, where the tail of a short launch weighs more
template <int WT, bool PURE>
constexpr int small_wgs()
{
    return WT <= 8 ? 16 : one_wgs<WT, PURE>();
}

// every shape stays within the launch limit of kMaxLaunchTiles tiles
static_assert(kMaxLaunchTiles * ShapeWave::P * ShapeWave::NT <
                  (int64_t(1) << 32) &&
              kMaxLaunchTiles * ShapeSmall::P * ShapeSmall::NT <
                  (int64_t(1) << 32),
              "one launch row of tiles fits the grid");

// Runtime W (outside the compiled set): one-wave workgroups whose batch
// covers W up to 32 at once, and few of them per CU.  Launches of
// kSmallLaunch tiles or more of the mixed-precision step take it on tiled
// gradients, and on plain slice rows for W <= 8 (a W = 20 batch of 32 slice
// rows ran at 53 %); those of the pure-bf16 step on tiled gradients above
// W = 8 (at W = 5 it lost); smaller launches of the mixed-precision step on
// tiled gradients above W = 8 (bucket groups).
template <bool PURE, class Args>
void launch_runtime_one(const Args& a, bool tiled, dim3 grid, hipStream_t s)
{
    if (a.W <= 8) {
        if constexpr (!PURE)
            launch_shape<0, Shape<64, 1, 8>, false, 12>(a, tiled, grid, s);
    } else if (a.W <= 16) {
        launch_kernel<0, true, Shape<64, 1, 16>, PURE, PURE ? 14 : 12>(
            a, grid, s);
    } else if (a.W <= 32) {
        launch_kernel<0, true, Shape<64, 1, 32>, PURE, 8>(a, grid, s);
    } else if (a.W <= 64) {
        launch_kernel<0, true, Shape<64, 1, 32>, PURE, 7>(a, grid, s);
    } else {
        launch_kernel<0, true, Shape<64, 1, 64>, PURE, 6>(a, grid, s);
    }
}

// grid: one x per tile (launch_kernel multiplies by the shape's P)
template <int WT, bool PURE, class Args>
void launch_step_w(const Args& a, bool tiled, dim3 grid, hipStream_t s)
{
    const int64_t tiles = (int64_t)grid.x * grid.y;
    constexpr bool kGroup = std::is_same<Args, GroupArgs>::value;
    constexpr bool kPlain = std::is_same<Args, PlainArgs>::value;
    if (tiles < kSmallLaunch) {
        if constexpr (WT > 0) {
            if (tiled || WT < 32) {
                launch_shape<WT, ShapeOne<WT>, PURE, small_wgs<WT, PURE>()>(
                    a, tiled, grid, s);
                return;
            }
        } else if constexpr (!PURE) {
            if (tiled && a.W > 8) {         // runtime W, as for large launches
                launch_runtime_one<PURE>(a, tiled, grid, s);
                return;
            }
        }
        launch_shape<WT, ShapeSmall, PURE, 0>(a, tiled, grid, s);
    } else if constexpr (WT > 0 && kGroup) {
        // large group launches (the whole-tensor step's owned tensors):
        // below W = 32 the member lookup of every workgroup wants more of
        // them per CU; at W >= 32 the One shape on tiled gradients
        if constexpr (WT < 32) {
            launch_shape<WT, ShapeWave, PURE, kWaveWgs>(a, tiled, grid, s);
        } else {
            if (tiled)
                launch_kernel<WT, true, ShapeOne<WT>, PURE,
                              one_wgs<WT, PURE>()>(a, grid, s);
            else
                launch_kernel<WT, false, ShapeDeep, PURE, 0>(a, grid, s);
        }
    } else if constexpr (WT > 0) {
        constexpr int kWgs = kPlain ? plain_wgs<WT>() : one_wgs<WT, PURE>();
        if (tiled || WT < 32)
            launch_shape<WT, ShapeOne<WT>, PURE, kWgs>(a, tiled, grid, s);
        else                                // W plain slice rows, W >= 32
            launch_kernel<WT, false, ShapeDeep, PURE, 0>(a, grid, s);
    } else {                                // runtime W
        if constexpr (!kGroup) {
            if (PURE ? tiled && a.W > 8 : tiled || a.W <= 8) {
                launch_runtime_one<PURE>(a, tiled, grid, s);
                return;
            }
        }
        if (a.W < 32)
            launch_shape<WT, ShapeWave, PURE, 0>(a, tiled, grid, s);
        else if constexpr (PURE)
            launch_shape<WT, ShapePureWide, PURE, 0>(a, tiled, grid, s);
        else
            launch_shape<WT, ShapeWide, PURE, 0>(a, tiled, grid, s);
    }
}

template <bool PURE = false, class Args>
int launch_step(const Args& a, bool tiled, dim3 grid, hipStream_t s)
{
    switch (a.W) {
    case 1: launch_step_w<1, PURE>(a, tiled, grid, s); break;
    case 2: launch_step_w<2, PURE>(a, tiled, grid, s); break;
    case 4: launch_step_w<4, PURE>(a, tiled, grid, s); break;
    case 8: launch_step_w<8, PURE>(a, tiled, grid, s); break;
    case 16: launch_step_w<16, PURE>(a, tiled, grid, s); break;
    case 32: launch_step_w<32, PURE>(a, tiled, grid, s); break;
    case 64: launch_step_w<64, PURE>(a, tiled, grid, s); break;
    default: launch_step_w<0, PURE>(a, tiled, grid, s); break;
    }
    return check_launch("step kernel");
}

// Checks shared by zs_step and zs_bucket_step.  `len` is the number of
// gradient elements per slice the call reads.
int check_step_args(const zs_layout* L, const uint16_t* grads,
                    int32_t grad_layout, int64_t grad_stride, int64_t len,
                    const float* state, const uint16_t* pshard,
                    const uint16_t* flat, const zs_adamw* hp, int64_t step)
{
    using zs::fail;
    if (!hp) return fail(ZS_EINVAL, "hp is NULL");
    if (step < 1) return fail(ZS_EINVAL, "step %lld < 1", (long long)step);
    if (grad_layout != ZS_GRADS_SLICES && grad_layout != ZS_GRADS_TILED)
        return fail(ZS_EINVAL, "unknown grad_layout %d", grad_layout);
    if (!grads || !state)
        return fail(ZS_EINVAL, "grads and state must be non-NULL");
    if (!pshard && !flat)
        return fail(ZS_EINVAL, "need param_shard or full_flat");
    if (!aligned16(grads) || !aligned16(state) ||
        (pshard && !aligned16(pshard)) || (flat && !aligned16(flat)))
        return fail(ZS_EALIGN, "device pointers must be 16-byte aligned");
    if (grad_layout == ZS_GRADS_SLICES) {
        if (grad_stride % 8)
            return fail(ZS_EALIGN, "grad_stride %lld is not a multiple of 8",
                        (long long)grad_stride);
        if (grad_stride < len)
            return fail(ZS_ERANGE, "grad_stride %lld < %lld elements per "
                        "slice", (long long)grad_stride, (long long)len);
        if (grad_stride > INT64_MAX / 2 / L->world)
            return fail(ZS_ERANGE, "W * grad_stride overflows");
    }
    return ZS_OK;
}

}  // namespace

namespace {

// Group launches over `count` buckets of the layout (ids[i]), each member's
// gradients at grads_of(i) (a bucket's staging, or its part of whole-shard
// gradients); state / pshard / flat are whole-shard bases.  PURE: state is
// the two-row [m|v] state and pshard / flat is the in-out parameter.
template <bool PURE, class GradsOf>
int launch_groups(const zs_layout* L, int32_t count, const int32_t* ids,
                  GradsOf grads_of, bool tiled, int64_t grad_stride,
                  float* state, uint16_t* pshard, uint16_t* flat,
                  const Consts& c, hipStream_t s)
{
    constexpr int kRows = PURE ? 2 : 3;
    for (int32_t g0 = 0; g0 < count;) {
        GroupArgs a;
        int32_t cnt = 0;
        a.start[0] = 0;
        for (; cnt < kMaxMembers && g0 + cnt < count; ++cnt) {
            const zs_bucket& b = L->buckets[ids[g0 + cnt]];
            const int64_t nt = tiles_for(b.slice_numel);
            if (cnt > 0 && a.start[cnt] + nt > kMaxLaunchTiles)
                break;
            GroupMember& mb = a.mb[cnt];
            mb.grads = grads_of(g0 + cnt);
            mb.state = state + b.tile_off * kRows * kTile;
            mb.pshard = pshard ? pshard + b.shard_off : nullptr;
            mb.flat = flat ? flat + slice_flat_pos(L, b) : nullptr;
            mb.slice = b.slice_numel;
            a.start[cnt + 1] = a.start[cnt] + nt;
        }
        a.count = cnt;
        g0 += cnt;
        a.gstride = grad_stride;
        a.W = L->world;
        a.c = c;
        const int rc = launch_step<PURE>(
            a, tiled, dim3((unsigned)a.start[cnt], 1), s);
        if (rc) return rc;
    }
    return ZS_OK;
}

// Whole-shard step, flat or whole-tensor layout.
template <bool PURE>
int shard_step(const zs_layout* L, const uint16_t* grads, bool tiled,
               int64_t grad_stride, float* state, uint16_t* pshard,
               uint16_t* flat, const Consts& c, hipStream_t s)
{
    constexpr int kRows = PURE ? 2 : 3;
    const int32_t W = L->world;
    if (L->whole_tensors) {
        const int32_t nb = (int32_t)L->buckets.size();
        std::vector<int32_t> ids(nb);
        for (int32_t i = 0; i < nb; ++i) ids[i] = i;
        return launch_groups<PURE>(
            L, nb, ids.data(),
            [&](int32_t i) {
                const zs_bucket& b = L->buckets[i];
                return tiled ? grads + b.tile_off * W * kTile
                             : grads + b.shard_off;
            },
            tiled, grad_stride, state, pshard, flat, c, s);
    }
    return for_shard_ranges(L, [&](const Range& R) {
        const zs_bucket& b0 = L->buckets[R.y0];
        StepArgs a;
        a.grads = tiled ? grads + b0.tile_off * W * kTile
                        : grads + b0.shard_off;
        a.gstride = grad_stride;
        a.state = state + b0.tile_off * kRows * kTile;
        a.pshard = pshard ? pshard + b0.shard_off : nullptr;
        a.flat = flat ? flat + b0.flat_off : nullptr;
        a.g = R.g;
        a.W = W;
        a.c = c;
        return launch_step<PURE>(a, tiled,
                                 dim3((unsigned)R.g.TPB, (unsigned)R.ny), s);
    });
}

// Whole-shard step on three plain arrays: one launch per range of regular
// buckets in the flat mode, one per owned tensor in the whole-tensor mode.
int plain_step(const zs_layout* L, const uint16_t* grads, bool tiled,
               int64_t grad_stride, float* master, float* m, float* v,
               uint16_t* pshard, uint16_t* flat, const Consts& c,
               hipStream_t s)
{
    const int32_t W = L->world;
    auto args = [&](const zs_bucket& b0, const Geom& g, int64_t fpos) {
        PlainArgs a;
        a.grads = tiled ? grads + b0.tile_off * W * kTile
                        : grads + b0.shard_off;
        a.gstride = grad_stride;
        a.master = master + b0.shard_off;
        a.m = m + b0.shard_off;
        a.v = v + b0.shard_off;
        a.pshard = pshard ? pshard + b0.shard_off : nullptr;
        a.flat = flat ? flat + fpos : nullptr;
        a.g = g;
        a.W = W;
        a.c = c;
        return a;
    };
    if (L->whole_tensors) {
        for (const zs_bucket& b : L->buckets) {
            Geom g = bucket_geom(L, b);
            g.rank = 0;               // the tensor's flat offset is absolute
            const int rc = launch_step<false>(
                args(b, g, slice_flat_pos(L, b)), tiled,
                dim3((unsigned)g.TPB, 1), s);
            if (rc) return rc;
        }
        return ZS_OK;
    }
    return for_shard_ranges(L, [&](const Range& R) {
        const zs_bucket& b0 = L->buckets[R.y0];
        return launch_step<false>(args(b0, R.g, b0.flat_off), tiled,
                                  dim3((unsigned)R.g.TPB, (unsigned)R.ny), s);
    });
}

}  // namespace

extern "C" int zs_step_plain(const zs_layout* L, const uint16_t* grads,
                             int32_t grad_layout, int64_t grad_stride,
                             float* master, float* m, float* v,
                             uint16_t* param_shard, uint16_t* full_flat,
                             const zs_adamw* hp, int64_t step,
                             void* hip_stream)
{
    zs::clear_error();
    if (!L) return zs::fail(ZS_EINVAL, "layout is NULL");
    if (!hp) return zs::fail(ZS_EINVAL, "hp is NULL");
    if (step < 1) return zs::fail(ZS_EINVAL, "step %lld < 1", (long long)step);
    if (L->shard_numel == 0)
        return ZS_OK;
    if (!m || !v)
        return zs::fail(ZS_EINVAL, "master, m and v must be non-NULL");
    if (!aligned16(m) || !aligned16(v))
        return zs::fail(ZS_EALIGN, "device pointers must be 16-byte aligned");
    int rc = check_step_args(L, grads, grad_layout, grad_stride,
                             L->shard_numel, master, param_shard, full_flat,
                             hp, step);
    if (rc) return rc;
    return plain_step(L, grads, grad_layout == ZS_GRADS_TILED, grad_stride,
                      master, m, v, param_shard, full_flat,
                      make_consts(*hp, step, L->world),
                      static_cast<hipStream_t>(hip_stream));
}

extern "C" int zs_step(const zs_layout* L, const uint16_t* grads,
                       int32_t grad_layout, int64_t grad_stride, float* state,
                       uint16_t* param_shard, uint16_t* full_flat,
                       const zs_adamw* hp, int64_t step, void* hip_stream)
{
    zs::clear_error();
    if (!L) return zs::fail(ZS_EINVAL, "layout is NULL");
    if (!hp) return zs::fail(ZS_EINVAL, "hp is NULL");
    if (step < 1) return zs::fail(ZS_EINVAL, "step %lld < 1", (long long)step);
    if (L->shard_numel == 0)
        return ZS_OK;
    int rc = check_step_args(L, grads, grad_layout, grad_stride,
                             L->shard_numel, state, param_shard, full_flat,
                             hp, step);
    if (rc) return rc;
    return shard_step<false>(L, grads, grad_layout == ZS_GRADS_TILED,
                             grad_stride, state, param_shard, full_flat,
                             make_consts(*hp, step, L->world),
                             static_cast<hipStream_t>(hip_stream));
}

extern "C" int zs_buckets_step(const zs_layout* L, int32_t count,
                               const int32_t* bucket_ids,
                               const uint16_t* const* grads,
                               int32_t grad_layout, int64_t grad_stride,
                               float* state, uint16_t* param_shard,
                               uint16_t* full_flat, const zs_adamw* hp,
                               int64_t step, void* hip_stream)
{
    using zs::fail;
    zs::clear_error();
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    if (count < 1 || count > kMaxGroup)
        return fail(ZS_EINVAL, "count %d outside [1, %d]", count, kMaxGroup);
    if (!bucket_ids || !grads)
        return fail(ZS_EINVAL, "bucket_ids and grads must be non-NULL");
    const int32_t nb = (int32_t)L->buckets.size();
    for (int32_t i = 0; i < count; ++i) {
        const int32_t b = bucket_ids[i];
        if (b < 0 || b >= nb)
            return fail(ZS_ERANGE, "bucket_ids[%d] = %d outside [0, %d)", i,
                        b, nb);
        for (int32_t k = 0; k < i; ++k)
            if (bucket_ids[k] == b)
                return fail(ZS_EINVAL, "bucket %d appears twice", b);
        const int rc = check_step_args(L, grads[i], grad_layout, grad_stride,
                                       L->buckets[b].slice_numel, state,
                                       param_shard, full_flat, hp, step);
        if (rc) return rc;
    }
    return launch_groups<false>(
        L, count, bucket_ids, [&](int32_t i) { return grads[i]; },
        grad_layout == ZS_GRADS_TILED, grad_stride, state, param_shard,
        full_flat, make_consts(*hp, step, L->world),
        static_cast<hipStream_t>(hip_stream));
}

extern "C" int zs_bucket_step(const zs_layout* L, int32_t bucket_id,
                              const uint16_t* grads, int32_t grad_layout,
                              int64_t grad_stride, float* state,
                              uint16_t* param_shard, uint16_t* full_flat,
                              const zs_adamw* hp, int64_t step,
                              void* hip_stream)
{
    zs::clear_error();
    if (!L) return zs::fail(ZS_EINVAL, "layout is NULL");
    if (bucket_id < 0 || bucket_id >= (int32_t)L->buckets.size())
        return zs::fail(ZS_ERANGE, "bucket_id %d outside [0, %d)", bucket_id,
                        (int)L->buckets.size());
    return zs_buckets_step(L, 1, &bucket_id, &grads, grad_layout,
                           grad_stride, state, param_shard, full_flat, hp,
                           step, hip_stream);
}

namespace {

// Pack (unpack) ROWS plain arrays into (out of) a tiled state.
template <int ROWS>
int convert_state(const zs_layout* L, bool pack, const float* const* in,
                  float* const* out, float* state_w, const float* state_r,
                  void* hip_stream)
{
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    return for_launches(L, [&](const auto& loc, dim3 grid, int64_t e,
                               int64_t t, int64_t) {
        Rows rw{};
        bool every_row = true;              // (pack) every row has a source
        for (int row = 0; row < ROWS; ++row) {
            rw.in[row] = (pack && in[row]) ? in[row] + e : nullptr;
            rw.out[row] = (!pack && out[row]) ? out[row] + e : nullptr;
            every_row = every_row && in && in[row];
        }
        using Loc = std::decay_t<decltype(loc)>;
        const int64_t t0 = t * ROWS * kTile;
        if (!pack) {
            grid.x *= st_parts<kStWave>();  // workgroups per row
            grid.z = ROWS;                  // state row
            hipLaunchKernelGGL((state_unpack_kernel<ROWS, Loc>), grid,
                               dim3(kStWave), 0, s, state_r + t0, rw, loc);
            return check_launch("state unpack kernel");
        }
        // the pack: tiles [x0, x0 + nx) of each row of the locator per launch
        const int64_t tiles = grid.x;
        for (int64_t x0 = 0; x0 < tiles; x0 += kOrderedLaunchTiles) {
            const int64_t nx = tiles - x0 < kOrderedLaunchTiles
                                   ? tiles - x0 : kOrderedLaunchTiles;
            if (every_row)
                hipLaunchKernelGGL(
                    (state_pack_kernel<ROWS, Loc, kStWave>),
                    dim3((unsigned)(nx * ROWS * st_parts<kStWave>()), grid.y),
                    dim3(kStWave), 0, s, rw, state_w + t0, x0, loc);
            else
                hipLaunchKernelGGL(
                    (state_pack_kernel<ROWS, Loc, kStWide>),
                    dim3((unsigned)(nx * ROWS * st_parts<kStWide>()), grid.y),
                    dim3(kStWide), 0, s, rw, state_w + t0, x0, loc);
            const int rc = check_launch("state pack kernel");
            if (rc) return rc;
        }
        return (int)ZS_OK;
    });
}

bool all_aligned16(std::initializer_list<const void*> ps)
{
    for (const void* p : ps)
        if (p && !aligned16(p))
            return false;
    return true;
}

}  // namespace

extern "C" int zs_state_pack(const zs_layout* L, const float* master,
                             const float* m, const float* v, float* state,
                             void* hip_stream)
{
    using zs::fail;
    zs::clear_error();
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    if (L->shard_numel == 0) return ZS_OK;
    if (!master || !state)
        return fail(ZS_EINVAL, "master and state must be non-NULL");
    if (!all_aligned16({master, m, v, state}))
        return fail(ZS_EALIGN, "device pointers must be 16-byte aligned");
    const float* in[3] = {master, m, v};
    return convert_state<3>(L, true, in, nullptr, state, nullptr,
                            hip_stream);
}

extern "C" int zs_state_unpack(const zs_layout* L, const float* state,
                               float* master, float* m, float* v,
                               void* hip_stream)
{
    using zs::fail;
    zs::clear_error();
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    if (L->shard_numel == 0) return ZS_OK;
    if (!state) return fail(ZS_EINVAL, "state is NULL");
    if (!all_aligned16({state, master, m, v}))
        return fail(ZS_EALIGN, "device pointers must be 16-byte aligned");
    if (!master && !m && !v) return ZS_OK;
    float* out[3] = {master, m, v};
    return convert_state<3>(L, false, nullptr, out, nullptr, state,
                            hip_stream);
}

extern "C" int zs_state_mv_pack(const zs_layout* L, const float* m,
                                const float* v, float* state_mv,
                                void* hip_stream)
{
    using zs::fail;
    zs::clear_error();
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    if (L->shard_numel == 0) return ZS_OK;
    if (!state_mv) return fail(ZS_EINVAL, "state_mv is NULL");
    if (!all_aligned16({m, v, state_mv}))
        return fail(ZS_EALIGN, "device pointers must be 16-byte aligned");
    const float* in[3] = {m, v, nullptr};
    return convert_state<2>(L, true, in, nullptr, state_mv, nullptr,
                            hip_stream);
}

extern "C" int zs_state_mv_unpack(const zs_layout* L, const float* state_mv,
                                  float* m, float* v, void* hip_stream)
{
    using zs::fail;
    zs::clear_error();
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    if (L->shard_numel == 0) return ZS_OK;
    if (!state_mv) return fail(ZS_EINVAL, "state_mv is NULL");
    if (!all_aligned16({state_mv, m, v}))
        return fail(ZS_EALIGN, "device pointers must be 16-byte aligned");
    if (!m && !v) return ZS_OK;
    float* out[3] = {m, v, nullptr};
    return convert_state<2>(L, false, nullptr, out, nullptr, state_mv,
                            hip_stream);
}

extern "C" int zs_step_bf16(const zs_layout* L, const uint16_t* grads,
                            int32_t grad_layout, int64_t grad_stride,
                            float* state_mv, uint16_t* params,
                            int32_t params_flat, const zs_adamw* hp,
                            int64_t step, void* hip_stream)
{
    using zs::fail;
    zs::clear_error();
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    if (!hp) return fail(ZS_EINVAL, "hp is NULL");
    if (step < 1) return fail(ZS_EINVAL, "step %lld < 1", (long long)step);
    if (params_flat != 0 && params_flat != 1)
        return fail(ZS_EINVAL, "params_flat must be 0 or 1");
    if (L->shard_numel == 0)
        return ZS_OK;
    uint16_t* pshard = params_flat ? nullptr : params;
    uint16_t* flat = params_flat ? params : nullptr;
    int rc = check_step_args(L, grads, grad_layout, grad_stride,
                             L->shard_numel, state_mv, pshard, flat, hp,
                             step);
    if (rc) return rc;
    return shard_step<true>(L, grads, grad_layout == ZS_GRADS_TILED,
                            grad_stride, state_mv, pshard, flat,
                            make_consts(*hp, step, L->world),
                            static_cast<hipStream_t>(hip_stream));
}

extern "C" int zs_grads_tile(const zs_layout* L, int32_t bucket_id,
                             const uint16_t* slices, int64_t stride,
                             uint16_t* tiled, void* hip_stream)
{
    using zs::fail;
    zs::clear_error();
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    if (bucket_id >= (int32_t)L->buckets.size())
        return fail(ZS_ERANGE, "bucket_id %d outside [0, %d)", bucket_id,
                    (int)L->buckets.size());
    if (L->shard_numel == 0) return ZS_OK;
    if (!slices || !tiled)
        return fail(ZS_EINVAL, "slices and tiled must be non-NULL");
    if (!aligned16(slices) || !aligned16(tiled))
        return fail(ZS_EALIGN, "device pointers must be 16-byte aligned");
    if (stride % 8)
        return fail(ZS_EALIGN, "stride %lld is not a multiple of 8",
                    (long long)stride);
    const int32_t W = L->world;
    const int64_t len = bucket_id < 0 ? L->shard_numel
                                      : L->buckets[bucket_id].slice_numel;
    if (stride < len)
        return fail(ZS_ERANGE, "stride %lld < %lld elements per slice",
                    (long long)stride, (long long)len);
    if (stride > INT64_MAX / 2 / W)
        return fail(ZS_ERANGE, "W * stride overflows");
    // tiles per launch: at most kGtLaunchTiles, and fewer than 2^32
    // work-items along x
    const int64_t per_tile = (int64_t)W * kGtParts * kGtThreads;
    int64_t chunk = (((int64_t)1 << 32) - 1) / per_tile;
    if (chunk > kGtLaunchTiles) chunk = kGtLaunchTiles;
    if (chunk < 1)
        return fail(ZS_ERANGE, "world %d too large for the tiling launch", W);
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    // launches over tiles [x0, x0 + nx) of each row of the locator
    auto launch = [&](const auto& loc, int64_t tiles, unsigned rows,
                      const uint16_t* src, uint16_t* dst) {
        using Loc = std::decay_t<decltype(loc)>;
        for (int64_t x0 = 0; x0 < tiles; x0 += chunk) {
            const int64_t nx = tiles - x0 < chunk ? tiles - x0 : chunk;
            hipLaunchKernelGGL(grads_tile_kernel<Loc>,
                               dim3((unsigned)(nx * W * kGtParts), rows),
                               dim3(kGtThreads), 0, s, src, stride, dst, W,
                               x0, loc);
            const int rc = check_launch("grads tile kernel");
            if (rc) return rc;
        }
        return (int)ZS_OK;
    };
    if (bucket_id >= 0) {
        // one bucket's staging: positions relative to the bucket
        GeomLoc loc;
        loc.g = bucket_geom(L, L->buckets[bucket_id]);
        return launch(loc, loc.g.TPB, 1u, slices, tiled);
    }
    return for_launches(L, [&](const auto& loc, dim3 grid, int64_t e,
                               int64_t t, int64_t) {
        return launch(loc, (int64_t)grid.x, grid.y, slices + e,
                      tiled + t * W * kTile);
    });
}

namespace {

// The two launches of the pack: the flat all-gather buffer, and every chunk
// of the chunk table `chunks` (device memory) into the tensors of the
// device pointer array `tensors`.
int launch_pack_flat(const zs_layout* L, const uint16_t* param_shard,
                     uint16_t* full_flat, hipStream_t s)
{
    return for_launches(L, [&](const auto& loc, dim3 grid, int64_t e,
                               int64_t, int64_t f) {
        using Loc = std::decay_t<decltype(loc)>;
        grid.x *= kPackP;
        hipLaunchKernelGGL(pack_flat_kernel<Loc>, grid, dim3(kPackNT), 0, s,
                           param_shard + e, full_flat + f, loc);
        return check_launch("pack flat kernel");
    });
}

int launch_pack_chunks(const zs_layout* L, const uint16_t* param_shard,
                       const zs_chunk* chunks, uint16_t* const* tensors,
                       hipStream_t s)
{
    const int32_t n_chunks = (int32_t)L->chunks.size();
    int64_t longest = 0;
    for (const zs_chunk& c : L->chunks)
        longest = c.numel > longest ? c.numel : longest;
    int64_t gx = (longest + kPackTile - 1) / kPackTile;
    if (gx > kPackGridX) gx = kPackGridX;
    for (int32_t c0 = 0; c0 < n_chunks; c0 += (int32_t)kMaxGridY) {
        const int32_t ny = n_chunks - c0 < kMaxGridY ? n_chunks - c0
                                                     : (int32_t)kMaxGridY;
        hipLaunchKernelGGL(pack_chunks_kernel,
                           dim3((unsigned)gx, (unsigned)ny),
                           dim3(kPackThreads), 0, s, param_shard, chunks, c0,
                           tensors);
        const int rc = check_launch("pack chunks kernel");
        if (rc) return rc;
    }
    return ZS_OK;
}

}  // namespace

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
        const int rc = launch_pack_flat(L, param_shard, full_flat, s);
        if (rc) return rc;
    }
    if (chunk_mode && n_chunks > 0)
        return launch_pack_chunks(L, param_shard, dev_chunks,
                                  dev_tensor_ptrs, s);
    return ZS_OK;
}

// ---- the pack with library-held staging (zs_pack_noalloc) -------------------
//
// zs_pack's per-tensor path reads the chunk table and the tensor pointer
// array from device memory that its caller allocates and uploads.
// zs_pack_noalloc stages both in `scratch`, a file-scope device array that
// every call on a device shares (it holds the last call's tables until the
// process ends; nothing in it needs to start at zero).  The array's name in
// host code is a host-side stand-in, not a device address: the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and only that address is used (copy destinations, kernel
// arguments).

constexpr int64_t kNoallocChunkBytes =
    (int64_t)ZS_PACK_NOALLOC_MAX_CHUNKS * (int64_t)sizeof(zs_chunk);
constexpr int64_t kNoallocBytes =
    kNoallocChunkBytes + (int64_t)ZS_PACK_NOALLOC_MAX_TENSORS * 8;
static_assert(kNoallocChunkBytes % 256 == 0, "pointer table alignment");

static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch[kScratchDevices] = {};

// The device address of `scratch` on `dev`, which must be the current
// device; looked up on the first call for that device.
int scratch_on(int dev, unsigned char** out)
{
    using zs::fail;
    if (dev < 0 || dev >= kScratchDevices)
        return fail(ZS_EDEVICE, "device %d beyond the %d this library tracks",
                    dev, kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(ZS_EDEVICE, "hipGetSymbolAddress(scratch): %s",
                        hipGetErrorString(e));
        g_scratch[dev] = static_cast<unsigned char*>(p);
    }
    *out = g_scratch[dev];
    return ZS_OK;
}

}  // namespace

extern "C" int32_t zs_set_residency_cap(int32_t on)
{
    return g_cap_on.exchange(on ? 1 : 0);
}

extern "C" int zs_pack_noalloc(const zs_layout* L,
                               const uint16_t* param_shard,
                               uint16_t* full_flat,
                               uint16_t* const* tensor_ptrs,
                               int32_t n_tensors, void* hip_stream)
{
    using zs::fail;
    zs::clear_error();
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    const int64_t n_chunks = (int64_t)L->chunks.size();
    const int64_t layout_tensors = (int64_t)L->tensor_numel.size();
    // the limits first: nothing is touched for a layout beyond them
    if (n_chunks > ZS_PACK_NOALLOC_MAX_CHUNKS)
        return fail(ZS_ERANGE, "%lld chunks above the %d the static staging "
                    "holds", (long long)n_chunks, ZS_PACK_NOALLOC_MAX_CHUNKS);
    if (layout_tensors > ZS_PACK_NOALLOC_MAX_TENSORS)
        return fail(ZS_ERANGE, "%lld tensors above the %d the static "
                    "staging holds", (long long)layout_tensors,
                    ZS_PACK_NOALLOC_MAX_TENSORS);
    if (!tensor_ptrs && !full_flat)
        return fail(ZS_EINVAL, "no destination: full_flat or tensor_ptrs");
    if (tensor_ptrs && n_tensors != layout_tensors)
        return fail(ZS_EINVAL, "n_tensors %d != layout's %lld", n_tensors,
                    (long long)layout_tensors);
    if (tensor_ptrs)
        for (const zs_chunk& c : L->chunks)
            if (!tensor_ptrs[c.tensor_id])
                return fail(ZS_EINVAL, "tensor_ptrs[%d] is NULL",
                            c.tensor_id);
    if (L->shard_numel == 0)
        return ZS_OK;
    if (!param_shard) return fail(ZS_EINVAL, "param_shard is NULL");
    if (!aligned16(param_shard) || (full_flat && !aligned16(full_flat)))
        return fail(ZS_EALIGN, "param_shard/full_flat not 16-byte aligned");
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);

    if (full_flat) {
        const int rc = launch_pack_flat(L, param_shard, full_flat, s);
        if (rc) return rc;
    }
    if (!tensor_ptrs || n_chunks == 0)
        return ZS_OK;
    // the staging lives on the stream's device, which must be current
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return fail(ZS_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (s) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(s, &sd);
        if (e != hipSuccess)
            return fail(ZS_EDEVICE, "hipStreamGetDevice: %s",
                        hipGetErrorString(e));
        if ((int)sd != cur)
            return fail(ZS_EINVAL, "the stream belongs to device %d, the "
                        "current device is %d", (int)sd, cur);
    }
    unsigned char* base = nullptr;
    const int rc = scratch_on(cur, &base);
    if (rc) return rc;
    zs_chunk* dchunks = reinterpret_cast<zs_chunk*>(base);
    uint16_t** dptrs =
        reinterpret_cast<uint16_t**>(base + kNoallocChunkBytes);
    // copies from the caller's host memory, in stream order after the work
    // already queued (an earlier call's kernels may still read the staging)
    e = hipMemcpyAsync(dchunks, L->chunks.data(),
                       (size_t)n_chunks * sizeof(zs_chunk),
                       hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(dptrs, tensor_ptrs,
                           (size_t)n_tensors * sizeof(uint16_t*),
                           hipMemcpyHostToDevice, s);
    if (e != hipSuccess)
        return fail(ZS_EDEVICE, "staging the tables: %s",
                    hipGetErrorString(e));
    return launch_pack_chunks(L, param_shard, dchunks, dptrs, s);
}
