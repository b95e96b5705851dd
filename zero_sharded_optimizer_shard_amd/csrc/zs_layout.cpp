// Host-side layout builder: flat buffer, fixed-size buckets, this rank's
// slices and its chunk table.  The rule is stated with zs_layout_build in
// include/zs.h; it follows the flattened, bucketed gradient buffer of the
// pages (podcast summary of "Training at thousands of GPUs", sections "Data
// parallelism" and "ZeRO optimizer"; DDP-to-ZeRO blog sections 2.1 and 3.3)
// and the reduce-scatter ownership of the CS336 lecture 8 ZeRO-1 example.

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <limits>
#include <new>
#include <string>

#include "zs_internal.h"

namespace zs {

static thread_local std::string g_err;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

void clear_error() { g_err.clear(); }

const char* last_error() { return g_err.c_str(); }

}  // namespace zs

namespace {

constexpr int64_t kMax = std::numeric_limits<int64_t>::max();

// a + b without overflow, false if it would overflow (a, b >= 0)
bool add_ok(int64_t a, int64_t b, int64_t* r)
{
    if (a > kMax - b) return false;
    *r = a + b;
    return true;
}

// round x up to a multiple of a (x >= 0, a > 0), false on overflow
bool roundup_ok(int64_t x, int64_t a, int64_t* r)
{
    int64_t t;
    if (!add_ok(x, a - 1, &t)) return false;
    *r = (t / a) * a;
    return true;
}

}  // namespace

extern "C" int zs_layout_build(const int64_t* tensor_numel, int32_t n_tensors,
                               int32_t world, int32_t rank,
                               int64_t bucket_cap_bytes, int32_t align_bytes,
                               zs_layout** out)
{
    using zs::fail;
    zs::clear_error();
    if (!out) return fail(ZS_EINVAL, "out is NULL");
    *out = nullptr;
    if (n_tensors < 0) return fail(ZS_EINVAL, "n_tensors < 0");
    if (n_tensors > 0 && !tensor_numel)
        return fail(ZS_EINVAL, "tensor_numel is NULL");
    if (world < 1) return fail(ZS_EINVAL, "world %d < 1", world);
    if (rank < 0 || rank >= world)
        return fail(ZS_EINVAL, "rank %d outside [0, %d)", rank, world);
    if (align_bytes < 16 || align_bytes % 16)
        return fail(ZS_EINVAL, "align_bytes %d is not a positive multiple "
                    "of 16", align_bytes);

    zs_layout* L = new (std::nothrow) zs_layout;
    if (!L) return fail(ZS_ENOMEM, "host allocation");
    try {
        L->world = world;
        L->rank = rank;
        L->align_elems = align_bytes / 2;
        const int64_t A = L->align_elems;

        // 1. tensor starts
        L->tensor_numel.assign(tensor_numel, tensor_numel + n_tensors);
        L->tensor_off.resize(n_tensors);
        int64_t pos = 0;
        for (int32_t k = 0; k < n_tensors; ++k) {
            int64_t n = tensor_numel[k];
            if (n < 0) {
                delete L;
                return fail(ZS_EINVAL, "tensor %d has numel %lld < 0", k,
                            (long long)n);
            }
            int64_t start, end;
            if (!roundup_ok(pos, A, &start) || !add_ok(start, n, &end)) {
                delete L;
                return fail(ZS_ERANGE, "flat size overflows int64");
            }
            L->tensor_off[k] = start;
            pos = end;
        }
        const int64_t content_end = pos;

        // 2. full bucket size
        if ((int64_t)world > kMax / A) {
            delete L;
            return fail(ZS_ERANGE, "world * align overflows");
        }
        const int64_t unit = (int64_t)world * A;
        int64_t full;
        if (bucket_cap_bytes <= 0) {
            if (!roundup_ok(content_end, unit, &full)) {
                delete L;
                return fail(ZS_ERANGE, "flat size overflows int64");
            }
            if (full == 0) full = unit;
        } else {
            full = ((bucket_cap_bytes / 2) / unit) * unit;
            if (full == 0) {
                delete L;
                return fail(ZS_EINVAL, "bucket_cap_bytes %lld below one "
                            "aligned slice per rank (%lld bytes)",
                            (long long)bucket_cap_bytes,
                            (long long)(unit * 2));
            }
        }
        L->bucket_elems = full;

        // 3. buckets, and where each slice's tiles start in the tiled
        //    layouts
        int64_t off = 0, shard = 0, tiles = 0;
        while (off < content_end) {
            int64_t rest;
            if (!roundup_ok(content_end - off, unit, &rest)) {
                delete L;
                return fail(ZS_ERANGE, "flat size overflows int64");
            }
            zs_bucket b;
            b.flat_off = off;
            b.numel = rest < full ? rest : full;
            b.slice_numel = b.numel / world;
            if ((b.slice_numel + ZS_TILE - 1) / ZS_TILE > kMaxLaunchTiles) {
                delete L;
                return fail(ZS_ERANGE, "bucket slice of %lld elements above "
                            "%lld tiles", (long long)b.slice_numel,
                            (long long)kMaxLaunchTiles);
            }
            b.shard_off = shard;
            b.tile_off = tiles;
            L->buckets.push_back(b);
            off += b.numel;
            shard += b.slice_numel;
            tiles += (b.slice_numel + ZS_TILE - 1) / ZS_TILE;
        }
        if ((int64_t)L->buckets.size() > std::numeric_limits<int32_t>::max()) {
            delete L;
            return fail(ZS_ERANGE, "more than 2^31-1 buckets");
        }
        L->flat_numel = off;
        L->shard_numel = shard;
        L->n_tiles = tiles;

        // 4. chunks: sweep tensors and this rank's slices together.  `first`
        //    is the first tensor that ends after the current slice start;
        //    slice starts increase with the bucket index.
        int32_t first = 0;
        for (int32_t b = 0; b < (int32_t)L->buckets.size(); ++b) {
            const zs_bucket& bk = L->buckets[b];
            const int64_t lo = bk.flat_off + (int64_t)rank * bk.slice_numel;
            const int64_t hi = lo + bk.slice_numel;
            while (first < n_tensors &&
                   L->tensor_off[first] + L->tensor_numel[first] <= lo)
                ++first;
            for (int32_t k = first; k < n_tensors && L->tensor_off[k] < hi;
                 ++k) {
                const int64_t t0 = L->tensor_off[k];
                const int64_t s = lo > t0 ? lo : t0;
                const int64_t e0 = t0 + L->tensor_numel[k];
                const int64_t e = hi < e0 ? hi : e0;
                if (e <= s) continue;
                zs_chunk c;
                c.tensor_id = k;
                c.bucket_id = b;
                c.tensor_off = s - t0;
                c.numel = e - s;
                c.shard_off = bk.shard_off + (s - lo);
                L->chunks.push_back(c);
            }
        }
        if ((int64_t)L->chunks.size() > std::numeric_limits<int32_t>::max()) {
            delete L;
            return fail(ZS_ERANGE, "more than 2^31-1 chunks");
        }
    } catch (const std::bad_alloc&) {
        delete L;
        return fail(ZS_ENOMEM, "host allocation");
    }
    *out = L;
    return ZS_OK;
}

// Whole-tensor mode (the rule is stated with zs_layout_build_tensors in
// include/zs.h): longest-first greedy assignment of whole tensors to ranks.
extern "C" int zs_layout_build_tensors(const int64_t* tensor_numel,
                                       int32_t n_tensors, int32_t world,
                                       int32_t rank, int32_t align_bytes,
                                       zs_layout** out)
{
    using zs::fail;
    zs::clear_error();
    if (!out) return fail(ZS_EINVAL, "out is NULL");
    *out = nullptr;
    if (n_tensors < 0) return fail(ZS_EINVAL, "n_tensors < 0");
    if (n_tensors > 0 && !tensor_numel)
        return fail(ZS_EINVAL, "tensor_numel is NULL");
    if (world < 1) return fail(ZS_EINVAL, "world %d < 1", world);
    if (rank < 0 || rank >= world)
        return fail(ZS_EINVAL, "rank %d outside [0, %d)", rank, world);
    if (align_bytes < 16 || align_bytes % 16)
        return fail(ZS_EINVAL, "align_bytes %d is not a positive multiple "
                    "of 16", align_bytes);
    zs_layout* L = new (std::nothrow) zs_layout;
    if (!L) return fail(ZS_ENOMEM, "host allocation");
    try {
        L->world = world;
        L->rank = rank;
        L->whole_tensors = true;
        L->align_elems = align_bytes / 2;
        const int64_t A = L->align_elems;
        L->tensor_numel.assign(tensor_numel, tensor_numel + n_tensors);
        L->tensor_off.resize(n_tensors);
        std::vector<int64_t> padded(n_tensors);
        int64_t pos = 0;
        for (int32_t k = 0; k < n_tensors; ++k) {
            const int64_t n = tensor_numel[k];
            if (n < 0) {
                delete L;
                return fail(ZS_EINVAL, "tensor %d has numel %lld < 0", k,
                            (long long)n);
            }
            int64_t start, end;
            if (!roundup_ok(pos, A, &start) || !add_ok(start, n, &end) ||
                !roundup_ok(n, A, &padded[k])) {
                delete L;
                return fail(ZS_ERANGE, "flat size overflows int64");
            }
            L->tensor_off[k] = start;
            pos = end;
        }
        if (!roundup_ok(pos, A, &L->flat_numel)) {
            delete L;
            return fail(ZS_ERANGE, "flat size overflows int64");
        }
        // longest first (ties: lower index), each to the least-loaded rank
        // (ties: lower rank)
        std::vector<int32_t> order(n_tensors);
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(),
                         [&](int32_t a, int32_t b) {
                             return padded[a] > padded[b];
                         });
        std::vector<int64_t> load(world, 0);
        L->owner.assign(n_tensors, 0);
        for (int32_t t : order) {
            if ((padded[t] + ZS_TILE - 1) / ZS_TILE > kMaxLaunchTiles) {
                delete L;
                return fail(ZS_ERANGE, "tensor %d of %lld elements above "
                            "%lld tiles", t, (long long)padded[t],
                            (long long)kMaxLaunchTiles);
            }
            int32_t r = 0;
            for (int32_t q = 1; q < world; ++q)
                if (load[q] < load[r]) r = q;
            L->owner[t] = r;
            load[r] += padded[t];
        }
        std::vector<int64_t> fill(world, 0);
        L->owner_shard_off.assign(n_tensors, 0);
        int64_t tiles = 0;
        for (int32_t t = 0; t < n_tensors; ++t) {
            const int32_t r = L->owner[t];
            L->owner_shard_off[t] = fill[r];
            fill[r] += padded[t];
            if (r != rank || tensor_numel[t] == 0) continue;
            zs_bucket b;
            b.flat_off = L->tensor_off[t];
            b.numel = padded[t];
            b.slice_numel = padded[t];
            b.shard_off = L->owner_shard_off[t];
            b.tile_off = tiles;
            tiles += (padded[t] + ZS_TILE - 1) / ZS_TILE;
            zs_chunk c;
            c.tensor_id = t;
            c.bucket_id = (int32_t)L->buckets.size();
            c.tensor_off = 0;
            c.numel = tensor_numel[t];
            c.shard_off = b.shard_off;
            L->buckets.push_back(b);
            L->chunks.push_back(c);
        }
        L->shard_numel = fill[rank];
        L->n_tiles = tiles;
        L->bucket_elems = 0;
    } catch (const std::bad_alloc&) {
        delete L;
        return fail(ZS_ENOMEM, "host allocation");
    }
    *out = L;
    return ZS_OK;
}

extern "C" int zs_layout_owners(const zs_layout* L, int32_t* owner,
                                int64_t* owner_shard_off, int32_t cap)
{
    using zs::fail;
    zs::clear_error();
    if (!L) return fail(ZS_EINVAL, "layout is NULL");
    if (!L->whole_tensors)
        return fail(ZS_EINVAL, "not a whole-tensor layout");
    const int64_t n = (int64_t)L->owner.size();
    if (cap < 0 || (cap > 0 && (!owner || !owner_shard_off)))
        return fail(ZS_EINVAL, "bad output buffers");
    if (cap < n)
        return fail(ZS_ERANGE, "capacity %d < %lld tensors", cap,
                    (long long)n);
    if (n) {
        std::memcpy(owner, L->owner.data(), (size_t)n * sizeof(int32_t));
        std::memcpy(owner_shard_off, L->owner_shard_off.data(),
                    (size_t)n * sizeof(int64_t));
    }
    return (int)n;
}

extern "C" int zs_layout_info(const zs_layout* L, int64_t* flat_numel,
                              int64_t* shard_numel, int32_t* n_buckets,
                              int32_t* n_chunks)
{
    zs::clear_error();
    if (!L) return zs::fail(ZS_EINVAL, "layout is NULL");
    if (flat_numel) *flat_numel = L->flat_numel;
    if (shard_numel) *shard_numel = L->shard_numel;
    if (n_buckets) *n_buckets = (int32_t)L->buckets.size();
    if (n_chunks) *n_chunks = (int32_t)L->chunks.size();
    return ZS_OK;
}

extern "C" int zs_layout_tiles(const zs_layout* L, int64_t* n_tiles)
{
    zs::clear_error();
    if (!L) return zs::fail(ZS_EINVAL, "layout is NULL");
    if (n_tiles) *n_tiles = L->n_tiles;
    return ZS_OK;
}

template <class T>
static int copy_out(const std::vector<T>& v, T* out, int32_t cap,
                    const char* what)
{
    zs::clear_error();
    const int64_t n = (int64_t)v.size();
    if (cap < 0 || (cap > 0 && !out))
        return zs::fail(ZS_EINVAL, "%s: bad output buffer", what);
    if (cap < n)
        return zs::fail(ZS_ERANGE, "%s: capacity %d < %lld entries", what,
                        cap, (long long)n);
    if (n) std::memcpy(out, v.data(), (size_t)n * sizeof(T));
    return (int)n;
}

extern "C" int zs_layout_buckets(const zs_layout* L, zs_bucket* out,
                                 int32_t cap)
{
    if (!L) return zs::fail(ZS_EINVAL, "layout is NULL");
    return copy_out(L->buckets, out, cap, "buckets");
}

extern "C" int zs_layout_chunks(const zs_layout* L, zs_chunk* out, int32_t cap)
{
    if (!L) return zs::fail(ZS_EINVAL, "layout is NULL");
    return copy_out(L->chunks, out, cap, "chunks");
}

extern "C" int zs_layout_tensor_offsets(const zs_layout* L, int64_t* out,
                                        int32_t cap)
{
    if (!L) return zs::fail(ZS_EINVAL, "layout is NULL");
    return copy_out(L->tensor_off, out, cap, "tensor offsets");
}

extern "C" int zs_layout_rank(const zs_layout* L, int32_t* world,
                              int32_t* rank)
{
    zs::clear_error();
    if (!L) return zs::fail(ZS_EINVAL, "layout is NULL");
    if (world) *world = L->world;
    if (rank) *rank = L->rank;
    return ZS_OK;
}

extern "C" void zs_layout_free(zs_layout* L) { delete L; }

extern "C" int zs_layout_fingerprint(const zs_layout* L, uint64_t* out)
{
    using zs::fail;
    zs::clear_error();
    if (!L || !out) return fail(ZS_EINVAL, "layout or out is NULL");
    // FNV-1a, 64-bit, over little-endian int64 fields
    uint64_t h = 0xcbf29ce484222325ull;
    auto mix = [&h](int64_t v) {
        const uint64_t u = static_cast<uint64_t>(v);
        for (int i = 0; i < 8; ++i) {
            h ^= (u >> (8 * i)) & 0xffu;
            h *= 0x100000001b3ull;
        }
    };
    mix(L->whole_tensors ? 1 : 0);
    mix(L->world);
    mix(L->rank);
    mix(L->align_elems);
    mix(L->whole_tensors ? 0 : L->bucket_elems);
    mix((int64_t)L->tensor_numel.size());
    for (int64_t n : L->tensor_numel)
        mix(n);
    *out = h;
    return ZS_OK;
}

extern "C" const char* zs_strerror(int code)
{
    switch (code) {
    case ZS_OK: return "success";
    case ZS_EINVAL: return "invalid argument";
    case ZS_EALIGN: return "pointer or stride not 16-byte aligned";
    case ZS_ERANGE: return "index or size out of range";
    case ZS_ENOMEM: return "host allocation failed";
    case ZS_EDEVICE: return "HIP launch error";
    case ZS_EIO: return "checkpoint file cannot be read or written, or is "
                        "not a valid checkpoint";
    case ZS_EMISMATCH: return "checkpoint written for another layout";
    default: return "unknown error code";
    }
}

extern "C" const char* zs_last_error(void) { return zs::last_error(); }
