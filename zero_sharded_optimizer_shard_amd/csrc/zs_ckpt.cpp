// Checkpoint and resume of one rank's optimizer state.
//
// The state of a ZeRO rank is its slice of the master weights and Adam
// moments; it is only meaningful under the layout that cut the parameters
// into slices, so the file carries the layout's fingerprint and a restore
// under any other layout is refused before the state is touched (the
// DDP-to-ZeRO blog, section 3.3, on ZeRO checkpoints that cannot be used
// without the right gathering step).
//
// Data path: device state <-> two pinned host staging buffers <-> file.
// While one buffer's piece is being written to (or read from) the file, the
// other buffer's device copy runs on the caller's stream, so the transfer
// over the host link overlaps the file I/O.  The library allocates no
// device memory; the pinned staging lives for the duration of one call.

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include <unistd.h>

#include "zs_internal.h"

namespace {

using zs::fail;

constexpr char kMagic[8] = {'Z', 'S', 'C', 'K', 'P', 'T', '0', '1'};
constexpr uint32_t kVersion = 1;
constexpr size_t kPiece = size_t(64) << 20;     // bytes per staging buffer
constexpr uint64_t kBasis = 0xcbf29ce484222325ull;
constexpr uint64_t kPrime = 0x100000001b3ull;

struct Header {
    char magic[8];
    uint32_t version;
    uint32_t rows;
    uint64_t fingerprint;
    int64_t step;
    int64_t n_tiles;
    int64_t shard_numel;
    int32_t world;
    int32_t rank;
    uint64_t payload;           // bytes of tiled state that follow
};
static_assert(sizeof(Header) == 64, "the header is 64 bytes on disk");

// payload checksum: FNV-1a's mixing step over 64-bit words
uint64_t mix_words(uint64_t h, const void* p, size_t bytes)
{
    const unsigned char* b = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < bytes; i += 8) {
        uint64_t w;
        std::memcpy(&w, b + i, 8);
        h = (h ^ w) * kPrime;
    }
    return h;
}

int hip_fail(hipError_t e, const char* what)
{
    return fail(ZS_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Two pinned staging buffers and an event per buffer: the event marks the
// end of the last device copy that used the buffer.
struct Staging {
    hipStream_t stream;
    void* buf[2] = {nullptr, nullptr};
    hipEvent_t ev[2] = {nullptr, nullptr};

    explicit Staging(hipStream_t s) : stream(s) {}

    int init()
    {
        for (int i = 0; i < 2; ++i) {
            hipError_t e = hipHostMalloc(&buf[i], kPiece, hipHostMallocDefault);
            if (e != hipSuccess) {
                buf[i] = nullptr;
                return fail(ZS_ENOMEM, "hipHostMalloc of %zu bytes: %s",
                            kPiece, hipGetErrorString(e));
            }
            e = hipEventCreateWithFlags(&ev[i], hipEventDisableTiming);
            if (e != hipSuccess) {
                ev[i] = nullptr;
                return hip_fail(e, "hipEventCreateWithFlags");
            }
        }
        return ZS_OK;
    }

    ~Staging()
    {
        // after an error a copy may still be in flight: drain the stream
        // before the buffers go back
        if (buf[0] || buf[1])
            (void)hipStreamSynchronize(stream);
        for (int i = 0; i < 2; ++i) {
            if (ev[i]) (void)hipEventDestroy(ev[i]);
            if (buf[i]) (void)hipHostFree(buf[i]);
        }
    }
};

int check_common(const zs_layout* L, const char* path, const void* state,
                 int32_t rows)
{
    if (!L || !path || !state)
        return fail(ZS_EINVAL, "layout, path and state must be non-NULL");
    if (rows != 2 && rows != 3)
        return fail(ZS_EINVAL, "rows %d is not 2 or 3", rows);
    if (reinterpret_cast<uintptr_t>(state) & 15u)
        return fail(ZS_EALIGN, "state not 16-byte aligned");
    return ZS_OK;
}

uint64_t payload_bytes(const zs_layout* L, int32_t rows)
{
    return (uint64_t)L->n_tiles * (uint64_t)rows * ZS_TILE * sizeof(float);
}

}  // namespace

extern "C" int zs_checkpoint_save(const zs_layout* L, const char* path,
                                  const float* state, int32_t rows,
                                  int64_t step, void* hip_stream)
{
    zs::clear_error();
    int rc = check_common(L, path, state, rows);
    if (rc) return rc;
    if (step < 0) return fail(ZS_EINVAL, "step %lld < 0", (long long)step);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);

    Header h{};
    std::memcpy(h.magic, kMagic, 8);
    h.version = kVersion;
    h.rows = (uint32_t)rows;
    (void)zs_layout_fingerprint(L, &h.fingerprint);
    h.step = step;
    h.n_tiles = L->n_tiles;
    h.shard_numel = L->shard_numel;
    h.world = L->world;
    h.rank = L->rank;
    h.payload = payload_bytes(L, rows);

    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    Staging st(s);
    if ((rc = st.init())) return rc;

    std::string tmp;
    try {
        tmp = std::string(path) + ".tmp";
    } catch (...) {
        return fail(ZS_ENOMEM, "host allocation");
    }
    FILE* f = std::fopen(tmp.c_str(), "wb");
    if (!f) return fail(ZS_EIO, "cannot create %s", tmp.c_str());
    auto abandon = [&](int code) {
        std::fclose(f);
        std::remove(tmp.c_str());
        return code;
    };
    if (std::fwrite(&h, sizeof h, 1, f) != 1)
        return abandon(fail(ZS_EIO, "write to %s failed", tmp.c_str()));

    // copy piece i into buffer i % 2 while piece i - 1 goes to the file
    const char* src = reinterpret_cast<const char*>(state);
    const uint64_t total = h.payload;
    const uint64_t n_pieces = (total + kPiece - 1) / kPiece;
    uint64_t sum = kBasis;
    for (uint64_t i = 0; i <= n_pieces; ++i) {
        if (i < n_pieces) {
            const uint64_t off = i * kPiece;
            const size_t len = (size_t)(total - off < kPiece ? total - off
                                                             : kPiece);
            e = hipMemcpyAsync(st.buf[i % 2], src + off, len,
                               hipMemcpyDeviceToHost, s);
            if (e == hipSuccess) e = hipEventRecord(st.ev[i % 2], s);
            if (e != hipSuccess)
                return abandon(hip_fail(e, "device-to-host copy"));
        }
        if (i > 0) {
            const uint64_t j = i - 1;
            const uint64_t off = j * kPiece;
            const size_t len = (size_t)(total - off < kPiece ? total - off
                                                             : kPiece);
            e = hipEventSynchronize(st.ev[j % 2]);
            if (e != hipSuccess)
                return abandon(hip_fail(e, "hipEventSynchronize"));
            sum = mix_words(sum, st.buf[j % 2], len);
            if (std::fwrite(st.buf[j % 2], 1, len, f) != len)
                return abandon(fail(ZS_EIO, "write to %s failed",
                                    tmp.c_str()));
        }
    }
    if (std::fwrite(&sum, sizeof sum, 1, f) != 1 || std::fflush(f) != 0 ||
        fsync(fileno(f)) != 0)
        return abandon(fail(ZS_EIO, "write to %s failed", tmp.c_str()));
    if (std::fclose(f) != 0) {
        std::remove(tmp.c_str());
        return fail(ZS_EIO, "closing %s failed", tmp.c_str());
    }
    if (std::rename(tmp.c_str(), path) != 0) {
        std::remove(tmp.c_str());
        return fail(ZS_EIO, "cannot rename %s to %s", tmp.c_str(), path);
    }
    return ZS_OK;
}

extern "C" int zs_checkpoint_load(const zs_layout* L, const char* path,
                                  float* state, int32_t rows, int64_t* step,
                                  void* hip_stream)
{
    zs::clear_error();
    int rc = check_common(L, path, state, rows);
    if (rc) return rc;
    if (!step) return fail(ZS_EINVAL, "step is NULL");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);

    FILE* f = std::fopen(path, "rb");
    if (!f) return fail(ZS_EIO, "cannot open %s", path);
    auto close_with = [&](int code) {
        std::fclose(f);
        return code;
    };
    Header h;
    if (std::fread(&h, sizeof h, 1, f) != 1)
        return close_with(fail(ZS_EIO, "%s: shorter than a checkpoint "
                               "header", path));
    if (std::memcmp(h.magic, kMagic, 8) != 0 || h.version != kVersion)
        return close_with(fail(ZS_EIO, "%s is not a checkpoint of this "
                               "format", path));
    uint64_t fp = 0;
    (void)zs_layout_fingerprint(L, &fp);
    if (h.fingerprint != fp || h.world != L->world || h.rank != L->rank ||
        h.n_tiles != L->n_tiles || h.shard_numel != L->shard_numel)
        return close_with(fail(ZS_EMISMATCH, "%s was written for another "
                               "layout (world %d, rank %d, %lld tiles; this "
                               "layout: world %d, rank %d, %lld tiles)",
                               path, h.world, h.rank, (long long)h.n_tiles,
                               L->world, L->rank, (long long)L->n_tiles));
    if (h.rows != (uint32_t)rows)
        return close_with(fail(ZS_EMISMATCH, "%s holds %u state rows, not "
                               "%d", path, h.rows, rows));
    if (h.payload != payload_bytes(L, rows) || h.step < 0)
        return close_with(fail(ZS_EIO, "%s: inconsistent header", path));

    Staging st(s);
    if ((rc = st.init())) return close_with(rc);
    // read piece i into buffer i % 2 once the copy that last used it is
    // done, then copy it to the device
    char* dst = reinterpret_cast<char*>(state);
    const uint64_t total = h.payload;
    uint64_t sum = kBasis;
    hipError_t e;
    for (uint64_t off = 0, i = 0; off < total; off += kPiece, ++i) {
        const size_t len = (size_t)(total - off < kPiece ? total - off
                                                         : kPiece);
        e = hipEventSynchronize(st.ev[i % 2]);
        if (e != hipSuccess)
            return close_with(hip_fail(e, "hipEventSynchronize"));
        if (std::fread(st.buf[i % 2], 1, len, f) != len)
            return close_with(fail(ZS_EIO, "%s: truncated payload", path));
        sum = mix_words(sum, st.buf[i % 2], len);
        e = hipMemcpyAsync(dst + off, st.buf[i % 2], len,
                           hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipEventRecord(st.ev[i % 2], s);
        if (e != hipSuccess)
            return close_with(hip_fail(e, "host-to-device copy"));
    }
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return close_with(hip_fail(e, "hipStreamSynchronize"));
    uint64_t want = 0;
    if (std::fread(&want, sizeof want, 1, f) != 1)
        return close_with(fail(ZS_EIO, "%s: no checksum", path));
    if (std::fgetc(f) != EOF)
        return close_with(fail(ZS_EIO, "%s: bytes after the checksum", path));
    std::fclose(f);
    if (want != sum)
        return fail(ZS_EIO, "%s: payload checksum mismatch", path);
    *step = h.step;
    return ZS_OK;
}
