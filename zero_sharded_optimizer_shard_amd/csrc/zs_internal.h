// Internal definitions shared by the host layout builder and the device
// launchers of libzs.  Not part of the public interface (include/zs.h).
#pragma once

#include <cstdarg>
#include <cstdint>
#include <vector>

#include "zs.h"

struct zs_layout {
    int32_t world = 1;
    int32_t rank = 0;
    int64_t align_elems = 128;
    int64_t bucket_elems = 0;   // numel of a full bucket
    int64_t flat_numel = 0;
    int64_t shard_numel = 0;
    int64_t n_tiles = 0;        // tiles of the shard in the tiled layouts
    std::vector<int64_t> tensor_numel;
    std::vector<int64_t> tensor_off;
    std::vector<zs_bucket> buckets;
    std::vector<zs_chunk> chunks;
    // whole-tensor mode: every tensor belongs to one rank; each owned tensor
    // is one bucket whose whole extent is this rank's slice
    bool whole_tensors = false;
    std::vector<int32_t> owner;            // per tensor
    std::vector<int64_t> owner_shard_off;  // per tensor, in the owner's shard
};

// Most tiles one kernel launch covers: the step's work shapes put up to
// 2048 threads per tile along x (32 one-wave workgroups, or 16 of 128
// threads), and HIP allows fewer than 2^32 work-items there.  A bucket
// slice (a whole tensor in the whole-tensor mode) is at most this many
// tiles, 17.2 G elements; group launches end a group early rather than pass
// it.
constexpr int64_t kMaxLaunchTiles = (int64_t(1) << 21) - 1;

// Flat position of this rank's slice of bucket b.
inline int64_t slice_flat_pos(const zs_layout* L, const zs_bucket& b)
{
    return b.flat_off + (L->whole_tensors ? 0 : (int64_t)L->rank *
                                                    b.slice_numel);
}

namespace zs {

// Record a failure text for zs_last_error() and return `code`.
int fail(int code, const char* fmt, ...);
// Clear the calling thread's failure text.
void clear_error();

}  // namespace zs
