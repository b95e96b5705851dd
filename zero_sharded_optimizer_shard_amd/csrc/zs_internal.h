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
};

namespace zs {

// Record a failure text for zs_last_error() and return `code`.
int fail(int code, const char* fmt, ...);
// Clear the calling thread's failure text.
void clear_error();

}  // namespace zs
