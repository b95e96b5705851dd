// Device-side helpers shared by the HIP sources of libzs (gfx950 only).
// Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace zsdev {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a gfx9-family buffer descriptor for raw (untyped) access:
// DATA_FORMAT = 32 bits (bits 18:15 = 4), everything else zero.
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy bits of gfx940-family vector memory instructions.
constexpr int kCpolSc0 = 1, kCpolNt = 2, kCpolSc1 = 16;
// Streamed outputs: non-temporal with system scope (sc0 sc1 nt), so the L2
// passes the written lines on to HBM instead of holding them dirty until
// eviction.  Measured on MI355X, it pays in a stream that reads twice what
// it writes: the 8B-shaped W = 8 optimizer step at 82.0-82.2 % of peak HBM
// bandwidth against 80.4 % with plain non-temporal stores, with the same
// HBM bytes.  For 1 : 1 copies it depends on the form: the one-wave packs
// gain (flat pack 84.7-85.0 % against 83.2-83.4 %, per-tensor pack 84.5 %
// against 83.1 %), and so does the ZeRO-3 gather with one copy per thread
// (82.6-82.7 % against 81.9-82.0 %); the one-wave gradient accumulation
// measured level (84.1-84.2 % per cycle) and keeps plain non-temporal
// stores.  In their earlier 256- and 512-thread forms all the copies lost
// by it.
constexpr int kStreamOut = kCpolSc0 | kCpolSc1 | kCpolNt;

// Store x (4, 8 or 16 bytes) at byte offset `off` of the output region
// [base, base + bytes).  base is wave-uniform (it becomes the scalar base of
// a buffer descriptor); the hardware drops a store outside the region.
template <class T>
__device__ __forceinline__ void stream_store(void* base, uint32_t bytes,
                                             uint32_t off, T x)
{
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, kRsrcWord3);
    if constexpr (sizeof(T) == 16)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x),
                                               r, (int)off, 0, kStreamOut);
    else if constexpr (sizeof(T) == 8)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x),
                                              r, (int)off, 0, kStreamOut);
    else {
        static_assert(sizeof(T) == 4, "4, 8 or 16 bytes");
        __builtin_amdgcn_raw_buffer_store_b32(
            __builtin_bit_cast(uint32_t, x), r, (int)off, 0, kStreamOut);
    }
}

}  // namespace zsdev
