"""One data-parallel rank's ZeRO-1/2 optimizer step on MI355X (gfx950).

The HIP library libzs.so (C-ABI in include/zs.h) does all the work; this
package is its ctypes binding, with the same names.
"""

from ._zs import (EXPORTS, LIB_PATH, ZS_ACC_ADD, ZS_ACC_FIRST, ZS_ACC_LAST,
                  ZS_EIO, ZS_EMISMATCH, zs_checkpoint_load,
                  zs_checkpoint_save, zs_layout_fingerprint,
                  ZS_GATHER_MAX_WORLD, ZS_GRADS_SLICES, ZS_GRADS_TILED,
                  ZS_MAX_GROUP, ZS_PACK_NOALLOC_MAX_CHUNKS,
                  ZS_PACK_NOALLOC_MAX_TENSORS, ZS_TILE, Layout, Prefetch,
                  Stream, ZsError,
                  chunks_bytes, lib, zs_accumulate, zs_adamw, zs_bucket,
                  zs_bucket_step, zs_buckets_step, zs_chunk, zs_gather,
                  zs_grads_tile, zs_last_error, zs_layout_buckets,
                  zs_layout_build, zs_layout_build_tensors, zs_layout_chunks,
                  zs_layout_info, zs_layout_owners, zs_layout_rank,
                  zs_layout_tensor_offsets, zs_layout_tiles, zs_pack,
                  zs_pack_noalloc, zs_prefetch_acquire, zs_prefetch_create,
                  zs_prefetch_free, zs_prefetch_issue, zs_prefetch_release, zs_state_mv_pack,
                  zs_state_mv_unpack, zs_state_pack, zs_state_unpack, zs_step,
                  zs_step_bf16, zs_step_plain, zs_stream_arrive, zs_stream_create,
                  zs_set_residency_cap, zs_stream_free, zs_stream_step_begin,
                  zs_stream_step_end, zs_strerror)

__all__ = ["EXPORTS", "LIB_PATH", "ZS_ACC_ADD", "ZS_ACC_FIRST", "ZS_ACC_LAST",
           "ZS_EIO", "ZS_EMISMATCH", "zs_checkpoint_load",
           "zs_checkpoint_save", "zs_layout_fingerprint",
           "ZS_GATHER_MAX_WORLD", "ZS_GRADS_SLICES", "ZS_GRADS_TILED",
           "ZS_MAX_GROUP", "ZS_PACK_NOALLOC_MAX_CHUNKS",
           "ZS_PACK_NOALLOC_MAX_TENSORS", "ZS_TILE", "Layout", "Prefetch",
           "Stream",
           "ZsError", "chunks_bytes", "lib", "zs_accumulate", "zs_adamw",
           "zs_bucket", "zs_bucket_step", "zs_buckets_step", "zs_chunk",
           "zs_gather", "zs_grads_tile", "zs_last_error", "zs_layout_buckets",
           "zs_layout_build", "zs_layout_build_tensors", "zs_layout_chunks",
           "zs_layout_info", "zs_layout_owners", "zs_layout_rank",
           "zs_layout_tensor_offsets", "zs_layout_tiles", "zs_pack",
           "zs_pack_noalloc", "zs_prefetch_acquire", "zs_prefetch_create",
           "zs_prefetch_free", "zs_prefetch_issue", "zs_prefetch_release", "zs_state_mv_pack",
           "zs_state_mv_unpack", "zs_state_pack", "zs_state_unpack",
           "zs_step", "zs_step_bf16", "zs_step_plain", "zs_stream_arrive", "zs_stream_create",
           "zs_set_residency_cap", "zs_stream_free", "zs_stream_step_begin",
           "zs_stream_step_end", "zs_strerror"]
