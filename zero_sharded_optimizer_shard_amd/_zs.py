"""ctypes binding of libzs (include/zs.h).  Argument marshalling only: every
step of the path runs in the HIP library; there is no fallback.  torch
tensors are used only as device memory and torch streams only as
hipStream_t handles.
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libzs.so")

ZS_OK, ZS_EINVAL, ZS_EALIGN, ZS_ERANGE, ZS_ENOMEM, ZS_EDEVICE = \
    0, -1, -2, -3, -4, -5
ZS_EIO, ZS_EMISMATCH = -6, -7
ZS_TILE = 8192
ZS_MAX_GROUP = 16
ZS_PACK_NOALLOC_MAX_CHUNKS = 32768
ZS_PACK_NOALLOC_MAX_TENSORS = 32768
ZS_GATHER_MAX_WORLD = 64
ZS_ACC_FIRST, ZS_ACC_ADD, ZS_ACC_LAST = 0, 1, 2
ZS_GRADS_SLICES, ZS_GRADS_TILED = 0, 1


class ZsError(RuntimeError):
    def __init__(self, code: int, func: str, detail: str):
        super().__init__(f"{func}: {detail} (code {code})")
        self.code = code


class zs_bucket(ctypes.Structure):
    _fields_ = [("flat_off", ctypes.c_int64), ("numel", ctypes.c_int64),
                ("slice_numel", ctypes.c_int64),
                ("shard_off", ctypes.c_int64), ("tile_off", ctypes.c_int64)]


class zs_chunk(ctypes.Structure):
    _fields_ = [("tensor_id", ctypes.c_int32), ("bucket_id", ctypes.c_int32),
                ("tensor_off", ctypes.c_int64), ("numel", ctypes.c_int64),
                ("shard_off", ctypes.c_int64)]


class zs_adamw(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float)]


_lib = None

EXPORTS = ["zs_layout_build", "zs_layout_build_tensors", "zs_layout_owners",
           "zs_layout_info", "zs_layout_tiles",
           "zs_layout_buckets", "zs_layout_chunks",
           "zs_layout_tensor_offsets", "zs_layout_rank", "zs_layout_free",
           "zs_step", "zs_step_plain", "zs_bucket_step", "zs_buckets_step",
           "zs_state_pack", "zs_state_unpack",
           "zs_grads_tile", "zs_gather", "zs_pack", "zs_pack_noalloc",
           "zs_step_bf16",
           "zs_state_mv_pack", "zs_state_mv_unpack", "zs_accumulate",
           "zs_stream_create", "zs_stream_create_multi",
           "zs_stream_step_begin", "zs_stream_arrive",
           "zs_stream_step_end", "zs_stream_free",
           "zs_prefetch_create", "zs_prefetch_issue", "zs_prefetch_acquire",
           "zs_prefetch_release", "zs_prefetch_free",
           "zs_layout_fingerprint", "zs_checkpoint_save",
           "zs_checkpoint_load",
           "zs_set_residency_cap", "zs_strerror", "zs_last_error"]


def lib():
    """Load libzs.so; raise loudly if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run "
                          "__graft_entry__.build() (the HIP library is the "
                          "only implementation)")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    P = ctypes.POINTER
    L.zs_layout_build.argtypes = [P(i64), i32, i32, i32, i64, i32, P(p)]
    L.zs_layout_info.argtypes = [p, P(i64), P(i64), P(i32), P(i32)]
    L.zs_layout_build_tensors.argtypes = [P(i64), i32, i32, i32, i32, P(p)]
    L.zs_layout_owners.argtypes = [p, P(i32), P(i64), i32]
    L.zs_layout_tiles.argtypes = [p, P(i64)]
    L.zs_layout_buckets.argtypes = [p, P(zs_bucket), i32]
    L.zs_layout_chunks.argtypes = [p, P(zs_chunk), i32]
    L.zs_layout_tensor_offsets.argtypes = [p, P(i64), i32]
    L.zs_layout_rank.argtypes = [p, P(i32), P(i32)]
    L.zs_layout_free.argtypes = [p]
    L.zs_layout_free.restype = None
    L.zs_step.argtypes = [p, p, i32, i64, p, p, p, P(zs_adamw), i64, p]
    L.zs_step_plain.argtypes = [p, p, i32, i64, p, p, p, p, p, P(zs_adamw),
                                i64, p]
    L.zs_bucket_step.argtypes = [p, i32, p, i32, i64, p, p, p, P(zs_adamw),
                                 i64, p]
    L.zs_buckets_step.argtypes = [p, i32, P(i32), P(p), i32, i64, p, p, p,
                                  P(zs_adamw), i64, p]
    L.zs_state_pack.argtypes = [p, p, p, p, p, p]
    L.zs_state_unpack.argtypes = [p, p, p, p, p, p]
    L.zs_grads_tile.argtypes = [p, i32, p, i64, p, p]
    L.zs_gather.argtypes = [p, P(p), i64, i64, p, p]
    L.zs_step_bf16.argtypes = [p, p, i32, i64, p, p, i32, P(zs_adamw), i64,
                               p]
    L.zs_state_mv_pack.argtypes = [p, p, p, p, p]
    L.zs_state_mv_unpack.argtypes = [p, p, p, p, p]
    L.zs_accumulate.argtypes = [i32, p, p, p, i64, i32, p]
    L.zs_pack.argtypes = [p, p, p, p, i32, p, p]
    L.zs_pack_noalloc.argtypes = [p, p, p, p, i32, p]
    L.zs_stream_create.argtypes = [p, i32, P(p), i32, i64, p, P(p), i32,
                                   P(p)]
    L.zs_stream_create_multi.argtypes = [p, i32, P(p), i32, i64, P(p), i32,
                                         P(p), i32, P(p)]
    L.zs_stream_step_begin.argtypes = [p, p, p, p, P(zs_adamw), i64]
    L.zs_stream_arrive.argtypes = [p, i32, p]
    L.zs_stream_step_end.argtypes = [p]
    L.zs_stream_free.argtypes = [p]
    L.zs_stream_free.restype = None
    L.zs_prefetch_create.argtypes = [p, P(p), P(p), i32, i64, p, P(p)]
    L.zs_prefetch_issue.argtypes = [p, i64, i64, P(i32)]
    L.zs_prefetch_acquire.argtypes = [p, i32, p, P(p)]
    L.zs_prefetch_release.argtypes = [p, i32, p]
    L.zs_prefetch_free.argtypes = [p]
    L.zs_prefetch_free.restype = None
    L.zs_layout_fingerprint.argtypes = [p, P(ctypes.c_uint64)]
    L.zs_checkpoint_save.argtypes = [p, ctypes.c_char_p, p, i32, i64, p]
    L.zs_checkpoint_load.argtypes = [p, ctypes.c_char_p, p, i32, P(i64), p]
    L.zs_strerror.argtypes = [ctypes.c_int]
    L.zs_strerror.restype = ctypes.c_char_p
    L.zs_last_error.argtypes = []
    L.zs_last_error.restype = ctypes.c_char_p
    L.zs_set_residency_cap.argtypes = [ctypes.c_int32]
    L.zs_set_residency_cap.restype = ctypes.c_int32
    for name in ("zs_layout_build", "zs_layout_build_tensors",
                 "zs_layout_owners", "zs_layout_info", "zs_layout_tiles",
                 "zs_layout_buckets", "zs_layout_chunks",
                 "zs_layout_tensor_offsets", "zs_layout_rank", "zs_step",
                 "zs_step_plain", "zs_bucket_step", "zs_buckets_step", "zs_state_pack",
                 "zs_state_unpack",
                 "zs_grads_tile", "zs_gather", "zs_pack", "zs_pack_noalloc",
                 "zs_step_bf16", "zs_state_mv_pack", "zs_state_mv_unpack",
                 "zs_accumulate", "zs_stream_create", "zs_stream_create_multi",
                 "zs_stream_step_begin",
                 "zs_stream_arrive", "zs_stream_step_end",
                 "zs_prefetch_create", "zs_prefetch_issue",
                 "zs_prefetch_acquire", "zs_prefetch_release",
                 "zs_layout_fingerprint", "zs_checkpoint_save",
                 "zs_checkpoint_load"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int, func: str) -> int:
    if rc < 0:
        raise ZsError(rc, func, lib().zs_last_error().decode() or
                      zs_strerror(rc))
    return rc


def zs_strerror(code: int) -> str:
    return lib().zs_strerror(code).decode()


def zs_last_error() -> str:
    return lib().zs_last_error().decode()


class Layout:
    """Owning handle of a zs_layout*."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)
        self._sizes = None

    @property
    def handle(self):
        return self._h

    def sizes(self):
        """(flat_numel, shard_numel, n_tiles, world, buckets), read from
        the library once; the bindings check tensor sizes against them."""
        if self._sizes is None:
            f, n = zs_layout_info(self)[:2]
            self._sizes = (f, n, zs_layout_tiles(self),
                           zs_layout_rank(self)[0], zs_layout_buckets(self))
        return self._sizes

    def __del__(self):
        if getattr(self, "_h", None) is not None and self._h.value and _lib:
            _lib.zs_layout_free(self._h)
            self._h = None


def zs_layout_build(tensor_numel: Sequence[int], world: int, rank: int,
                    bucket_cap_bytes: int = 25 << 20,
                    align_bytes: int = 256) -> Layout:
    n = len(tensor_numel)
    arr = (ctypes.c_int64 * max(n, 1))(*tensor_numel)
    out = ctypes.c_void_p()
    _check(lib().zs_layout_build(arr, n, world, rank, bucket_cap_bytes,
                                 align_bytes, ctypes.byref(out)),
           "zs_layout_build")
    return Layout(out.value)


def zs_layout_build_tensors(tensor_numel: Sequence[int], world: int,
                            rank: int, align_bytes: int = 256) -> Layout:
    """Whole-tensor shard assignment (see include/zs.h)."""
    n = len(tensor_numel)
    arr = (ctypes.c_int64 * max(n, 1))(*tensor_numel)
    out = ctypes.c_void_p()
    _check(lib().zs_layout_build_tensors(arr, n, world, rank, align_bytes,
                                         ctypes.byref(out)),
           "zs_layout_build_tensors")
    return Layout(out.value)


def zs_layout_owners(layout: Layout, n_tensors: int):
    """(owner rank per tensor, offset in the owner's shard per tensor)."""
    o = (ctypes.c_int32 * max(n_tensors, 1))()
    off = (ctypes.c_int64 * max(n_tensors, 1))()
    n = _check(lib().zs_layout_owners(layout.handle, o, off, n_tensors),
               "zs_layout_owners")
    return list(o[:n]), list(off[:n])


def zs_layout_info(layout: Layout):
    f, s = ctypes.c_int64(), ctypes.c_int64()
    nb, nc = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().zs_layout_info(layout.handle, ctypes.byref(f),
                                ctypes.byref(s), ctypes.byref(nb),
                                ctypes.byref(nc)), "zs_layout_info")
    return f.value, s.value, nb.value, nc.value


def zs_layout_tiles(layout: Layout) -> int:
    n = ctypes.c_int64()
    _check(lib().zs_layout_tiles(layout.handle, ctypes.byref(n)),
           "zs_layout_tiles")
    return n.value


def zs_layout_rank(layout: Layout):
    w, r = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().zs_layout_rank(layout.handle, ctypes.byref(w),
                                ctypes.byref(r)), "zs_layout_rank")
    return w.value, r.value


def zs_layout_buckets(layout: Layout) -> List[zs_bucket]:
    nb = zs_layout_info(layout)[2]
    out = (zs_bucket * max(nb, 1))()
    n = _check(lib().zs_layout_buckets(layout.handle, out, nb),
               "zs_layout_buckets")
    return list(out[:n])


def zs_layout_chunks(layout: Layout) -> List[zs_chunk]:
    nc = zs_layout_info(layout)[3]
    out = (zs_chunk * max(nc, 1))()
    n = _check(lib().zs_layout_chunks(layout.handle, out, nc),
               "zs_layout_chunks")
    return list(out[:n])


def zs_layout_tensor_offsets(layout: Layout, n_tensors: int) -> List[int]:
    out = (ctypes.c_int64 * max(n_tensors, 1))()
    n = _check(lib().zs_layout_tensor_offsets(layout.handle, out, n_tensors),
               "zs_layout_tensor_offsets")
    return list(out[:n])


def chunks_bytes(chunks: List[zs_chunk]) -> bytes:
    """The chunk table as raw bytes, for a device copy (zs_pack)."""
    arr = (zs_chunk * len(chunks))(*chunks)
    return bytes(arr)


# ---- device calls ------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _bf16(t, name):
    if t is not None and t.element_size() != 2:
        raise TypeError(f"{name}: need a 2-byte (bf16 bits) tensor")
    return _ptr(t)


def _f32(t, name):
    import torch
    if t.dtype != torch.float32:
        raise TypeError(f"{name}: need float32")
    return _ptr(t)


def _need(t, numel: int, name: str) -> None:
    """The kernels address a buffer by the layout's sizes alone: refuse a
    tensor shorter than that here, before any device access."""
    if t is not None and numel > 0 and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, the layout needs "
                         f"at least {numel}")


def _tiles(slice_numel: int) -> int:
    return -(-slice_numel // ZS_TILE)


def _grads_need(W: int, tiles: int, slice_numel: int, code: int,
                stride: int) -> int:
    """Elements a gradient buffer must hold: [tiles][W][ZS_TILE] tiled, or
    W rows of `slice_numel` at `stride` (a stride below the slice length is
    the library's to refuse)."""
    if code == ZS_GRADS_TILED:
        return tiles * W * ZS_TILE
    return (W - 1) * max(stride, 0) + slice_numel


def _step_need(layout: Layout, grads, code: int, stride: int, state, rows,
               param_shard, full_flat, names=("state", "param_shard",
                                              "full_flat")) -> None:
    f, n, nt, W, _ = layout.sizes()
    if n == 0:
        return
    _need(grads, _grads_need(W, nt, n, code, stride), "grads")
    _need(state, nt * rows * ZS_TILE, names[0])
    _need(param_shard, n, names[1])
    _need(full_flat, f, names[2])


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _hp(lr, beta1, beta2, eps, weight_decay):
    return zs_adamw(lr, beta1, beta2, eps, weight_decay)


def _layout_code(grad_layout) -> int:
    codes = {"slices": ZS_GRADS_SLICES, "tiled": ZS_GRADS_TILED,
             ZS_GRADS_SLICES: ZS_GRADS_SLICES, ZS_GRADS_TILED: ZS_GRADS_TILED}
    if grad_layout not in codes:
        # unknown codes go through unchanged so the library reports them
        return int(grad_layout)
    return codes[grad_layout]


def zs_step(layout: Layout, grads, state, param_shard=None, full_flat=None,
            *, grad_layout="slices", grad_stride: int = 0, lr: float,
            beta1: float, beta2: float, eps: float, weight_decay: float,
            step: int, stream=None) -> None:
    """grads: [W][grad_stride] slices (grad_layout "slices") or
    [n_tiles][W][ZS_TILE] ("tiled"); state: tiled fp32 state."""
    hp = _hp(lr, beta1, beta2, eps, weight_decay)
    _step_need(layout, grads, _layout_code(grad_layout), grad_stride, state,
               3, param_shard, full_flat)
    _check(lib().zs_step(layout.handle, _bf16(grads, "grads"),
                         _layout_code(grad_layout), grad_stride,
                         _f32(state, "state"),
                         _bf16(param_shard, "param_shard"),
                         _bf16(full_flat, "full_flat"), ctypes.byref(hp),
                         step, _stream(stream)), "zs_step")


def zs_step_plain(layout: Layout, grads, master, m, v, param_shard=None,
                  full_flat=None, *, grad_layout="slices",
                  grad_stride: int = 0, lr: float, beta1: float, beta2: float,
                  eps: float, weight_decay: float, step: int,
                  stream=None) -> None:
    """zs_step on three plain fp32 [shard_numel] arrays master, m, v."""
    hp = _hp(lr, beta1, beta2, eps, weight_decay)
    _step_need(layout, grads, _layout_code(grad_layout), grad_stride, None,
               3, param_shard, full_flat)
    n = layout.sizes()[1]
    for t, name in ((master, "master"), (m, "m"), (v, "v")):
        _need(t, n, name)
    _check(lib().zs_step_plain(layout.handle, _bf16(grads, "grads"),
                               _layout_code(grad_layout), grad_stride,
                               _f32(master, "master"), _f32(m, "m"),
                               _f32(v, "v"),
                               _bf16(param_shard, "param_shard"),
                               _bf16(full_flat, "full_flat"),
                               ctypes.byref(hp), step, _stream(stream)),
           "zs_step_plain")


def zs_bucket_step(layout: Layout, bucket_id: int, grads, state,
                   param_shard=None, full_flat=None, *,
                   grad_layout="slices", grad_stride: int = 0, lr: float,
                   beta1: float, beta2: float, eps: float,
                   weight_decay: float, step: int, stream=None) -> None:
    hp = _hp(lr, beta1, beta2, eps, weight_decay)
    _buckets_need(layout, [bucket_id], [grads], _layout_code(grad_layout),
                  grad_stride, state, param_shard, full_flat)
    _check(lib().zs_bucket_step(layout.handle, bucket_id,
                                _bf16(grads, "grads"),
                                _layout_code(grad_layout), grad_stride,
                                _f32(state, "state"),
                                _bf16(param_shard, "param_shard"),
                                _bf16(full_flat, "full_flat"),
                                ctypes.byref(hp), step, _stream(stream)),
           "zs_bucket_step")


def _buckets_need(layout: Layout, bucket_ids, grads, code: int, stride: int,
                  state, param_shard, full_flat) -> None:
    f, n, nt, W, buckets = layout.sizes()
    for b, g in zip(bucket_ids, grads):
        if 0 <= b < len(buckets):       # other ids: the library's to refuse
            sl = buckets[b].slice_numel
            _need(g, _grads_need(W, _tiles(sl), sl, code, stride), "grads")
    _step_need(layout, None, code, stride, state, 3, param_shard, full_flat)


def zs_buckets_step(layout: Layout, bucket_ids, grads, state,
                    param_shard=None, full_flat=None, *,
                    grad_layout="slices", grad_stride: int = 0, lr: float,
                    beta1: float, beta2: float, eps: float,
                    weight_decay: float, step: int, stream=None) -> None:
    """bucket_ids: sequence of bucket ids; grads: one staging tensor per
    bucket, in the same order."""
    n = len(bucket_ids)
    if len(grads) != n:
        raise ValueError("one staging tensor per bucket")
    _buckets_need(layout, bucket_ids, grads, _layout_code(grad_layout),
                  grad_stride, state, param_shard, full_flat)
    ids = (ctypes.c_int32 * max(n, 1))(*bucket_ids)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[_bf16(g, "grads") for g in grads])
    hp = _hp(lr, beta1, beta2, eps, weight_decay)
    _check(lib().zs_buckets_step(layout.handle, n, ids, ptrs,
                                 _layout_code(grad_layout), grad_stride,
                                 _f32(state, "state"),
                                 _bf16(param_shard, "param_shard"),
                                 _bf16(full_flat, "full_flat"),
                                 ctypes.byref(hp), step, _stream(stream)),
           "zs_buckets_step")


def zs_state_pack(layout: Layout, master, m, v, state, stream=None) -> None:
    """Plain master/m/v (m, v may be None: zeros) -> tiled state."""
    _state_need(layout, state, 3, master=master, m=m, v=v)
    _check(lib().zs_state_pack(layout.handle, _f32(master, "master"),
                               None if m is None else _f32(m, "m"),
                               None if v is None else _f32(v, "v"),
                               _f32(state, "state"), _stream(stream)),
           "zs_state_pack")


def _state_need(layout: Layout, state, rows: int, **plain) -> None:
    f, n, nt, W, _ = layout.sizes()
    if n == 0:
        return
    _need(state, nt * rows * ZS_TILE, "state" if rows == 3 else "state_mv")
    for name, t in plain.items():
        _need(t, n, name)


def zs_state_unpack(layout: Layout, state, master=None, m=None, v=None,
                    stream=None) -> None:
    _state_need(layout, state, 3, master=master, m=m, v=v)
    _check(lib().zs_state_unpack(layout.handle, _f32(state, "state"),
                                 None if master is None
                                 else _f32(master, "master"),
                                 None if m is None else _f32(m, "m"),
                                 None if v is None else _f32(v, "v"),
                                 _stream(stream)), "zs_state_unpack")


def zs_grads_tile(layout: Layout, bucket_id: int, slices, stride: int,
                  tiled, stream=None) -> None:
    f, n, nt, W, buckets = layout.sizes()
    if bucket_id < 0:
        sl, tiles = n, nt
    elif bucket_id < len(buckets):
        sl = buckets[bucket_id].slice_numel
        tiles = _tiles(sl)
    else:
        sl = tiles = 0                  # the library refuses the id
    if n:
        _need(slices, _grads_need(W, tiles, sl, ZS_GRADS_SLICES, stride),
              "slices")
        _need(tiled, tiles * W * ZS_TILE, "tiled")
    _check(lib().zs_grads_tile(layout.handle, bucket_id,
                               _bf16(slices, "slices"), stride,
                               _bf16(tiled, "tiled"), _stream(stream)),
           "zs_grads_tile")


def zs_step_bf16(layout: Layout, grads, state_mv, params, *,
                 params_flat: bool = False, grad_layout="slices",
                 grad_stride: int = 0, lr: float, beta1: float, beta2: float,
                 eps: float, weight_decay: float, step: int,
                 stream=None) -> None:
    """Pure-bf16 step: params (bf16 shard, or the flat buffer when
    params_flat) updated in place; state_mv tiled [tiles][2][ZS_TILE]."""
    hp = _hp(lr, beta1, beta2, eps, weight_decay)
    _step_need(layout, grads, _layout_code(grad_layout), grad_stride,
               state_mv, 2, None if params_flat else params,
               params if params_flat else None,
               ("state_mv", "params", "params"))
    _check(lib().zs_step_bf16(layout.handle, _bf16(grads, "grads"),
                              _layout_code(grad_layout), grad_stride,
                              _f32(state_mv, "state_mv"),
                              _bf16(params, "params"), int(params_flat),
                              ctypes.byref(hp), step, _stream(stream)),
           "zs_step_bf16")


def zs_state_mv_pack(layout: Layout, m, v, state_mv, stream=None) -> None:
    _state_need(layout, state_mv, 2, m=m, v=v)
    _check(lib().zs_state_mv_pack(layout.handle,
                                  None if m is None else _f32(m, "m"),
                                  None if v is None else _f32(v, "v"),
                                  _f32(state_mv, "state_mv"),
                                  _stream(stream)), "zs_state_mv_pack")


def zs_state_mv_unpack(layout: Layout, state_mv, m=None, v=None,
                       stream=None) -> None:
    _state_need(layout, state_mv, 2, m=m, v=v)
    _check(lib().zs_state_mv_unpack(layout.handle,
                                    _f32(state_mv, "state_mv"),
                                    None if m is None else _f32(m, "m"),
                                    None if v is None else _f32(v, "v"),
                                    _stream(stream)), "zs_state_mv_unpack")


def zs_accumulate(mode: int, acc, grad, out=None, k: int = 0,
                  stream=None) -> None:
    """One micro-batch of gradient accumulation (ZS_ACC_FIRST / _ADD /
    _LAST); acc fp32, grad and out bf16, all of the same length."""
    n = grad.numel()
    _need(acc, n, "acc")
    _need(out, n, "out")
    _check(lib().zs_accumulate(mode, _f32(acc, "acc"), _bf16(grad, "grad"),
                               _bf16(out, "out"), n, k, _stream(stream)),
           "zs_accumulate")


def zs_gather(layout: Layout, shards, flat_lo: int, flat_hi: int, out,
              stream=None) -> None:
    """shards: one bf16 shard tensor per rank, in rank order; out: at least
    flat_hi - flat_lo bf16 elements."""
    _need(out, flat_hi - flat_lo, "out")
    ptrs = (ctypes.c_void_p * max(len(shards), 1))(
        *[_bf16(t, "shards") for t in shards])
    _check(lib().zs_gather(layout.handle, ptrs, flat_lo, flat_hi,
                           _bf16(out, "out"), _stream(stream)), "zs_gather")


def zs_pack(layout: Layout, param_shard, full_flat=None, dev_chunks=None,
            n_chunks: int = 0, dev_tensor_ptrs=None, stream=None) -> None:
    """dev_chunks: device tensor holding chunks_bytes(); dev_tensor_ptrs:
    device int64 tensor of per-tensor data pointers."""
    f, n = layout.sizes()[:2]
    if n:
        _need(param_shard, n, "param_shard")
        _need(full_flat, f, "full_flat")
    _check(lib().zs_pack(layout.handle, _bf16(param_shard, "param_shard"),
                         _bf16(full_flat, "full_flat"), _ptr(dev_chunks),
                         n_chunks, _ptr(dev_tensor_ptrs), _stream(stream)),
           "zs_pack")


def zs_set_residency_cap(on: bool) -> bool:
    """Switch the step launches' LDS reservation on or off for the process;
    returns the previous setting."""
    return bool(lib().zs_set_residency_cap(1 if on else 0))


def zs_pack_noalloc(layout: Layout, param_shard, full_flat=None,
                    tensors=None, stream=None) -> None:
    """zs_pack with the library's own static staging: tensors is a list of
    per-tensor bf16 device tensors (or device addresses as ints), indexed
    by tensor id, handed over as a host pointer array; None for the flat
    output alone."""
    f, n = layout.sizes()[:2]
    if n:
        _need(param_shard, n, "param_shard")
        _need(full_flat, f, "full_flat")
    arr, count = None, 0
    if tensors is not None:
        count = len(tensors)
        arr = (ctypes.c_void_p * max(count, 1))(
            *[x if isinstance(x, int) else _bf16(x, "tensors")
              for x in tensors])
    _check(lib().zs_pack_noalloc(layout.handle,
                                 _bf16(param_shard, "param_shard"),
                                 _bf16(full_flat, "full_flat"), arr, count,
                                 _stream(stream)), "zs_pack_noalloc")


# ---- ZeRO-2 streaming engine -------------------------------------------------

class Stream:
    """Owning handle of a zs_stream* (see include/zs.h).  Keeps the layout,
    the staging slots and the streams it was given alive."""

    def __init__(self, handle: int, keep):
        self._h = ctypes.c_void_p(handle)
        self._keep = keep

    @property
    def handle(self):
        return self._h

    def __del__(self):
        if getattr(self, "_h", None) is not None and self._h.value and _lib:
            _lib.zs_stream_free(self._h)
            self._h = None


def zs_stream_create(layout: Layout, group: int, slots, upload_stream,
                     step_streams) -> Stream:
    """slots: device bf16 staging tensors (the ring); upload_stream: a torch
    stream, or a list of them (zs_stream_create_multi: arrivals take them in
    turn); step_streams: torch streams."""
    n = len(slots)
    arr = (ctypes.c_void_p * max(n, 1))(*[_bf16(t, "slots") for t in slots])
    k = len(step_streams)
    ss = (ctypes.c_void_p * max(k, 1))(*[t.cuda_stream for t in step_streams])
    elems = min(t.numel() for t in slots) if n else 0
    out = ctypes.c_void_p()
    if isinstance(upload_stream, (list, tuple)):
        nu = len(upload_stream)
        us = (ctypes.c_void_p * max(nu, 1))(*[t.cuda_stream
                                              for t in upload_stream])
        _check(lib().zs_stream_create_multi(layout.handle, group, arr, n,
                                            elems, us, nu, ss, k,
                                            ctypes.byref(out)),
               "zs_stream_create_multi")
        ups = list(upload_stream)
    else:
        _check(lib().zs_stream_create(
            layout.handle, group, arr, n, elems,
            ctypes.c_void_p(upload_stream.cuda_stream), ss, k,
            ctypes.byref(out)), "zs_stream_create")
        ups = upload_stream
    return Stream(out.value, (layout, list(slots), ups, list(step_streams)))


def zs_stream_step_begin(stream: Stream, state, param_shard=None,
                         full_flat=None, *, lr: float, beta1: float,
                         beta2: float, eps: float, weight_decay: float,
                         step: int) -> None:
    hp = _hp(lr, beta1, beta2, eps, weight_decay)
    _step_need(stream._keep[0], None, ZS_GRADS_TILED, 0, state, 3,
               param_shard, full_flat)
    _check(lib().zs_stream_step_begin(stream.handle, _f32(state, "state"),
                                      _bf16(param_shard, "param_shard"),
                                      _bf16(full_flat, "full_flat"),
                                      ctypes.byref(hp), step),
           "zs_stream_step_begin")


def zs_stream_arrive(stream: Stream, bucket_id: int, src) -> None:
    """src: the bucket's tiled gradients, a device tensor or a pinned host
    tensor (2-byte elements, contiguous)."""
    if src.element_size() != 2 or not src.is_contiguous():
        raise TypeError("src: need a contiguous 2-byte tensor")
    if not (src.is_cuda or src.is_pinned()):
        raise ValueError("src: need device or pinned host memory")
    f, n, nt, W, buckets = stream._keep[0].sizes()
    if 0 <= bucket_id < len(buckets):   # other ids: the library's to refuse
        _need(src, _tiles(buckets[bucket_id].slice_numel) * W * ZS_TILE,
              "src")
    _check(lib().zs_stream_arrive(stream.handle, bucket_id,
                                  ctypes.c_void_p(src.data_ptr())),
           "zs_stream_arrive")


def zs_stream_step_end(stream: Stream) -> int:
    """Steps the pending partial group; returns the buckets stepped in the
    step."""
    return _check(lib().zs_stream_step_end(stream.handle),
                  "zs_stream_step_end")


def zs_stream_free(stream: Stream) -> None:
    if stream._h is not None and stream._h.value:
        lib().zs_stream_free(stream._h)
        stream._h = None


# ---- ZeRO-3 / FSDP prefetch -----------------------------------------------------

class Prefetch:
    """Owning handle of a zs_prefetch* (see include/zs.h).  Keeps the
    layout, shards, buffers and gather stream it was given alive."""

    def __init__(self, handle: int, keep):
        self._h = ctypes.c_void_p(handle)
        self._keep = keep

    @property
    def handle(self):
        return self._h

    def __del__(self):
        if getattr(self, "_h", None) is not None and self._h.value and _lib:
            _lib.zs_prefetch_free(self._h)
            self._h = None


def zs_prefetch_create(layout: Layout, shards, buffers,
                       gather_stream) -> Prefetch:
    """shards: the world's device bf16 shards; buffers: device bf16 unit
    buffers (the ring); gather_stream: a torch stream."""
    sh = (ctypes.c_void_p * max(len(shards), 1))(
        *[_bf16(t, "shards") for t in shards])
    n = len(buffers)
    bu = (ctypes.c_void_p * max(n, 1))(*[_bf16(t, "buffers") for t in buffers])
    elems = min(t.numel() for t in buffers) if n else 0
    out = ctypes.c_void_p()
    _check(lib().zs_prefetch_create(layout.handle, sh, bu, n, elems,
                                    ctypes.c_void_p(gather_stream.cuda_stream),
                                    ctypes.byref(out)),
           "zs_prefetch_create")
    return Prefetch(out.value, (layout, list(shards), list(buffers),
                                gather_stream))


def zs_prefetch_issue(prefetch: Prefetch, flat_lo: int, flat_hi: int) -> int:
    """Gathers [flat_lo, flat_hi) into the next buffer; returns its slot."""
    slot = ctypes.c_int32()
    _check(lib().zs_prefetch_issue(prefetch.handle, flat_lo, flat_hi,
                                   ctypes.byref(slot)), "zs_prefetch_issue")
    return slot.value


def zs_prefetch_acquire(prefetch: Prefetch, slot: int, compute_stream=None):
    """Orders compute_stream after the slot's gather; returns the buffer
    tensor the slot stands for."""
    _check(lib().zs_prefetch_acquire(prefetch.handle, slot,
                                     _stream(compute_stream), None),
           "zs_prefetch_acquire")
    return prefetch._keep[2][slot]


def zs_prefetch_release(prefetch: Prefetch, slot: int,
                        compute_stream=None) -> None:
    _check(lib().zs_prefetch_release(prefetch.handle, slot,
                                     _stream(compute_stream)),
           "zs_prefetch_release")


def zs_prefetch_free(prefetch: Prefetch) -> None:
    if prefetch._h is not None and prefetch._h.value:
        lib().zs_prefetch_free(prefetch._h)
        prefetch._h = None


# ---- checkpoint and resume ----------------------------------------------------

def zs_layout_fingerprint(layout: Layout) -> int:
    """64-bit fingerprint of the layout's defining inputs."""
    out = ctypes.c_uint64()
    _check(lib().zs_layout_fingerprint(layout.handle, ctypes.byref(out)),
           "zs_layout_fingerprint")
    return out.value


def _path(path) -> bytes:
    return os.fsencode(path)


def zs_checkpoint_save(layout: Layout, path, state, step: int, rows: int = 3,
                       stream=None) -> None:
    """Write the tiled state (rows 3: master|m|v; 2: m|v) and the step
    counter to `path`, replacing it atomically."""
    if rows in (2, 3):
        _need(state, layout.sizes()[2] * rows * ZS_TILE, "state")
    _check(lib().zs_checkpoint_save(layout.handle, _path(path),
                                    _f32(state, "state"), rows, step,
                                    _stream(stream)), "zs_checkpoint_save")


def zs_checkpoint_load(layout: Layout, path, state, rows: int = 3,
                       stream=None) -> int:
    """Restore a checkpoint of this layout into the tiled state; returns
    its step counter."""
    if rows in (2, 3):
        _need(state, layout.sizes()[2] * rows * ZS_TILE, "state")
    step = ctypes.c_int64()
    _check(lib().zs_checkpoint_load(layout.handle, _path(path),
                                    _f32(state, "state"), rows,
                                    ctypes.byref(step), _stream(stream)),
           "zs_checkpoint_load")
    return step.value
