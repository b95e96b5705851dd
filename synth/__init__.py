"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke
check: parameter-list workloads and one counter-based generator implemented
twice from its definition (gen.c on the CPU, gen.hip on the GPU).

Nothing here computes any part of the optimizer step.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from .workloads import (TAG_GRAD, TAG_M, TAG_MASTER, TAG_SENTINEL, TAG_V,
                        Workload, presets)

_HERE = os.path.dirname(os.path.abspath(__file__))
_cpu = None
_dev = None

__all__ = ["cpu_normal_f32", "cpu_normal_bf16", "cpu_bits16",
           "dev_normal_f32", "dev_normal_bf16", "dev_bits16", "dev_copy",
           "dev_mix_stream", "Workload", "presets", "TAG_GRAD",
           "TAG_MASTER", "TAG_M", "TAG_V", "TAG_SENTINEL"]


def _load(name):
    path = os.path.join(_HERE, name)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
    return ctypes.CDLL(path)


def _cpu_lib():
    global _cpu
    if _cpu is None:
        L = _load("libsynth_cpu.so")
        u64, i64, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        L.synth_normal_f32.argtypes = [p, i64, u64, u64, u64, u64, i64,
                                       ctypes.c_double, ctypes.c_int32]
        L.synth_normal_bf16.argtypes = [p, i64, u64, u64, u64, u64, i64,
                                        ctypes.c_double]
        L.synth_bits16.argtypes = [p, i64, u64, u64, u64, u64, i64]
        for f in (L.synth_normal_f32, L.synth_normal_bf16, L.synth_bits16):
            f.restype = None
        _cpu = L
    return _cpu


def _dev_lib():
    global _dev
    if _dev is None:
        L = _load("libsynth_dev.so")
        u64, i64, i32, p = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                            ctypes.c_void_p)
        L.synth_normal_f32_dev.argtypes = [p, i64, u64, u64, u64, u64, i64,
                                           ctypes.c_double, i32, p]
        L.synth_normal_bf16_dev.argtypes = [p, i64, u64, u64, u64, u64, i64,
                                            ctypes.c_double, p]
        L.synth_bits16_dev.argtypes = [p, i64, u64, u64, u64, u64, i64, p]
        L.synth_copy_dev.argtypes = [p, p, i64, p]
        L.synth_read_dev.argtypes = [p, i64, p, p]
        L.synth_mix_stream_dev.argtypes = [p, p, p, i32, i64, i64, i64,
                                           i32, p]
        for f in (L.synth_normal_f32_dev, L.synth_normal_bf16_dev,
                  L.synth_bits16_dev, L.synth_copy_dev, L.synth_read_dev,
                  L.synth_mix_stream_dev):
            f.restype = ctypes.c_int
        _dev = L
    return _dev


# ---- CPU ------------------------------------------------------------------

def cpu_normal_f32(n, seed, tag, step, src, index_base, sigma, absval=False):
    out = np.empty(n, np.float32)
    _cpu_lib().synth_normal_f32(out.ctypes.data, n, seed, tag, step, src,
                                index_base, sigma, int(absval))
    return out


def cpu_normal_bf16(n, seed, tag, step, src, index_base, sigma):
    """Returns the bf16 bit patterns as uint16."""
    out = np.empty(n, np.uint16)
    _cpu_lib().synth_normal_bf16(out.ctypes.data, n, seed, tag, step, src,
                                 index_base, sigma)
    return out


def cpu_bits16(n, seed, tag, step, src, index_base):
    out = np.empty(n, np.uint16)
    _cpu_lib().synth_bits16(out.ctypes.data, n, seed, tag, step, src,
                            index_base)
    return out


# ---- GPU (torch tensors are only device memory here) ----------------------

def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def dev_normal_f32(t, seed, tag, step, src, index_base, sigma, absval=False,
                   stream=None):
    import torch
    assert t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()
    _ok(_dev_lib().synth_normal_f32_dev(t.data_ptr(), t.numel(), seed, tag,
                                        step, src, index_base, sigma,
                                        int(absval), _stream_handle(stream)),
        "synth_normal_f32_dev")


def dev_normal_bf16(t, seed, tag, step, src, index_base, sigma, stream=None):
    import torch
    assert t.is_cuda and t.element_size() == 2 and t.is_contiguous()
    _ok(_dev_lib().synth_normal_bf16_dev(t.data_ptr(), t.numel(), seed, tag,
                                         step, src, index_base, sigma,
                                         _stream_handle(stream)),
        "synth_normal_bf16_dev")


def dev_bits16(t, seed, tag, step, src, index_base, stream=None):
    assert t.is_cuda and t.element_size() == 2 and t.is_contiguous()
    _ok(_dev_lib().synth_bits16_dev(t.data_ptr(), t.numel(), seed, tag, step,
                                    src, index_base, _stream_handle(stream)),
        "synth_bits16_dev")


def dev_copy(dst, src, nbytes, stream=None):
    _ok(_dev_lib().synth_copy_dev(dst.data_ptr(), src.data_ptr(), nbytes,
                                  _stream_handle(stream)), "synth_copy_dev")


def dev_read(src, nbytes, sink, stream=None):
    """Read nbytes of src (the read-only ceiling); sink: >= 16 bytes."""
    _ok(_dev_lib().synth_read_dev(src.data_ptr(), nbytes, sink.data_ptr(),
                                  _stream_handle(stream)), "synth_read_dev")


def dev_mix_stream(grads_tiled, state, flat, W, S, S_last, B, nb,
                   stream=None):
    """The step's access pattern on tiled gradients/state (bench ceiling)."""
    _ok(_dev_lib().synth_mix_stream_dev(grads_tiled.data_ptr(),
                                        state.data_ptr(), flat.data_ptr(), W,
                                        S, S_last, B, nb,
                                        _stream_handle(stream)),
        "synth_mix_stream_dev")
