"""numpy front end of the C step oracle (oracle/zs_oracle.c).

TEST INFRASTRUCTURE: see oracle/__init__.py.  Arrays are numpy; bf16 values
travel as their uint16 bit patterns.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_DEFAULT_LIB = os.path.join(_HERE, "libzs_oracle.so")
# ZS_ORACLE_LIB names another build of zs_oracle.c to load instead; the
# mutation test uses it to run the pins against planted mistakes.
_LIB_PATH = os.environ.get("ZS_ORACLE_LIB") or _DEFAULT_LIB
_lib = None


class _HP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float)]


@dataclass(frozen=True)
class AdamW:
    """Hyper-parameters; defaults are the workloads' lr 3e-4, betas 0.9/0.95,
    eps 1e-8, weight decay 0.1."""
    lr: float = 3e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1

    def c(self) -> _HP:
        return _HP(self.lr, self.beta1, self.beta2, self.eps,
                   self.weight_decay)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            if _LIB_PATH != _DEFAULT_LIB:
                raise FileNotFoundError(_LIB_PATH)
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.oracle_constants.argtypes = [ctypes.POINTER(_HP), i64, p]
        L.oracle_bf16_round.argtypes = [p, p, i64]
        L.oracle_reduce_mean.argtypes = [i32, p, i64, i64, p]
        L.oracle_adamw.argtypes = [i64, p, p, p, p, p, ctypes.POINTER(_HP),
                                   i64]
        L.oracle_step.argtypes = [i32, p, i64, i64, p, p, p, p,
                                  ctypes.POINTER(_HP), i64]
        L.oracle_step_bf16.argtypes = [i32, p, i64, i64, p, p, p,
                                       ctypes.POINTER(_HP), i64]
        L.oracle_accumulate.argtypes = [i32, p, i64, i64, p]
        for f in (L.oracle_constants, L.oracle_bf16_round,
                  L.oracle_reduce_mean, L.oracle_adamw, L.oracle_step,
                  L.oracle_step_bf16, L.oracle_accumulate):
            f.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype \
            or not a.flags.c_contiguous:
        raise TypeError(f"{name}: need a C-contiguous numpy {dtype} array")


def constants(hp: AdamW, t: int) -> np.ndarray:
    out = np.zeros(8, np.float32)
    lib().oracle_constants(ctypes.byref(hp.c()), t, _ptr(out))
    return out


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_bf16_round(_ptr(x), _ptr(out), x.size)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def reduce_mean(grads: np.ndarray) -> np.ndarray:
    """grads: uint16 [W][n] -> fp32 [n], the fixed-order mean."""
    _check(grads, np.uint16, "grads")
    W, n = grads.shape
    out = np.empty(n, np.float32)
    lib().oracle_reduce_mean(W, _ptr(grads), n, n, _ptr(out))
    return out


def adamw(grad: np.ndarray, master: np.ndarray, m: np.ndarray, v: np.ndarray,
          hp: AdamW, t: int) -> np.ndarray:
    """In-place AdamW on fp32 arrays; returns the bf16 bits of the result."""
    for a, nm in ((grad, "grad"), (master, "master"), (m, "m"), (v, "v")):
        _check(a, np.float32, nm)
    n = master.size
    p16 = np.empty(n, np.uint16)
    lib().oracle_adamw(n, _ptr(grad), _ptr(master), _ptr(m), _ptr(v),
                       _ptr(p16), ctypes.byref(hp.c()), t)
    return p16


def step(grads: np.ndarray, master: np.ndarray, m: np.ndarray, v: np.ndarray,
         hp: AdamW, t: int, grad_stride: int | None = None) -> np.ndarray:
    """One ZeRO step over a contiguous run of shard elements, in place.

    grads: uint16, either [W][n] or a flat buffer read as [W][grad_stride].
    Returns the bf16 bits of the updated master.
    """
    _check(grads, np.uint16, "grads")
    for a, nm in ((master, "master"), (m, "m"), (v, "v")):
        _check(a, np.float32, nm)
    n = master.size
    if grads.ndim == 2:
        W = grads.shape[0]
        stride = grads.shape[1]
    else:
        if grad_stride is None:
            raise ValueError("flat grads need grad_stride")
        stride = grad_stride
        W = grads.size // stride
    if stride < n or grads.size < W * stride - (stride - n):
        raise ValueError("grads too small")
    p16 = np.empty(n, np.uint16)
    lib().oracle_step(W, _ptr(grads), stride, n, _ptr(master), _ptr(m),
                      _ptr(v), _ptr(p16), ctypes.byref(hp.c()), t)
    return p16


def step_bf16(grads: np.ndarray, param: np.ndarray, m: np.ndarray,
              v: np.ndarray, hp: AdamW, t: int) -> None:
    """Pure-bf16 step (no fp32 master) over a contiguous run, in place:
    grads uint16 [W][n], param uint16 [n] (bf16 bits), m and v fp32 [n]."""
    _check(grads, np.uint16, "grads")
    _check(param, np.uint16, "param")
    for a, nm in ((m, "m"), (v, "v")):
        _check(a, np.float32, nm)
    W, n = grads.shape
    if param.size != n or m.size != n or v.size != n:
        raise ValueError("size mismatch")
    lib().oracle_step_bf16(W, _ptr(grads), n, n, _ptr(param), _ptr(m),
                           _ptr(v), ctypes.byref(hp.c()), t)


def accumulate(grads: np.ndarray) -> np.ndarray:
    """Gradient accumulation: uint16 [k][n] micro-batch gradients (bf16
    bits) -> the bf16 bits of their fp32 mean, summed in order."""
    _check(grads, np.uint16, "grads")
    k, n = grads.shape
    out = np.empty(n, np.uint16)
    lib().oracle_accumulate(k, _ptr(grads), n, n, _ptr(out))
    return out
