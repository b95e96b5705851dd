"""Comparison helpers for GPU-vs-oracle parity.

Bars (fixed by the step's contract): fp32 master, m and v within 1e-6
relative error with an absolute floor of 1e-9; bf16 parameters within one
ordinal step (1 ulp).  The library also aims for bit-identical results (same
operation order, one rounding per operation, correctly rounded divide and
square root on both sides); `exact` reports whether it got them.
"""

from __future__ import annotations

import numpy as np

REL, ABS = 1e-6, 1e-9


def f32_report(x, ref):
    x = np.asarray(x, np.float32)
    ref = np.asarray(ref, np.float32)
    nan_x, nan_r = np.isnan(x), np.isnan(ref)
    both = ~(nan_x | nan_r)
    d = np.abs(x[both].astype(np.float64) - ref[both].astype(np.float64))
    bar = np.maximum(REL * np.abs(ref[both].astype(np.float64)), ABS)
    ok = bool(np.array_equal(nan_x, nan_r) and np.all(d <= bar))
    same = (x.view(np.uint32) == ref.view(np.uint32)) | (nan_x & nan_r)
    n_diff = int(np.count_nonzero(~same))
    ulp = 0.0
    if n_diff:
        sp = np.spacing(np.abs(ref[both])).astype(np.float64)
        ulp = float(np.max(d / np.maximum(sp, 1e-45))) if d.size else 0.0
    return dict(ok=ok, exact=n_diff == 0, n_diff=n_diff, max_ulp=ulp)


def bf16_ordinal(bits):
    b = np.asarray(bits, np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7fff), b)


def bf16_report(x, ref):
    x = np.asarray(x, np.uint16)
    ref = np.asarray(ref, np.uint16)
    nan_x = ((x & 0x7f80) == 0x7f80) & ((x & 0x7f) != 0)
    nan_r = ((ref & 0x7f80) == 0x7f80) & ((ref & 0x7f) != 0)
    both = ~(nan_x | nan_r)
    dist = np.abs(bf16_ordinal(x[both]) - bf16_ordinal(ref[both]))
    ok = bool(np.array_equal(nan_x, nan_r) and (dist.max(initial=0) <= 1))
    n_diff = int(np.count_nonzero((x != ref) & ~(nan_x & nan_r)))
    return dict(ok=ok, exact=n_diff == 0, n_diff=n_diff,
                max_dist=int(dist.max(initial=0)))


def assert_parity(got: dict, ref: dict, where: str, exact: bool = True):
    """got/ref: name -> array; names starting with 'p' are bf16 bits."""
    for name in ref:
        rep = (bf16_report if name.startswith("p") else f32_report)(
            got[name], ref[name])
        assert rep["ok"], f"{where}: {name} outside the bar: {rep}"
        if exact:
            assert rep["exact"], f"{where}: {name} not bit-identical: {rep}"
