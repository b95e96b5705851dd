"""Pins of oracle/accounting.py against the figures the pages print
(tests/golden/pages_accounting.json, each entry cites its page and section).
"""

import json
import os

import pytest

from oracle import accounting as A

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "pages_accounting.json")))


def near_printed(x, printed, digits):
    return abs(x - printed) <= 10.0 ** (-digits) + 1e-12


def test_bytes_per_param():
    g = GOLD["bytes_per_param"]
    assert A.MIXED.param == g["param"] and A.MIXED.grad == g["grad"]
    assert A.MIXED.optim == g["master"] + g["adam_m"] + g["adam_v"]
    assert A.MIXED.total == g["total"]


@pytest.mark.parametrize("row", GOLD["memory_7b"]["rows"],
                         ids=lambda r: f"stage{r['stage']}")
def test_memory_7b(row):
    g = GOLD["memory_7b"]
    gb = A.per_rank_bytes(g["params"], g["cards"], row["stage"]) / 1e9
    assert near_printed(gb, row["printed_gb"], row["digits"])
    if "parts_gb" in row:
        P = g["params"]
        assert [P * A.MIXED.param / 1e9, P * A.MIXED.grad / 1e9,
                P * A.MIXED.optim / 1e9] == row["parts_gb"]


@pytest.mark.parametrize("row", GOLD["fit_table"]["rows"],
                         ids=lambda r: f"stage{r['stage']}")
def test_fit_table(row):
    g = GOLD["fit_table"]
    assert A.PURE_BF16.total == g["bytes_per_param"]
    p = A.max_params(g["mem_gb"] * 1e9, g["cards"], row["stage"],
                     A.PURE_BF16) / 1e9
    assert near_printed(p, row["printed_b"], row["digits"])


def test_comm_volume():
    g = GOLD["comm_volume"]
    P = 1.0
    assert A.comm_elems(P, 1) == g["zero1_over_params"] * P
    assert A.comm_elems(P, 2) == A.comm_elems(P, 0)   # same as DDP
    assert A.comm_elems(P, 3) == g["zero3_over_params"] * P
    assert A.comm_elems(P, 3) / A.comm_elems(P, 0) == g["zero3_over_ddp"]


def test_ring_allreduce_about_twice_the_gradients():
    g = GOLD["ring_allreduce_7b"]
    for N in (8, 64, 1024):
        b = A.ring_allreduce_bytes_per_card(g["grad_gb"], N)
        assert b < 2 * g["grad_gb"] and b >= 1.75 * g["grad_gb"]
    assert A.ring_allreduce_bytes_per_card(g["grad_gb"], 10 ** 9) == \
        pytest.approx(g["printed_gb"], rel=1e-6)


@pytest.mark.parametrize("W", [1, 4, 8, 16, 64])
def test_step_bytes_follow_the_16_byte_accounting(W):
    """The fused step reads W bf16 gradient values and the fp32 master, m, v
    of each shard element, writes master, m, v and the bf16 parameter."""
    b = A.MIXED
    assert A.step_bytes_per_param(W) == W * b.grad + 2 * b.optim + b.param
