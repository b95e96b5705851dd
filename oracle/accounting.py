"""Memory and communication accounting of ZeRO data parallelism.

TEST INFRASTRUCTURE: see oracle/__init__.py.

Sources (page titles and sections):
* CS336 lecture 8 notes "Parallelism basics", core concepts: plain DDP with
  mixed-precision Adam holds 16 bytes per parameter (2 bf16 param, 2 bf16
  grad, 4 fp32 master, 4 + 4 Adam moments); ZeRO-1 holds (4 + K/N)*P with K
  the optimizer bytes; communication 2*P for ZeRO-1/2 and 3*P for ZeRO-3;
  FSDP code section: the "does it fit" table on 8 x 80 GB at 12 B/param.
* DDP-to-ZeRO blog, sections 1.1 and 3.1: the 7B example, 14 + 14 + 84 GB
  under DDP and the per-card figures for ZeRO-1/2/3 at 64 cards; section 2.2:
  a ring all-reduce moves about twice the gradient bytes per card.
"""

from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Bytes:
    """Bytes per parameter of each resident buffer."""
    param: int = 2          # bf16 working copy
    grad: int = 2           # bf16 gradient
    optim: int = 12         # fp32 master + m + v (K)

    @property
    def total(self) -> int:
        return self.param + self.grad + self.optim


MIXED = Bytes(2, 2, 12)     # 16 B/param, the pages' mixed-precision AdamW
PURE_BF16 = Bytes(2, 2, 8)  # 12 B/param, "pure bf16" (K = 8)


def per_rank_bytes(P: float, N: int, stage: int, b: Bytes = MIXED) -> float:
    """Resident model-state bytes of one rank (activations excluded).

    stage 0 = DDP (everything replicated), 1 = optimizer state sharded,
    2 = + gradients sharded, 3 = + parameters sharded.
    """
    if stage == 0:
        return P * b.total
    if stage == 1:
        return P * (b.param + b.grad) + P * b.optim / N
    if stage == 2:
        return P * b.param + P * (b.grad + b.optim) / N
    if stage == 3:
        return P * b.total / N
    raise ValueError("stage must be 0..3")


def max_params(mem_bytes: float, N: int, stage: int,
               b: Bytes = MIXED) -> float:
    """Largest parameter count whose model state fits in mem_bytes per rank."""
    return mem_bytes / per_rank_bytes(1.0, N, stage, b)


def comm_elems(P: float, stage: int) -> float:
    """Elements moved per step per the pages' counting: an all-reduce (DDP)
    or reduce-scatter + all-gather (ZeRO-1/2) is 2P; ZeRO-3 adds a second
    parameter all-gather for the backward, 3P."""
    return 3 * P if stage == 3 else 2 * P


def ring_allreduce_bytes_per_card(grad_bytes: float, N: int) -> float:
    """Bytes one card sends in a ring all-reduce: N-1 reduce-scatter steps
    and N-1 all-gather steps of grad_bytes/N each."""
    return 2 * (N - 1) * grad_bytes / N


def step_bytes_per_param(W: int) -> int:
    """Algorithmic HBM bytes per shard element of the fused step: read W bf16
    gradient slices and fp32 master/m/v, write master/m/v and the bf16
    parameter.  2W + 12 + 12 + 2."""
    return 2 * W + 26
