"""Synthetic workloads: parameter lists shaped like the pages' models.

Seeded, synthetic inputs only; no weights or datasets.  Each list is the
per-tensor element counts of an architecture in forward registration order.
This module holds no arithmetic of the optimizer step.

GPT-2-small shape: tied embeddings; wte, wpe, 12 blocks of [ln_1 w,b;
attn.c_attn w,b; attn.c_proj w,b; ln_2 w,b; mlp.c_fc w,b; mlp.c_proj w,b],
ln_f w,b.  Llama-shaped lists: untied; embed, L blocks of [attn_norm, q, k,
v, o, ffn_norm, gate, up, down], final norm, lm_head; no biases.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List


def tiny() -> List[int]:
    """Eight tensors: 512x512, 512x1024, 1024x256, four of 512, 1024x64."""
    return [512 * 512, 512 * 1024, 1024 * 256, 512, 512, 512, 512, 1024 * 64]


def gpt2_small(n_layer=12, d=768, ffn=3072, vocab=50257, ctx=1024) -> List[int]:
    out = [vocab * d, ctx * d]
    for _ in range(n_layer):
        out += [d, d,                       # ln_1
                d * 3 * d, 3 * d,           # c_attn
                d * d, d,                   # attn c_proj
                d, d,                       # ln_2
                d * ffn, ffn,               # c_fc
                ffn * d, d]                 # mlp c_proj
    out += [d, d]                           # ln_f
    return out


def llama(n_layer: int, d: int, kv: int, ffn: int, vocab: int) -> List[int]:
    out = [vocab * d]
    for _ in range(n_layer):
        out += [d,                          # attn_norm
                d * d, kv * d, kv * d,      # q, k, v
                d * d,                      # o
                d,                          # ffn_norm
                ffn * d, ffn * d, d * ffn]  # gate, up, down
    out += [d, vocab * d]                   # final norm, lm_head
    return out


def llama3_8b() -> List[int]:
    return llama(32, 4096, 1024, 14336, 128256)


def dense_7b() -> List[int]:
    return llama(32, 4096, 4096, 11008, 32000)


def llama3_70b() -> List[int]:
    return llama(80, 8192, 1024, 28672, 128256)


@dataclass(frozen=True)
class Workload:
    name: str
    numels: List[int] = field(repr=False)
    world: int
    rank: int
    grad_sigma: float
    master_sigma: float
    steps: int
    warm_steps: int = 0
    streaming: bool = False
    seed: int = 0


def presets() -> dict:
    """The five configurations: tiny parity case, GPT-2-small (parity), the
    Llama-3-8B-shaped W=8 shard (headline), 7B dense at W=64 and the
    Llama-3-70B-shaped streaming case at W=16."""
    return {
        "tiny": Workload("tiny", tiny(), 4, 0, 1e-3, 0.02, 3),
        "gpt2": Workload("gpt2-small", gpt2_small(), 8, 0, 1e-3, 0.02, 3,
                         warm_steps=10),
        "llama8b": Workload("llama3-8b", llama3_8b(), 8, 0, 1e-4, 0.02, 5),
        "dense7b": Workload("dense-7b", dense_7b(), 64, 0, 1e-4, 0.02, 5),
        "llama70b": Workload("llama3-70b", llama3_70b(), 16, 0, 1e-4, 0.02, 2,
                             streaming=True),
    }


# Generator tags: one independent stream per kind of synthetic input.
TAG_GRAD = 1
TAG_MASTER = 2
TAG_M = 3
TAG_V = 4
TAG_SENTINEL = 5
