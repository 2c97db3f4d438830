"""Seeded synthetic inputs and the workload shapes they follow.

This module is shared by the oracle tests, the HIP parity tests and the benchmark. It
holds no attention arithmetic: only shapes and a seeded N(0, 1) generator. Values are
drawn in fp32 by a torch CPU generator and rounded to bf16 (round-to-nearest-even) when
the workload is bf16, so every consumer sees the same stored values.

Shapes follow the pages' settings: a 7B dense model sharded over one 8-GPU node
("Folding Tensor and Sequence Parallelism ...", section 4, results on MI300X nodes of
8 GPUs with a 7B dense model, sequence lengths 16K-128K), the 24-query / 4-KV-head,
head-dim 256 attention and its 262,144-token context ("Tensor, pipeline e sequence
parallelism", section 01, GQA and sequence-parallel paragraphs), and the Ulysses
head-subset layout (same lesson page, sequence-parallel paragraph; "AutoSP ...",
section 2.A, buffer resizing).
"""

from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S_total: int
    D: int
    ranks: tuple
    Hq: int
    Hkv: int
    dh: int
    dtype: str  # "f32" or "bf16"
    index: int  # seed family

    @property
    def S_local(self) -> int:
        return self.S_total // self.D

    @property
    def C(self) -> int:
        return self.S_total // (2 * self.D)

    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = [
    Workload("tiny_zigzag_gqa_f32", 1, 512, 4, (1,), 4, 1, 64, "f32", 0),
    Workload("tsp_7b_shard_s32k", 1, 32768, 8, (3,), 32, 32, 128, "bf16", 1),
    Workload("gqa_shard_s64k", 1, 65536, 4, (2,), 24, 4, 256, "bf16", 2),
    Workload("ulysses_head_subset_s128k", 1, 131072, 1, (0,), 4, 4, 128, "bf16", 3),
    Workload("long_context_s256k", 1, 262144, 8, (0, 7), 24, 4, 256, "bf16", 4),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def _randn(shape, seed: int, dtype) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    return x.to(dtype)


def seeds(index: int, rank: int):
    """(q_local, k_full, v_full, full-sequence q) seeds of a workload family."""
    return 1000 * index + 10 * rank + 1, 1000 * index + 2, 1000 * index + 3, 1000 * index + 1


def make_inputs(w: Workload, rank: int, dtype=None):
    """CPU tensors q_local [B,S_local,Hq,dh], k_full, v_full [B,S_total,Hkv,dh]."""
    dt = w.torch_dtype() if dtype is None else dtype
    sq, sk, sv, _ = seeds(w.index, rank)
    q = _randn((w.B, w.S_local, w.Hq, w.dh), sq, dt)
    k = _randn((w.B, w.S_total, w.Hkv, w.dh), sk, dt)
    v = _randn((w.B, w.S_total, w.Hkv, w.dh), sv, dt)
    return q, k, v


def make_full_q(w: Workload, dtype=None) -> torch.Tensor:
    """Full-sequence queries [B, S_total, Hq, dh] (for the shard-concatenation identity)."""
    dt = w.torch_dtype() if dtype is None else dtype
    return _randn((w.B, w.S_total, w.Hq, w.dh), seeds(w.index, 0)[3], dt)


def make_custom(B, S_total, D, Hq, Hkv, dh, dtype, seed):
    """Inputs of an arbitrary shape (small parity cases): (q_local, k_full, v_full)."""
    S_local = S_total // D
    q = _randn((B, S_local, Hq, dh), seed + 1, dtype)
    k = _randn((B, S_total, Hkv, dh), seed + 2, dtype)
    v = _randn((B, S_total, Hkv, dh), seed + 3, dtype)
    return q, k, v


def make_grad(shape, seed: int, dtype) -> torch.Tensor:
    """A seeded upstream gradient (N(0, 1), rounded like the inputs) for backward tests."""
    return _randn(tuple(shape), seed, dtype)
