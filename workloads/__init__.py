"""Seeded synthetic inputs for the attention workloads (shared by tests, smoke and bench).

This module only draws random numbers and shapes tensors.  It holds none of the
attention arithmetic, so both the fp64 oracle and the HIP path can be fed from it
without sharing any of the method.

Recipe (the same everywhere):
  * ``torch.Generator('cpu').manual_seed(seed)``; by default ``seed`` is the
    workload number.
  * Draw order: Q, K, V, dO, each ``torch.randn`` fp32 N(0, 1) with its full
    shape ([B,Hq,S,d] for Q and dO, [B,Hkv,S,d] for K and V).
  * Long-context workload only: for each batch entry, ``floor(0.01 * S)`` distinct
    positions from ``torch.randperm(S)``; the K rows at those positions (all KV
    heads) are multiplied by 3 in fp32, giving large-max outlier scores.
  * Everything is then rounded to bf16 (round to nearest even) on the CPU.
The scale is ``1/sqrt(d)`` for every workload.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    number: int
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    d: int
    causal: bool
    passes: Tuple[str, ...]
    outlier_frac: float = 0.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def fwd_flop(self) -> float:
        """Algorithmic forward flop: 4*B*Hq*S^2*d, halved when causal."""
        f = 4.0 * self.B * self.Hq * self.S * self.S * self.d
        return f / 2 if self.causal else f

    def bwd_flop(self) -> float:
        """Algorithmic backward flop: 2.5x the forward (five products, recompute included)."""
        return 2.5 * self.fwd_flop()

    def describe(self) -> str:
        return (f"B={self.B} Hq={self.Hq} Hkv={self.Hkv} S={self.S} d={self.d} "
                f"{'causal' if self.causal else 'non-causal'}")


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny_fwd", 1, 2, 2, 128, 64, False, ("fwd",)),
    2: Workload(2, "prefill_fwd", 4, 16, 16, 2048, 128, True, ("fwd",)),
    3: Workload(3, "long_context_fwd", 1, 16, 16, 32768, 128, True, ("fwd",), outlier_frac=0.01),
    4: Workload(4, "bwd", 4, 16, 16, 4096, 128, True, ("fwd", "bwd")),
    5: Workload(5, "gqa_fwd_bwd", 2, 32, 8, 8192, 128, True, ("fwd", "bwd")),
    # Longer contexts and the non-causal long forward (the pages' long-context motivation:
    # throughput against S beyond 32k).
    6: Workload(6, "long_64k_fwd", 1, 8, 8, 65536, 128, True, ("fwd",)),
    7: Workload(7, "long_128k_fwd", 1, 4, 1, 131072, 128, True, ("fwd",)),
    8: Workload(8, "long_noncausal_fwd", 1, 16, 16, 32768, 128, False, ("fwd",)),
}


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """A packed (variable-length) forward batch: ``n`` sequences whose lengths are drawn
    log-uniformly in [min_len, max_len] from the workload's seed, laid end to end."""
    number: int
    name: str
    n: int
    min_len: int
    max_len: int
    Hq: int
    Hkv: int
    d: int
    causal: bool
    passes: Tuple[str, ...] = ("fwd",)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def lengths(self):
        g = torch.Generator("cpu").manual_seed(self.number)
        u = torch.empty(self.n, dtype=torch.float64).uniform_(math.log(self.min_len), math.log(self.max_len + 1), generator=g)
        return [min(self.max_len, max(self.min_len, int(x))) for x in torch.exp(u).floor().tolist()]

    def fwd_flop(self) -> float:
        """Algorithmic forward flop: sum over sequences of 4*Hq*len^2*d, halved when causal."""
        f = sum(4.0 * self.Hq * n * n * self.d for n in self.lengths())
        return f / 2 if self.causal else f

    def bwd_flop(self) -> float:
        """Algorithmic backward flop: 2.5 x the forward's (its five products)."""
        return 2.5 * self.fwd_flop()

    def describe(self) -> str:
        ls = self.lengths()
        return (f"{self.n} sequences, lengths {min(ls)}..{max(ls)} (total {sum(ls)} tokens), Hq={self.Hq} "
                f"Hkv={self.Hkv} d={self.d} {'causal' if self.causal else 'non-causal'}")


VARLEN_WORKLOADS: Dict[int, VarlenWorkload] = {
    # A prefill batch of prompts of mixed lengths (the pages' integration target: prefill
    # in SGLang/vLLM).
    9: VarlenWorkload(9, "varlen_prefill_fwd", 32, 256, 8192, 32, 8, 128, True),
    # A packed training batch of the same kind of mix: forward and backward.
    10: VarlenWorkload(10, "varlen_train_fwd_bwd", 32, 256, 8192, 32, 8, 128, True, ("fwd", "bwd")),
}


def make_varlen_tensors(lengths, Hq: int, Hkv: int, d: int, seed: int,
                        with_do: bool = False) -> Dict[str, torch.Tensor]:
    """Seeded packed bf16 CPU tensors: q [T,Hq,d], k, v [T,Hkv,d] (T = sum of lengths), drawn
    in that order as fp32 N(0,1) after ``seed`` and rounded to bf16 (with_do: then the
    upstream gradient do [T,Hq,d], drawn last, so q, k and v do not depend on it), and the
    int32 offsets cu_seqlens [n+1]."""
    g = torch.Generator("cpu").manual_seed(seed)
    T = int(sum(lengths))
    q = torch.randn((T, Hq, d), generator=g, dtype=torch.float32)
    k = torch.randn((T, Hkv, d), generator=g, dtype=torch.float32)
    v = torch.randn((T, Hkv, d), generator=g, dtype=torch.float32)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    out = {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16), "cu_seqlens": cu}
    if with_do:
        out["do"] = torch.randn((T, Hq, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return out


def make_varlen_inputs(w: VarlenWorkload, seed: int | None = None, with_do: bool = False) -> Dict[str, torch.Tensor]:
    """Inputs of the packed workload ``w`` (seed defaults to its number + 100, so that the
    tensor draws do not repeat the draws of its lengths)."""
    return make_varlen_tensors(w.lengths(), w.Hq, w.Hkv, w.d, w.number + 100 if seed is None else seed,
                               with_do=with_do)


def make_tensors(B: int, Hq: int, Hkv: int, S: int, d: int, seed: int,
                 outlier_frac: float = 0.0, with_do: bool = True) -> Dict[str, torch.Tensor]:
    """Seeded bf16 CPU tensors q, k, v (and do) following the recipe above."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, Hq, S, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, S, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, S, d), generator=g, dtype=torch.float32)
    do = torch.randn((B, Hq, S, d), generator=g, dtype=torch.float32) if with_do else None
    if outlier_frac > 0.0:
        n = int(math.floor(outlier_frac * S))
        for b in range(B):
            pos = torch.randperm(S, generator=g)[:n]
            k[b, :, pos, :] *= 3.0
    out = {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16)}
    if do is not None:
        out["do"] = do.to(torch.bfloat16)
    return out


def make_inputs(w: Workload, seed: int | None = None, with_do: bool = True) -> Dict[str, torch.Tensor]:
    """Inputs of workload ``w`` (seed defaults to the workload number)."""
    return make_tensors(w.B, w.Hq, w.Hkv, w.S, w.d, w.number if seed is None else seed,
                        w.outlier_frac, with_do)


def outlier_positions(w: Workload, seed: int | None = None):
    """The outlier positions per batch entry that ``make_inputs`` scaled (same draws)."""
    if w.outlier_frac <= 0.0:
        return [torch.empty(0, dtype=torch.long) for _ in range(w.B)]
    g = torch.Generator("cpu").manual_seed(w.number if seed is None else seed)
    for shape in ((w.B, w.Hq, w.S, w.d), (w.B, w.Hkv, w.S, w.d), (w.B, w.Hkv, w.S, w.d), (w.B, w.Hq, w.S, w.d)):
        torch.randn(shape, generator=g, dtype=torch.float32)
    n = int(math.floor(w.outlier_frac * w.S))
    return [torch.randperm(w.S, generator=g)[:n] for _ in range(w.B)]
