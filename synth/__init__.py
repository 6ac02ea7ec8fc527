"""Seeded synthetic inputs for the 4-bit-base LoRA linear.

This module is shared by the GPU path (bench, tests) and the CPU oracle. It
holds none of the method's arithmetic: it only draws random numbers, rounds
them to bf16 storage, and describes the layer shapes of the five workloads.

Workloads (rows ``M`` are tokens, a layer is ``K = d_in -> N = d_out``):

1. ``single``: one NF4 linear, M=256, K=N=1024, rank 16, alpha 32.
2. ``llama8b``: a Llama-3-8B-shaped layer set on M=4096 tokens, NF4 with
   64-element blocks: q and o 4096->4096, k and v 4096->1024, gate and up
   4096->14336, down 14336->4096; rank 16, alpha 32.
3. ``llama70b``: Llama-70B-shaped MXFP4 layers on M=8192 tokens: 8192->8192,
   8192->28672, 28672->8192; rank 64, alpha 128.
4. ``moe``: 64 experts with hidden 7168 and intermediate 2048 (gate and up
   7168->2048, down 2048->7168), MXFP4, rank 16, alpha 32; 4096 tokens are
   routed top-8 by N(0,1) logits, so the 32768 rows form variable-size
   groups, one per expert.
5. ``longctx``: M=32768 tokens, 5120->5120, NF4 with double-quantized
   scales, rank 128, alpha 256.
6. ``multilora``: the ``llama8b`` layer set with 16 rank-16 adapters over
   each layer's one NF4 base, the 4096 tokens split among the adapters at
   15 cut points drawn uniformly without replacement (groups of 1 to ~700
   rows).

Distributions (all drawn in float32 and rounded to bf16, round to nearest
even): X ~ N(0,1), dY ~ N(0,1), W ~ N(0, 0.02) (NF4 workloads) or
N(0, 0.015) (MXFP4 workloads), A ~ U(-1/sqrt(K), 1/sqrt(K)), B ~ N(0, 0.01).
Each tensor has its own numpy PCG64 stream seeded
``1000*workload + 10*layer + tensor_id`` (X=1, W=2, A=3, B=4, dY=5, logits=6).
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

NF4, NF4_DQ, MXFP4, NVFP4 = "nf4", "nf4_dq", "mxfp4", "nvfp4"
TID = {"X": 1, "W": 2, "A": 3, "B": 4, "dY": 5, "logits": 6}


@dataclass
class Layer:
    workload: int
    index: int
    name: str
    M: int
    K: int
    N: int
    r: int
    alpha: float
    fmt: str
    w_std: float
    experts: int = 1
    offsets: Optional[List[int]] = field(default=None)
    shared_base: bool = False        # groups are adapters over one W (not experts)

    @property
    def s(self):
        return self.alpha / self.r

    @property
    def block(self):
        return {MXFP4: 32, NVFP4: 16}.get(self.fmt, 64)

    def flops(self):
        """Algorithmic fwd+bwd flops: 4MNK + 6Mr(N+K) (no dW, Z kept)."""
        return 4 * self.M * self.N * self.K + 6 * self.M * self.r * (self.N + self.K)


WORKLOAD_NAMES = {1: "single", 2: "llama8b", 3: "llama70b", 4: "moe", 5: "longctx", 6: "multilora"}


def moe_routing(tokens=4096, experts=64, topk=8, seed=1000 * 4 + TID["logits"]):
    """Top-k routing of N(0,1) logits -> per-expert row counts and offsets.

    Softmax is monotone, so the top-k of the softmax is the top-k of the
    logits; equal logits go to the lower expert index.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    logits = rng.standard_normal((tokens, experts), dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    counts = np.bincount(order.reshape(-1), minlength=experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return order, counts, offsets


def layers(workload):
    """The layers of a workload, in order."""
    w = workload
    if w == 1:
        return [Layer(1, 0, "linear", 256, 1024, 1024, 16, 32.0, NF4, 0.02)]
    if w == 2:
        shapes = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
                  ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)]
        return [Layer(2, i, n, 4096, k, nn, 16, 32.0, NF4, 0.02) for i, (n, k, nn) in enumerate(shapes)]
    if w == 3:
        shapes = [("attn", 8192, 8192), ("up", 8192, 28672), ("down", 28672, 8192)]
        return [Layer(3, i, n, 8192, k, nn, 64, 128.0, MXFP4, 0.015) for i, (n, k, nn) in enumerate(shapes)]
    if w == 4:
        _, _, offs = moe_routing()
        offs = [int(v) for v in offs]
        M = offs[-1]
        shapes = [("gate", 7168, 2048), ("up", 7168, 2048), ("down", 2048, 7168)]
        return [Layer(4, i, n, M, k, nn, 16, 32.0, MXFP4, 0.015, experts=64, offsets=offs)
                for i, (n, k, nn) in enumerate(shapes)]
    if w == 5:
        return [Layer(5, 0, "proj", 32768, 5120, 5120, 128, 256.0, NF4_DQ, 0.02)]
    if w == 6:
        rng = np.random.Generator(np.random.PCG64(1000 * 6 + TID["logits"]))
        cuts = np.sort(rng.choice(np.arange(1, 4096), 15, replace=False))
        offs = [0] + [int(c) for c in cuts] + [4096]
        shapes = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
                  ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)]
        return [Layer(6, i, n, 4096, k, nn, 16, 32.0, NF4, 0.02, experts=16, offsets=offs, shared_base=True)
                for i, (n, k, nn) in enumerate(shapes)]
    raise ValueError(f"unknown workload {workload}")


def to_bf16(x):
    """float32 -> bf16 storage (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _rng(workload, layer, tid):
    return np.random.Generator(np.random.PCG64(1000 * workload + 10 * layer + tid))


def draw(workload, layer, name, shape, dist, scale):
    """One seeded tensor: dist 'normal' (std=scale) or 'uniform' (+-scale), as bf16."""
    rng = _rng(workload, layer, TID[name])
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
    elif dist == "uniform":
        x = rng.random(shape, dtype=np.float32)
        x = (x * np.float32(2.0) - np.float32(1.0)) * np.float32(scale)
    else:
        raise ValueError(dist)
    return to_bf16(x)


def inputs(lay, names=("X", "W", "A", "B", "dY")):
    """bf16 inputs of one layer. Grouped layers stack W, A, B per expert;
    layers whose groups share one base stack only A and B."""
    E = lay.experts
    out = {}
    for nm in names:
        if nm == "X":
            out[nm] = draw(lay.workload, lay.index, "X", (lay.M, lay.K), "normal", 1.0)
        elif nm == "dY":
            out[nm] = draw(lay.workload, lay.index, "dY", (lay.M, lay.N), "normal", 1.0)
        elif nm == "W":
            shape = (lay.N, lay.K) if E == 1 or lay.shared_base else (E, lay.N, lay.K)
            out[nm] = draw(lay.workload, lay.index, "W", shape, "normal", lay.w_std)
        elif nm == "A":
            shape = (lay.r, lay.K) if E == 1 else (E, lay.r, lay.K)
            out[nm] = draw(lay.workload, lay.index, "A", shape, "uniform", 1.0 / np.sqrt(lay.K))
        elif nm == "B":
            shape = (lay.N, lay.r) if E == 1 else (E, lay.N, lay.r)
            out[nm] = draw(lay.workload, lay.index, "B", shape, "normal", 0.01)
        else:
            raise KeyError(nm)
    return out


def small_layer(M, K, N, r, fmt=NF4, alpha=None, seed_workload=9, index=0, experts=1, offsets=None,
                w_std=0.02):
    """A layer of arbitrary small shape (tests), seeded like the workloads."""
    return Layer(seed_workload, index, "test", M, K, N, r, float(alpha if alpha is not None else 2 * r),
                 fmt, w_std, experts=experts, offsets=offsets)
