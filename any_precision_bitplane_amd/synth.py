"""Seeded synthetic inputs for the fused mixed-precision MoE expert layer.

This module only draws random arrays and lays them out in the input format the
library and the oracle both accept. It holds none of the method's arithmetic:
no bit-plane decoding, no table lookup, no matrix product, no activation.

Input format (the same for every consumer):

* ``planes[e][m]``  uint32 ``[8][N][K/32]``: eight bit planes of one expert
  linear block, plane 0 first.  Bit ``j`` (LSB = 0) of word ``[p][n][c]`` is the
  ``p``-th most significant bit of the 8-bit code of weight ``(n, 32c + j)``.
  Uniform random 8-bit codes are the same thing as independent fair bits, so the
  words are drawn directly as uniform uint32 values.
* ``lut[e][m]``  fp16 bits (uint16) ``[504 * N]``: per-row tables for the
  bitwidths b = 3..8, concatenated b-major; the table of bitwidth b starts at
  element ``N * (2**b - 8)`` and is ``[N][2**b]``.  Each row of each table is
  ``2**b`` sorted draws of N(0, 0.02) rounded to fp16.
* ``q``  uint8 ``[E][2]``: committed bitwidth per block (column 0 gate_up,
  column 1 down).
* ``x``  fp16 ``[T][H]``, ``ids`` int32 ``[T][k]``, ``w`` fp32 ``[T][k]``.

Block shapes: gate_up is ``[2I][H]`` (rows ``[0, I)`` gate, ``[I, 2I)`` up), down
is ``[H][I]``.

The workloads follow the layer shapes of the models the PagedWeight summary
evaluates on (technical summary: PagedWeight, "Main contributions" item 4):
Qwen1.5-MoE-A2.7B and Mixtral-8x7B.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

GATE_UP = 0
DOWN = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    I: int
    E: int
    k: int
    T: int
    seed: int
    router: str = "softmax"      # "softmax" or "zipf"
    qmode: str = "uniform38"     # "uniform38", "hot8", "skewed"
    description: str = ""

    def block_shape(self, m: int):
        """(N, K) of module m: gate_up [2I x H], down [H x I]."""
        return (2 * self.I, self.H) if m == GATE_UP else (self.H, self.I)

    def with_T(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=T, name=f"{self.name.split('@')[0]}@T{T}")


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", H=256, I=512, E=8, k=2, T=16, seed=1000,
        description="tiny MoE layer: H=256, I=512, E=8, top-2, T=16"),
    "qwen_decode": Workload(
        "qwen_decode", H=2048, I=1408, E=60, k=4, T=4, seed=1001,
        description="Qwen1.5-MoE-A2.7B-shaped decode layer: H=2048, I=1408, "
                    "E=60 routed, top-4, T=4, bitwidths uniform in 3..8"),
    "qwen_batched": Workload(
        "qwen_batched", H=2048, I=1408, E=60, k=4, T=256, seed=1002,
        router="zipf", qmode="hot8",
        description="Qwen1.5-MoE-A2.7B-shaped batched decode: T=256, Zipf(1.1) "
                    "router skew, hottest 20% of experts at 8 bits, others in {3,4,5}"),
    "mixtral_decode": Workload(
        "mixtral_decode", H=4096, I=14336, E=8, k=2, T=8, seed=1003,
        description="Mixtral-8x7B-shaped decode layer: H=4096, I=14336, E=8, "
                    "top-2, T in {1, 8, 64}, bitwidths uniform in 3..8"),
    "mixtral_prefill": Workload(
        "mixtral_prefill", H=4096, I=14336, E=8, k=2, T=4096, seed=1004,
        qmode="skewed",
        description="Mixtral-8x7B-shaped prefill layer: T=4096, bitwidths skewed "
                    "(2 experts at 8, 3 at 4, 3 at 3; gate_up and down independent)"),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def draw_planes(seed: int, e: int, m: int, N: int, K: int) -> np.ndarray:
    """Eight uint32 plane words per 32 weights: uniform random 8-bit codes."""
    assert K % 32 == 0
    return _rng(seed, 1, e, m).integers(0, 2 ** 32, size=(8, N, K // 32), dtype=np.uint32)


def draw_lut(seed: int, e: int, m: int, N: int) -> np.ndarray:
    """b-major concatenation of per-row sorted fp16 tables, returned as uint16 bits."""
    rng = _rng(seed, 2, e, m)
    parts = []
    for b in range(3, 9):
        t = np.sort(rng.normal(0.0, 0.02, size=(N, 2 ** b)), axis=1).astype(np.float16)
        parts.append(t.reshape(-1))
    return np.concatenate(parts).view(np.uint16)


def draw_x(seed: int, T: int, H: int) -> np.ndarray:
    return _rng(seed, 4).standard_normal((T, H)).astype(np.float16)


def draw_router_weights(seed: int, E: int, H: int) -> np.ndarray:
    """Router matrix fp16 [E][H] ~ N(0, 1/H), so logits of N(0, 1) tokens are about N(0, 1)."""
    return (_rng(seed, 6).standard_normal((E, H)) / np.sqrt(H)).astype(np.float16)


def draw_sensitivity(seed: int, nblocks: int) -> np.ndarray:
    """Synthetic offline sensitivity scores fp32 [nblocks][6] for bitwidths 3..8:
    positive, decreasing in the bitwidth, zero-free (stand-ins for Hessian-weighted
    scores, which need trained weights)."""
    rng = _rng(seed, 7)
    steps = rng.exponential(1.0, size=(nblocks, 6)) * rng.lognormal(0.0, 1.0, size=(nblocks, 1))
    return np.cumsum(steps[:, ::-1], axis=1)[:, ::-1].astype(np.float32)


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=1, keepdims=True)


def draw_router(wl: Workload):
    """Top-k expert ids (int32 [T][k], descending logit, ties to the lower id) and
    routing weights (fp32 [T][k], softmax over the selected logits)."""
    T, E, k = wl.T, wl.E, wl.k
    if wl.router == "softmax":
        logits = _rng(wl.seed, 5).standard_normal((T, E))
    elif wl.router == "zipf":
        rng = _rng(wl.seed, 5)
        rank = rng.permutation(E)
        p = (rank + 1.0) ** -1.1
        p = p / p.sum()
        logits = np.log(p)[None, :] + rng.gumbel(0.0, 1.0, size=(T, E))
    else:
        raise ValueError(wl.router)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    w = _softmax_rows(sel).astype(np.float32)
    return ids, w


def draw_q(wl: Workload, ids: np.ndarray, w: np.ndarray) -> np.ndarray:
    E = wl.E
    rng = _rng(wl.seed, 3)
    if wl.qmode == "uniform38":
        q = rng.integers(3, 9, size=(E, 2))
    elif wl.qmode == "hot8":
        mass = np.zeros(E, dtype=np.float64)
        np.add.at(mass, ids.reshape(-1).astype(np.int64), w.reshape(-1).astype(np.float64))
        nhot = int(math.ceil(0.2 * E))
        hot = np.argsort(-mass, kind="stable")[:nhot]
        q = rng.choice(np.array([3, 4, 5]), size=(E, 2))
        q[hot, :] = 8
    elif wl.qmode == "skewed":
        base = np.array([8, 8, 4, 4, 4, 3, 3, 3])
        assert E == len(base)
        q = np.stack([rng.permutation(base), rng.permutation(base)], axis=1)
    else:
        raise ValueError(wl.qmode)
    return np.ascontiguousarray(q.astype(np.uint8))


@dataclasses.dataclass
class Layer:
    wl: Workload
    planes: List[List[np.ndarray]]   # [E][2] uint32 [8][N][K/32]
    luts: List[List[np.ndarray]]     # [E][2] uint16 [504 N]
    q: np.ndarray                    # uint8 [E][2]
    x: np.ndarray                    # fp16 [T][H]
    ids: np.ndarray                  # int32 [T][k]
    w: np.ndarray                    # fp32 [T][k]

    def active_experts(self) -> np.ndarray:
        v = self.ids.reshape(-1)
        v = v[(v >= 0) & (v < self.wl.E)]
        return np.unique(v)


def make_layer(wl: Workload, experts: Optional[List[int]] = None) -> Layer:
    """Draw a whole layer.  ``experts`` restricts which blocks get drawn
    (others are left as zero arrays of the right shape), which keeps the
    cost of drawing big layers down when only the routed experts are read."""
    ids, w = draw_router(wl)
    q = draw_q(wl, ids, w)
    x = draw_x(wl.seed, wl.T, wl.H)
    planes, luts = [], []
    for e in range(wl.E):
        pe, le = [], []
        for m in (GATE_UP, DOWN):
            N, K = wl.block_shape(m)
            if experts is None or e in experts:
                pe.append(draw_planes(wl.seed, e, m, N, K))
                le.append(draw_lut(wl.seed, e, m, N))
            else:
                pe.append(np.zeros((8, N, K // 32), dtype=np.uint32))
                le.append(np.zeros(504 * N, dtype=np.uint16))
        planes.append(pe)
        luts.append(le)
    return Layer(wl, planes, luts, q, x, ids, w)


def make_routed_layer(wl: Workload) -> Layer:
    """Like make_layer, but only the experts the router selects get drawn."""
    ids, _ = draw_router(wl)
    v = ids.reshape(-1)
    return make_layer(wl, experts=sorted(set(int(e) for e in v)))
