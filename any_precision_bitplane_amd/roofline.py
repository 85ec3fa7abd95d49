"""Algorithmic work of one layer call: the bytes the method must move and the
flops it must do, independent of how the kernels move them.

bytes = sum over routed blocks (e, m) of  q/8 * N*K  (planes 0..q-1)
                                        + N * 2^q * 2 (the bitwidth-q tables)
        + activations in and out (x: T*H*2, y: T*H*2) + router ids and weights
          (T*k*8) + the q table (2E).
Intermediates (h, o) are implementation traffic and are not counted.
flops = 2 * (T*k) * (2I*H + H*I) = 6 T k H I.

MI355X peaks used for the fractions: HBM3E 8.0 TB/s; dense fp16 MFMA
2.5 PFLOP/s.
"""
from __future__ import annotations

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0


def routed_experts(ids: np.ndarray, E: int) -> np.ndarray:
    v = np.asarray(ids).reshape(-1)
    return np.unique(v[(v >= 0) & (v < E)])


def block_bytes(N: int, K: int, q: int) -> int:
    return q * N * K // 8 + N * (2 ** q) * 2


def layer_bytes(q, ids, H, I, E, T, k) -> int:
    total = 0
    for e in routed_experts(ids, E):
        total += block_bytes(2 * I, H, int(q[e][0])) + block_bytes(H, I, int(q[e][1]))
    return total + 2 * T * H * 2 + T * k * 8 + 2 * E


def module_bytes(q, ids, H, I, E, T, k, module: int) -> int:
    """Bytes of one product: the routed blocks of that module plus its input
    activations (x for gate_up) or its output (y for down) and the router
    arrays it reads."""
    total = 0
    for e in routed_experts(ids, E):
        N, K = (2 * I, H) if module == 0 else (H, I)
        total += block_bytes(N, K, int(q[e][module]))
    return total + T * H * 2 + T * k * 4


def layer_flops(T, k, H, I) -> int:
    return 6 * T * k * H * I


def module_flops(T, k, H, I, module: int) -> int:
    """Flops of one product: 2 per weight per routed slot (gate_up 2I x H, down H x I)."""
    return 2 * T * k * (2 * I * H if module == 0 else H * I)


def bound(flops: float, nbytes: float) -> str:
    """'mfma' when the arithmetic intensity exceeds the ridge point of the two peaks."""
    ridge = MFMA_FP16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    return "mfma" if flops / max(nbytes, 1) > ridge else "hbm"
