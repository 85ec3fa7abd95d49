"""CPU oracle for the quality-aware bitwidth planner (test infrastructure).

Plain Python statement of the planner; only the tests may use it.  It shares
no code with the library and imports nothing from it.

Source: "Technical summary: PagedWeight", gist.science (ja) and its Hindi
twin, Core components 2 (quality-aware runtime planner):
  - offline global sensitivity: a Hessian-weighted score per linear block
    estimates how much the block suffers from quantization;
  - online routing statistics: experts' routing mass is tracked; frequently
    routed (hot) experts are protected by higher bitwidth floors and damage
    multipliers;
  - prompt residuals: a prompt-specific correction of the sensitivity;
  - the planner scores the damage of candidate bitwidth reductions and, when
    memory pressure sets a target, greedily picks the reductions with the
    least damage per byte saved until the target is met.

Readings (the pages give no formulas):
  - the damage of running block b at bitwidth q is
        D_b(q) = mu_b * (S_b(q) + R_b(q))
    with S the offline score table, R the prompt correction (0 if absent) and
    mu_b the hot multiplier (1 for blocks of experts that are not hot);
  - hot experts: among experts with positive routing mass, the
    ceil(hot_fraction * E) largest masses (equal masses: lower expert id);
  - floors: floor_hot for blocks of hot experts, floor_cold otherwise; a block
    below its floor is first raised to it;
  - a reduction step lowers one block by one bit; it saves that block's plane
    bytes and costs D_b(q-1) - D_b(q); the step with the smallest cost per
    byte is taken first (equal: lower block index), until the resident plane
    bytes fit the budget or no step is left;
  - when the bytes already fit, the mirror step restores bits: raising block b
    by one bit gains D_b(q) - D_b(q+1) for its plane bytes; the step with the
    largest gain per byte that still fits is taken (equal: lower block index),
    until none fits;
  - costs and gains per byte are evaluated in fp64 as
        (mu * (S[q'] + R[q']) - mu * (S[q] + R[q])) / plane_bytes
    with S, R fp32 inputs widened to fp64.

Parity pins: tests/test_planner_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

MIN_BITS = 3
MAX_BITS = 8


def hot_experts(mass, hot_fraction: float) -> set:
    """Ids of the hot experts."""
    if mass is None:
        return set()
    E = len(mass)
    n = int(math.ceil(hot_fraction * E))
    ranked = sorted((e for e in range(E) if mass[e] > 0), key=lambda e: (-float(mass[e]), e))
    return set(ranked[:n])


def damage(mu: float, S_row, R_row, q: int) -> float:
    """D_b(q) in fp64."""
    s = float(np.float32(S_row[q - MIN_BITS]))
    r = float(np.float32(R_row[q - MIN_BITS])) if R_row is not None else 0.0
    return mu * (s + r)


def plan(q_cur, plane_bytes, expert_of, S, R, mass, hot_fraction, floor_cold, floor_hot, hot_multiplier,
         budget_bytes):
    """Returns (q_out list, resident plane bytes, fits budget)."""
    B = len(q_cur)
    hot = hot_experts(mass, hot_fraction)
    mu = [float(np.float32(hot_multiplier)) if expert_of[b] in hot else 1.0 for b in range(B)]
    floor = [floor_hot if expert_of[b] in hot else floor_cold for b in range(B)]
    q = [max(int(q_cur[b]), floor[b]) for b in range(B)]
    used = sum(q[b] * int(plane_bytes[b]) for b in range(B))
    Rr = (lambda b: None) if R is None else (lambda b: R[b])

    if used > budget_bytes:
        while used > budget_bytes:
            best, best_key = None, None
            for b in range(B):
                if q[b] - 1 < floor[b]:
                    continue
                cost = damage(mu[b], S[b], Rr(b), q[b] - 1) - damage(mu[b], S[b], Rr(b), q[b])
                key = cost / float(plane_bytes[b])
                if best is None or key < best_key:
                    best, best_key = b, key
            if best is None:
                break
            q[best] -= 1
            used -= int(plane_bytes[best])
    else:
        while True:
            best, best_key = None, None
            for b in range(B):
                if q[b] + 1 > MAX_BITS or used + int(plane_bytes[b]) > budget_bytes:
                    continue
                gain = damage(mu[b], S[b], Rr(b), q[b]) - damage(mu[b], S[b], Rr(b), q[b] + 1)
                key = gain / float(plane_bytes[b])
                if best is None or key > best_key:
                    best, best_key = b, key
            if best is None:
                break
            q[best] += 1
            used += int(plane_bytes[best])
    return q, used, used <= budget_bytes
