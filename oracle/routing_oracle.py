"""CPU oracle for the router and the online routing statistics (test
infrastructure).

A plain fp64 statement of what the router kernel computes.  Only the tests,
the smoke check and the benchmark's CPU-baseline leg may use it; it shares no
code with the HIP library and imports nothing from it.

Sources:

* [PW] "Technical summary: PagedWeight", gist.science (ja) and its Hindi twin,
  Core components 2, second bullet ("Online routing statistics"): the system
  tracks each expert's routing mass, i.e. how often it is selected and with
  what weight; frequently routed ("hot") experts get protected.
* The configuration of the synthetic tiny layer: routing weights are a softmax
  over the top-k router logits.

The pages do not print the router, so the plainest reading of a top-k MoE
router is used:

* logits[t, e] = sum_h x[t, h] * Wr[e, h]  (fp16 inputs, exact products in fp64);
* the k selected experts of token t are the k largest logits, listed in
  descending logit order; equal logits list the lower expert id first;
* w[t, j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the selected logits
  (l_0 the largest), i.e. a softmax over the top-k;
* routing statistics of a batch: count[e] = number of (t, j) slots routed to
  e, mass[e] = sum of their weights.  Statistics accumulate over batches.

Parity pins: tests/test_routing_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np


def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """fp64 [T][E] router logits from fp16 x [T][H] and fp16 Wr [E][H]."""
    return np.asarray(x, dtype=np.float16).astype(np.float64) @ np.asarray(wr, dtype=np.float16).astype(np.float64).T


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """int32 [T][k]: per token, expert ids ordered by (-logit, id)."""
    T, E = logits.shape
    assert 1 <= k <= E
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))
        ids[t] = order[:k]
    return ids


def topk_softmax(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """fp64 [T][k]: softmax over the selected logits of each token."""
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def route(x: np.ndarray, wr: np.ndarray, k: int):
    """(ids int32 [T][k], w fp64 [T][k], logits fp64 [T][E])."""
    logits = router_logits(x, wr)
    ids = topk_select(logits, k)
    return ids, topk_softmax(logits, ids), logits


def routing_stats(ids: np.ndarray, w: np.ndarray, E: int):
    """(count int64 [E], mass fp64 [E]) of one batch ([PW] Core components 2)."""
    count = np.zeros(E, dtype=np.int64)
    mass = np.zeros(E, dtype=np.float64)
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            count[e] += 1
            mass[e] += float(w[t, j])
    return count, mass
