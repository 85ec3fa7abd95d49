"""The library's planner (C ABI, host code) against the planner oracle: the
same integer plan, resident bytes and fit flag on random instances (both sides
evaluate costs in fp64 in the same order), plus argument checks."""
import numpy as np
import pytest

import oracle.planner_oracle as po
from any_precision_bitplane_amd import binding as B


@pytest.fixture(scope="module")
def lib():
    return B.load()


def instance(rng, B_, E, with_R, with_mass, ties):
    if ties:   # few distinct values: many equal costs, so the tie rule decides
        S = np.sort(rng.integers(0, 4, (B_, 6)).astype(np.float32), axis=1)[:, ::-1].copy()
        pb = np.full(B_, 512, np.int64)
    else:
        S = np.sort(rng.uniform(0, 5, (B_, 6)).astype(np.float32), axis=1)[:, ::-1].copy()
        pb = rng.integers(1, 400, B_).astype(np.int64) * 256
    R = rng.normal(0, 0.2, (B_, 6)).astype(np.float32) if with_R else None
    eo = np.sort(rng.integers(0, E, B_)).astype(np.int32)
    mass = None
    if with_mass:
        mass = (rng.uniform(0, 10, E) * (rng.uniform(0, 1, E) > 0.3)).astype(np.float32)
        if ties:
            mass = np.round(mass).astype(np.float32)
    q_cur = rng.integers(3, 9, B_).astype(np.int32)
    return S, R, pb, eo, mass, q_cur


@pytest.mark.parametrize("seed", range(40))
def test_matches_oracle(lib, seed):
    rng = np.random.default_rng(seed)
    B_ = int(rng.choice([1, 3, 16, 120, 240]))
    E = int(rng.integers(1, 64))
    S, R, pb, eo, mass, q_cur = instance(rng, B_, E, seed % 2 == 0, seed % 3 != 0, seed % 4 == 1)
    frac = float(rng.choice([0.0, 0.2, 0.25, 1 / 3, 1.0]))
    floor_cold = int(rng.integers(3, 6))
    floor_hot = int(rng.integers(floor_cold, 9))
    mult = float(np.float32(rng.choice([1.0, 2.0, 3.5])))
    full = int((8 * pb).sum())
    for budget in [0, int(full * 0.4), int(full * 0.6), int(full * 0.8), full, full * 2,
                   int(rng.integers(0, full + 1))]:
        st, q, used, fits = B.pw_plan_bitwidths(q_cur, pb, eo, S, R, mass, frac, floor_cold, floor_hot, mult,
                                                budget)
        oq, oused, ofits = po.plan(q_cur.tolist(), pb.tolist(), eo.tolist(), S, R, mass, frac, floor_cold,
                                   floor_hot, mult, budget)
        assert st == B.PW_OK
        assert q.tolist() == oq, (seed, budget)
        assert used == oused and fits == ofits


def test_multi_layer_scale(lib):
    # 24 Qwen-shaped layers (2880 blocks) plan in well under a second
    import time
    rng = np.random.default_rng(5)
    B_ = 24 * 120
    S = np.sort(rng.uniform(0, 5, (B_, 6)).astype(np.float32), axis=1)[:, ::-1].copy()
    pb = np.array([2816 * 2048 // 8 if b % 2 == 0 else 2048 * 1408 // 8 for b in range(B_)], np.int64)
    eo = (np.arange(B_) // 2).astype(np.int32)
    q_cur = np.full(B_, 8, np.int32)
    t0 = time.time()
    st, q, used, fits = B.pw_plan_bitwidths(q_cur, pb, eo, S, budget_bytes=int((pb * 4).sum()))
    assert st == B.PW_OK and fits and used <= int((pb * 4).sum())
    assert time.time() - t0 < 1.0


def test_rejects_bad_arguments(lib):
    S = np.ones((2, 6), np.float32)
    args = ([8, 8], [256, 256], [0, 1], S)
    assert B.pw_plan_bitwidths([8, 9], *args[1:], budget_bytes=1, check=False)[0] == B.PW_ERR_BITWIDTH
    assert B.pw_plan_bitwidths(*args, floor_cold=2, budget_bytes=1, check=False)[0] == B.PW_ERR_BITWIDTH
    assert B.pw_plan_bitwidths([8, 8], [256, 0], [0, 1], S, budget_bytes=1, check=False)[0] == B.PW_ERR_INVALID_ARG
    assert B.pw_plan_bitwidths([8, 8], [256, 256], [0, 5], S, routing_mass=np.ones(2, np.float32),
                               budget_bytes=1, check=False)[0] == B.PW_ERR_INVALID_ARG
    assert lib.pw_plan_bitwidths(None, None, 0, None, None, None) == B.PW_ERR_INVALID_ARG
