"""Pins of the planner oracle to things other than itself: a hand-worked plan,
exhaustive search on tiny instances where the greedy is provably optimal,
invariants of a budgeted greedy, and planted mistakes the pins must catch."""
import itertools

import numpy as np
import pytest

import oracle.planner_oracle as po

# hand-worked instance: three blocks of 100-byte planes, experts 0, 1, 2
S_HAND = [[8, 4, 2, 1, 0.5, 0],       # marginal cost of 8->7, 7->6, 6->5, 5->4, 4->3: 0.5, 0.5, 1, 2, 4
          [16, 8, 4, 2, 1, 0],        # 1, 1, 2, 4, 8
          [3, 2.5, 2, 1.5, 1, 0.5]]   # 0.5 each
PB = [100, 100, 100]


def hand(q_cur, budget, mass=None, frac=0.0, floor_hot=3, mult=1.0):
    return po.plan(q_cur, PB, [0, 1, 2], S_HAND, None, mass, frac, 3, floor_hot, mult, budget)


def test_hand_worked_reduction():
    # 2400 -> 1900 bytes: five planes.  Costs per byte: b0 .005, b1 .01, b2 .005 -> b0 (lower id), b0 again
    # (.005), then b0 costs .01 and b2 .005 three times: [6, 8, 5].
    q, used, ok = hand([8, 8, 8], 1900)
    assert q == [6, 8, 5] and used == 1900 and ok


def test_hand_worked_hot_expert():
    # expert 0 hot (floor 7, damage x2): b0's first step costs .01, so b2 goes to its floor 3 first
    q, used, ok = hand([8, 8, 8], 1900, mass=[5.0, 0.0, 0.0], frac=1 / 3, floor_hot=7, mult=2.0)
    assert q == [8, 8, 3] and used == 1900
    # two more planes: b0 and b1 tie at .01 -> b0 first (lower id); b0 then sits on its floor
    q, used, ok = hand([8, 8, 8], 1700, mass=[5.0, 0.0, 0.0], frac=1 / 3, floor_hot=7, mult=2.0)
    assert q == [7, 7, 3] and ok
    # a hot block below its floor is raised to it first
    q, _, _ = hand([3, 8, 8], 10 ** 6, mass=[5.0, 0.0, 0.0], frac=1 / 3, floor_hot=7, mult=2.0)
    assert q[0] >= 7


def test_hand_worked_restoration():
    # 900 -> 1300 bytes: gains per byte b0 .04, b1 .08, b2 .005 -> b1; then b0/b1 tie at .04 -> b0;
    # then b1 (.04); then b0/b1 tie at .02 -> b0: [5, 5, 3]
    q, used, ok = hand([3, 3, 3], 1300)
    assert q == [5, 5, 3] and used == 1300 and ok
    # budget below the floors: nothing can be saved, reported as not fitting
    q, used, ok = hand([3, 3, 3], 200)
    assert q == [3, 3, 3] and used == 900 and not ok


def convex_table(rng):
    inc = np.sort(rng.uniform(0.0, 1.0, 5))[::-1]          # cost of 4->3 largest ... 8->7 smallest
    S = np.concatenate([np.cumsum(inc[::-1])[::-1], [0.0]])  # S(3..8), S(8) = 0, convex
    return S.astype(np.float32)


@pytest.mark.parametrize("seed", range(12))
def test_greedy_is_optimal_on_convex_equal_size_instances(seed):
    # equal plane bytes and convex damage: the greedy's total damage equals the exhaustive optimum
    rng = np.random.default_rng(seed)
    B = 4
    S = [convex_table(rng) for _ in range(B)]
    q_cur = [8] * B
    budget = int(rng.integers(3 * B, 8 * B + 1)) * 64
    q, used, ok = po.plan(q_cur, [64] * B, list(range(B)), S, None, None, 0.0, 3, 3, 1.0, budget)
    assert ok and used <= budget
    best = None
    for qs in itertools.product(range(3, 9), repeat=B):
        if sum(qs) * 64 > budget:
            continue
        d = sum(float(S[b][qs[b] - 3]) for b in range(B))
        best = d if best is None else min(best, d)
    got = sum(float(S[b][q[b] - 3]) for b in range(B))
    assert abs(got - best) < 1e-9


def random_instance(rng, B=24, E=12):
    S = [np.sort(rng.uniform(0, 5, 6))[::-1].astype(np.float32) for _ in range(B)]
    R = rng.normal(0, 0.1, (B, 6)).astype(np.float32)
    pb = rng.integers(1, 50, B) * 256
    expert_of = [b // 2 for b in range(B)]
    mass = rng.uniform(0, 10, E) * (rng.uniform(0, 1, E) > 0.2)
    q_cur = rng.integers(3, 9, B)
    return S, R, pb, expert_of, mass, q_cur


@pytest.mark.parametrize("seed", range(6))
def test_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    S, R, pb, expert_of, mass, q_cur = random_instance(rng)
    args = dict(plane_bytes=pb, expert_of=expert_of, S=S, R=R, mass=mass, hot_fraction=0.25, floor_cold=3,
                floor_hot=5, hot_multiplier=3.0)
    hot = po.hot_experts(mass, 0.25)
    assert len(hot) == min(3, int((mass > 0).sum()))
    floors = [5 if expert_of[b] in hot else 3 for b in range(len(pb))]
    for budget in sorted(rng.integers(int(sum(pb) * 3), int(sum(pb) * 8), 8)):
        q, used, ok = po.plan(q_cur=q_cur, budget_bytes=int(budget), **args)
        assert used == sum(q[b] * int(pb[b]) for b in range(len(pb)))
        assert all(floors[b] <= q[b] <= 8 for b in range(len(pb)))
        feasible = sum(floors[b] * int(pb[b]) for b in range(len(pb))) <= budget
        assert ok == feasible
        if ok:
            assert used <= budget
        start = [max(int(q_cur[b]), floors[b]) for b in range(len(pb))]
        if sum(start[b] * int(pb[b]) for b in range(len(pb))) > budget:
            assert all(q[b] <= start[b] for b in range(len(pb)))       # only reductions
        else:
            assert all(q[b] >= start[b] for b in range(len(pb)))       # only restorations


@pytest.mark.parametrize("seed", range(4))
def test_reduction_is_a_prefix_of_one_sequence(seed):
    rng = np.random.default_rng(200 + seed)
    S, R, pb, expert_of, mass, _ = random_instance(rng)
    q_cur = [8] * len(pb)
    args = dict(plane_bytes=pb, expert_of=expert_of, S=S, R=R, mass=mass, hot_fraction=0.25, floor_cold=3,
                floor_hot=5, hot_multiplier=3.0)
    top = sum(8 * int(p) for p in pb)
    budgets = sorted(set(int(b) for b in rng.integers(int(top * 0.45), top, 10)), reverse=True)
    prev = None
    for budget in budgets:
        q, _, _ = po.plan(q_cur=q_cur, budget_bytes=budget, **args)
        if prev is not None:
            assert all(q[b] <= prev[b] for b in range(len(pb)))
        prev = q


def test_planted_mistakes_are_caught(monkeypatch):
    good = po.damage

    def no_multiplier(mu, S_row, R_row, q):
        return good(1.0, S_row, R_row, q)

    def sign_flipped(mu, S_row, R_row, q):
        return -good(mu, S_row, R_row, q)

    for fn in (no_multiplier, sign_flipped):
        with monkeypatch.context() as m:
            m.setattr(po, "damage", fn)
            results = (hand([8, 8, 8], 1900), hand([8, 8, 8], 1900, mass=[5.0, 0, 0], frac=1 / 3, floor_hot=7,
                                                    mult=2.0), hand([3, 3, 3], 1300))
            assert [r[0] for r in results] != [[6, 8, 5], [8, 8, 3], [5, 5, 3]], fn.__name__

    def wrong_hot(mass, frac):
        return set()

    with monkeypatch.context() as m:
        m.setattr(po, "hot_experts", wrong_hot)
        assert hand([8, 8, 8], 1900, mass=[5.0, 0, 0], frac=1 / 3, floor_hot=7, mult=2.0)[0] != [8, 8, 3]
