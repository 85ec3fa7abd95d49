"""GPU tests of the weight pager through the C ABI: bitwidth requests, page
movement, safe-boundary commits ("Technical summary: PagedWeight", Core
components 1 third bullet and Core components 3 first bullet).

The forward's output is deterministic, so a layer served from pager-managed
storage must give the same bits as the same layer served from static storage
with the same q table; one case per test is also checked against the oracle.
Every case prints what it runs before it launches anything.
"""
import sys

import numpy as np
import pytest

import oracle.pagedweight_oracle as orc
from any_precision_bitplane_amd import binding as B
from any_precision_bitplane_amd import synth

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_ABS = 2e-2
ALIGN = 256


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    B.load()
    return _t


@pytest.fixture(scope="module")
def tiny():
    return synth.make_layer(synth.WORKLOADS["tiny"])


@pytest.fixture(scope="module")
def static(torch, tiny):
    from any_precision_bitplane_amd.device import DeviceLayer
    return DeviceLayer(tiny)


def rnd(n):
    return (n + ALIGN - 1) // ALIGN * ALIGN


def static_y(torch, static, q, path=B.PW_PATH_AUTO):
    static.set_q(np.asarray(q, np.uint8).reshape(-1, 2))
    static.forward(B.make_options(path=path))
    torch.cuda.synchronize()
    return static.y.cpu().numpy().view(np.uint16).copy()


def paged_y(torch, paged, path=B.PW_PATH_AUTO):
    paged.forward(B.make_options(path=path))
    torch.cuda.synchronize()
    return paged.y.cpu().numpy().view(np.uint16).copy()


def oracle_check(layer, y_bits, q):
    ref = orc.moe_forward_layer(layer, q=np.asarray(q, np.uint8).reshape(-1, 2))
    got = y_bits.view(np.float16).astype(np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mx = float(np.max(np.abs(got - ref)))
    say(f"  oracle: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS, (rel, mx)


def make_paged(layer, arena_bytes):
    from any_precision_bitplane_amd.device import PagedLayer
    return PagedLayer(layer, arena_bytes)


def plane_bytes(layer):
    """Bytes of one plane of each block, in page-table order (2e + m)."""
    wl = layer.wl
    return [(2 * wl.I * wl.H if b % 2 == 0 else wl.H * wl.I) // 8 for b in range(2 * wl.E)]


def full_arena(layer):
    return sum(rnd(8 * p) for p in plane_bytes(layer))


def test_commit_takes_effect_at_the_boundary(torch, tiny, static):
    say("pager: tiny layer, initial load, then a mixed plan (some blocks up, some down)")
    # room for every block at 8 planes twice over, so no plan runs out of space
    paged = make_paged(tiny, 2 * full_arena(tiny))
    copy = torch.cuda.Stream()
    q0 = tiny.q.copy()
    rng = np.random.default_rng(7)
    q1 = q0.copy()
    while np.array_equal(q1, q0) or not (q1 > q0).any() or not (q1 < q0).any():
        q1 = rng.integers(3, 9, q0.shape).astype(np.uint8)
    for b in range(paged.nblocks):
        info = paged.info(b)
        assert info.state == B.PW_PAGE_CPU and info.committed == 0 and info.resident == 0

    paged.request(q0)
    paged.execute(copy)
    n = paged.commit(wait=True)
    assert n == paged.nblocks
    y0 = paged_y(torch, paged)
    assert np.array_equal(y0, static_y(torch, static, q0))
    assert np.array_equal(paged.committed(), q0)

    paged.request(q1)
    paged.execute(copy)
    # staged but not committed: forwards still see q0
    y_before = paged_y(torch, paged)
    assert np.array_equal(y_before, y0)
    for b in range(paged.nblocks):
        info = paged.info(b)
        assert info.committed == q0.reshape(-1)[b]
        assert info.pending == (q1.reshape(-1)[b] if q1.reshape(-1)[b] != q0.reshape(-1)[b] else 0)
    n = paged.commit(wait=True)
    assert n == int((q1 != q0).sum())
    y1 = paged_y(torch, paged)
    assert np.array_equal(y1, static_y(torch, static, q1))
    oracle_check(tiny, y1, q1)
    for b in range(paged.nblocks):
        info = paged.info(b)
        assert info.committed == q1.reshape(-1)[b] and info.resident == info.committed
        assert info.state == B.PW_PAGE_GPU and info.pending == 0
    # once the stream has passed the commit, the lowered blocks' suffixes are free again
    torch.cuda.synchronize()
    paged.execute(copy)   # nothing staged: only reclaims
    want = sum(rnd(int(q1.reshape(-1)[b]) * paged.plane_bytes(b)) for b in range(paged.nblocks))
    assert B.pw_pager_arena_used(paged.pager) == want
    # the MFMA family reads the same page table
    assert np.array_equal(paged_y(torch, paged, B.PW_PATH_MFMA), static_y(torch, static, q1, B.PW_PATH_MFMA))
    paged.close()


def test_relocation_and_out_of_memory(torch, tiny, static):
    say("pager: tiny layer, tight arena: in-place growth impossible, block moves; then an over-full plan")
    pb = plane_bytes(tiny)
    q0 = np.full(tiny.q.shape, 4, np.uint8)
    spare = rnd(8 * max(pb))
    arena = sum(rnd(4 * p) for p in pb) + spare
    paged = make_paged(tiny, arena)
    copy = torch.cuda.Stream()
    paged.request(q0)
    paged.execute(copy)
    paged.commit(wait=True)
    off1 = paged.info(1).arena_offset
    assert paged.info(2).arena_offset == off1 + rnd(4 * pb[1])   # packed: block 2 right after block 1

    q1 = q0.copy()
    q1.reshape(-1)[1] = 8
    paged.request(q1)
    paged.execute(copy)
    paged.commit(wait=True)
    assert paged.info(1).arena_offset != off1          # moved
    assert np.array_equal(paged_y(torch, paged), static_y(torch, static, q1))

    # every block to 8 cannot fit: the call reports the shortage, what it staged
    # before that is committed, and the output follows the committed table
    torch.cuda.synchronize()
    paged.request(np.full(tiny.q.shape, 8, np.uint8))
    st = paged.execute(copy, check=False)
    assert st == B.PW_ERR_OUT_OF_MEMORY
    paged.commit(wait=True)
    qc = paged.committed()
    assert (qc == 8).any() and (qc < 8).any()
    assert np.array_equal(paged_y(torch, paged), static_y(torch, static, qc))

    # lower everything, then the freed planes let a later plan through
    torch.cuda.synchronize()
    paged.request(np.full(tiny.q.shape, 3, np.uint8))
    paged.execute(copy)
    paged.commit(wait=True)
    y3 = paged_y(torch, paged)
    assert np.array_equal(y3, static_y(torch, static, np.full(tiny.q.shape, 3, np.uint8)))
    oracle_check(tiny, y3, np.full(tiny.q.shape, 3, np.uint8))
    # raising to 4 fits in the suffix the lowering freed: every block grows in place
    torch.cuda.synchronize()
    offs = [paged.info(b).arena_offset for b in range(paged.nblocks)]
    q2 = np.random.default_rng(5).integers(3, 5, tiny.q.shape).astype(np.uint8)
    paged.request(q2)
    assert paged.execute(copy, check=False) == B.PW_OK
    paged.commit(wait=True)
    assert [paged.info(b).arena_offset for b in range(paged.nblocks)] == offs
    assert np.array_equal(paged_y(torch, paged), static_y(torch, static, q2))
    paged.close()


def test_unused_arena_is_never_read(torch, tiny, static):
    say("pager: tiny layer, every arena byte outside the committed prefixes overwritten with 0xFF")
    paged = make_paged(tiny, full_arena(tiny))
    copy = torch.cuda.Stream()
    paged.request(np.full(tiny.q.shape, 8, np.uint8))
    paged.execute(copy)
    paged.commit(wait=True)
    q1 = tiny.q.copy()
    paged.request(q1)
    paged.execute(copy)
    paged.commit(wait=True)
    torch.cuda.synchronize()
    keep = np.zeros(paged.arena_bytes, bool)
    for b in range(paged.nblocks):
        info = paged.info(b)
        keep[info.arena_offset: info.arena_offset + info.resident * paged.plane_bytes(b)] = True
    mask = torch.from_numpy(~keep).to(paged.arena.device)
    paged.arena.masked_fill_(mask, 0xFF)
    torch.cuda.synchronize()
    y = paged_y(torch, paged)
    assert np.array_equal(y, static_y(torch, static, q1))
    for path in (B.PW_PATH_GEMV, B.PW_PATH_MGEMV, B.PW_PATH_MFMA):
        assert np.array_equal(paged_y(torch, paged, path), static_y(torch, static, q1, path)), path
    assert paged.status() == 0
    paged.close()


def test_captured_graph_follows_commits(torch, tiny, static):
    say("pager: tiny layer forward captured in a HIP graph, replayed across three commits")
    paged = make_paged(tiny, 2 * full_arena(tiny))
    copy = torch.cuda.Stream()
    q0 = tiny.q.copy()
    paged.request(q0)
    paged.execute(copy)
    paged.commit(wait=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        paged.forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        paged.forward()
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    plans = [q0, rng.integers(3, 9, q0.shape).astype(np.uint8), np.full(q0.shape, 3, np.uint8)]
    for i, q in enumerate(plans):
        paged.request(q)
        paged.execute(copy)
        paged.commit(wait=True)      # on the current stream, where replays run
        want = static_y(torch, static, q)
        for rep in range(3):
            g.replay()
            torch.cuda.synchronize()
            got = paged.y.cpu().numpy().view(np.uint16).copy()
            assert np.array_equal(got, want), (i, rep)
            # eager work between replays
            paged.forward(y=torch.empty_like(paged.y))
            torch.cuda.synchronize()
    assert paged.status() == 0
    paged.close()


def test_routing_statistics_plan_and_commit(torch, tiny, static):
    say("pager: tiny layer, router statistics -> planner at 55% of the 8-bit plane bytes -> pager -> forward")
    import oracle.routing_oracle as ro
    wl = tiny.wl
    paged = make_paged(tiny, 2 * full_arena(tiny))
    copy = torch.cuda.Stream()
    paged.request(np.full(tiny.q.shape, 8, np.uint8))
    paged.execute(copy)
    paged.commit(wait=True)
    # route the tokens on the GPU, collecting the routing statistics
    wr = synth.draw_router_weights(wl.seed, wl.E, wl.H)
    wrd = torch.from_numpy(wr).to(paged.device)
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=paged.device)
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=paged.device)
    cnt = torch.zeros(wl.E, dtype=torch.int32, device=paged.device)
    mass = torch.zeros(wl.E, dtype=torch.float32, device=paged.device)
    B.pw_router_topk(paged.shape, wl.T, paged.x, wrd, ids, w, cnt, mass, paged.ws)
    torch.cuda.synchronize()
    pb = np.array(plane_bytes(tiny), np.int64)
    budget = int(0.55 * (8 * pb).sum())
    sens = synth.draw_sensitivity(wl.seed, 2 * wl.E)
    st, plan, used, fits = B.pw_plan_bitwidths(np.full(2 * wl.E, 8), pb, np.arange(2 * wl.E) // 2, sens,
                                               routing_mass=mass.cpu().numpy(), hot_fraction=0.25, floor_cold=3,
                                               floor_hot=6, hot_multiplier=2.0, budget_bytes=budget)
    assert fits and used <= budget
    hot = np.argsort(-mass.cpu().numpy(), kind="stable")[:2]
    assert all(plan[2 * e + m] >= 6 for e in hot for m in (0, 1))
    paged.request(plan.reshape(-1, 2))
    paged.execute(copy)
    paged.commit(wait=True)
    paged.ids, paged.w = ids, w
    y = paged_y(torch, paged)
    oids, ow, _ = ro.route(tiny.x, wr, wl.k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    ref = orc.moe_forward_layer(tiny, q=plan.reshape(-1, 2).astype(np.uint8), ids=oids, w=ow.astype(np.float32))
    got = y.view(np.float16).astype(np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mx = float(np.max(np.abs(got - ref)))
    say(f"  plan {plan.tolist()} ({used} of {int((8 * pb).sum())} plane bytes): rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= REL_L2 and mx <= MAX_ABS
    torch.cuda.synchronize()
    paged.execute(copy)
    assert B.pw_pager_arena_used(paged.pager) == sum(rnd(int(plan[b]) * int(pb[b])) for b in range(len(pb)))
    paged.close()


def test_forwards_during_a_full_size_reload_use_the_old_bitwidths(torch):
    say("pager: Qwen-shaped decode layer, every block at 3 bits, layer bitwidths reloaded (about 150 MB of planes) "
        "on a copy stream while 40 forwards run")
    from any_precision_bitplane_amd.device import DeviceLayer
    wl = synth.WORKLOADS["qwen_decode"]
    layer = synth.make_routed_layer(wl)
    static = DeviceLayer(layer)
    q3 = np.full(layer.q.shape, 3, np.uint8)
    want3 = static_y(torch, static, q3)
    want = static_y(torch, static, layer.q)
    paged = make_paged(layer, 2 * full_arena(layer))
    copy = torch.cuda.Stream()
    paged.request(q3)
    paged.execute(copy)
    paged.commit(wait=True)
    torch.cuda.synchronize()
    assert np.array_equal(paged_y(torch, paged), want3)
    paged.request(layer.q)
    paged.execute(copy)                  # host-to-device copies of planes 3..q-1 in flight
    seen_in_transfer = any(paged.info(b).state == B.PW_PAGE_IN_TRANSFER for b in range(paged.nblocks))
    ys = [torch.empty_like(paged.y) for _ in range(40)]
    for y in ys:
        paged.forward(y=y)
    torch.cuda.synchronize()
    for i, y in enumerate(ys):
        assert np.array_equal(y.cpu().numpy().view(np.uint16), want3), i
    assert seen_in_transfer
    paged.commit(wait=True)
    y = paged_y(torch, paged)
    assert np.array_equal(y, want)
    oracle_check(layer, y, layer.q)
    assert paged.status() == 0
    paged.close()
