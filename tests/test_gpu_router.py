"""GPU parity of the router, the routing statistics and the routed layer call
against the CPU oracle ("Technical summary: PagedWeight", Core components 2,
online routing statistics).

The GPU sums logits in fp32 and the oracle in fp64, so the top-k decision can
differ only between logits closer than the fp32 sums' error; where the two
lists differ, the test checks that the GPU's choice is such a near tie (several
results are correct) and compares the rest exactly.  Weights: max abs error
2e-6.  Statistics: counts exact against the GPU's own ids, mass within 1e-5
relative (fp32 atomic sums).  Every case prints what it runs first.
"""
import sys

import numpy as np
import pytest

import oracle.pagedweight_oracle as orc
import oracle.routing_oracle as ro
from any_precision_bitplane_amd import binding as B
from any_precision_bitplane_amd import synth

pytestmark = pytest.mark.gpu

W_ABS = 2e-6
TIE = 1e-4        # logits closer than this may legitimately order either way in fp32


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


def run_router(torch, x, wr, E, k, stats=None, repeat=1):
    T, H = x.shape
    shp = B.shape(H, 32, E, k)
    dev = "cuda:0"
    xd = torch.from_numpy(x).to(dev)
    wd = torch.from_numpy(wr).to(dev)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    w = torch.full((T, k), -1.0, dtype=torch.float32, device=dev)
    cnt = torch.zeros(E, dtype=torch.int32, device=dev) if stats else None
    mass = torch.zeros(E, dtype=torch.float32, device=dev) if stats else None
    ws = torch.empty(max(B.pw_workspace_bytes(shp, T), 256), dtype=torch.uint8, device=dev)
    B.pw_workspace_init(ws)
    for _ in range(repeat):
        B.pw_router_topk(shp, T, xd, wd, ids, w, cnt, mass, ws)
    torch.cuda.synchronize()
    out = (ids.cpu().numpy(), w.cpu().numpy())
    if stats:
        out += (cnt.cpu().numpy().astype(np.int64), mass.cpu().numpy().astype(np.float64))
    return out


def check_route(gids, gw, x, wr, k):
    oids, ow, logits = ro.route(x, wr, k)
    assert gids.shape == oids.shape and gw.shape == ow.shape
    T = x.shape[0]
    ties = 0
    for t in range(T):
        if np.array_equal(gids[t], oids[t]):
            continue
        ties += 1
        # a valid top-k: distinct ids whose oracle logits match the oracle's list up to near ties
        assert len(set(gids[t].tolist())) == k
        np.testing.assert_allclose(np.sort(logits[t, gids[t]]), np.sort(logits[t, oids[t]]), atol=TIE)
        assert np.all(np.diff(logits[t, gids[t]]) <= TIE)
    same = np.all(gids == oids, axis=1)
    err = np.abs(gw[same] - ow[same]).max() if same.any() else 0.0
    say(f"  ids equal on {same.sum()}/{T} tokens (near ties elsewhere: {ties}); weights max abs err {err:.2e}")
    assert err <= W_ABS
    assert ties <= max(1, T // 50)
    np.testing.assert_allclose(gw.sum(axis=1), 1.0, atol=1e-5)
    return oids, ow


CASES = [
    # (name, T, H, E, k, seed)
    ("tiny", 16, 256, 8, 2, 1000),
    ("qwen_decode", 4, 2048, 60, 4, 1001),
    ("qwen_batched", 256, 2048, 60, 4, 1002),
    ("mixtral_decode_T8", 8, 4096, 8, 2, 1003),
    ("mixtral_prefill", 4096, 4096, 8, 2, 1004),
    ("ragged_T7_k1", 7, 96, 5, 1, 7),
    ("k_equals_E", 9, 64, 8, 8, 8),
    ("E256_k64", 5, 128, 256, 64, 9),
]


@pytest.mark.parametrize("name,T,H,E,k,seed", CASES, ids=[c[0] for c in CASES])
def test_router_matches_oracle(torch, name, T, H, E, k, seed):
    say(f"router: {name} T={T} H={H} E={E} k={k}")
    x = synth.draw_x(seed, T, H)
    wr = synth.draw_router_weights(seed, E, H)
    gids, gw = run_router(torch, x, wr, E, k)
    check_route(gids, gw, x, wr, k)


def test_router_forms_agree_bit_for_bit(torch):
    """Batches of up to 256 tokens take one workgroup per token, larger ones
    four tokens per workgroup; both sum every logit in the same order, so 256
    tokens routed alone and as the first rows of a 257-token batch get the
    same ids and the same weight bits."""
    for (H, E, k, seed) in [(2048, 60, 4, 21), (96, 5, 1, 23), (128, 256, 64, 24)]:
        say(f"router forms: H={H} E={E} k={k}, T=256 alone and inside T=257")
        x = synth.draw_x(seed, 257, H)
        wr = synth.draw_router_weights(seed, E, H)
        ids256, w256 = run_router(torch, x[:256], wr, E, k)
        ids257, w257 = run_router(torch, x, wr, E, k)
        assert np.array_equal(ids256, ids257[:256])
        assert np.array_equal(w256.view(np.uint32), w257[:256].view(np.uint32))
        check_route(ids256, w256, x[:256], wr, k)


def test_router_ties_pick_lower_ids(torch):
    say("router: all logits equal (x = 0) -> ids 0..k-1, uniform weights")
    x = np.zeros((6, 64), np.float16)
    wr = synth.draw_router_weights(3, 10, 64)
    gids, gw = run_router(torch, x, wr, 10, 3)
    assert gids.tolist() == [[0, 1, 2]] * 6
    np.testing.assert_allclose(gw, 1 / 3, atol=1e-7)


def test_routing_statistics_accumulate(torch):
    say("router statistics: qwen_batched shapes, two calls accumulate")
    T, H, E, k = 256, 2048, 60, 4
    x = synth.draw_x(1002, T, H)
    wr = synth.draw_router_weights(1002, E, H)
    gids, gw, cnt, mass = run_router(torch, x, wr, E, k, stats=True, repeat=2)
    assert np.array_equal(cnt, 2 * np.bincount(gids.reshape(-1), minlength=E))
    want = 2 * np.bincount(gids.reshape(-1), weights=gw.reshape(-1).astype(np.float64), minlength=E)
    np.testing.assert_allclose(mass, want, rtol=1e-5, atol=1e-6)
    oids, ow = check_route(gids, gw, x, wr, k)
    ocnt, omass = ro.routing_stats(oids, ow, E)
    if np.array_equal(gids, oids):
        assert np.array_equal(cnt, 2 * ocnt)
        np.testing.assert_allclose(mass, 2 * omass, rtol=1e-5, atol=1e-6)
    assert abs(mass.sum() - 2 * T) < 1e-2


@pytest.mark.parametrize("path", [B.PW_PATH_AUTO, B.PW_PATH_MFMA], ids=["auto", "mfma"])
def test_routed_forward(torch, path):
    say(f"routed forward: tiny layer, router in front of the fused layer, path={path}")
    from any_precision_bitplane_amd.device import DeviceLayer
    wl = synth.WORKLOADS["tiny"]
    L = synth.make_layer(wl)
    wr = synth.draw_router_weights(wl.seed, wl.E, wl.H)
    dev = DeviceLayer(L)
    wrd = torch.from_numpy(wr).to(dev.device)
    cnt = torch.zeros(wl.E, dtype=torch.int32, device=dev.device)
    mass = torch.zeros(wl.E, dtype=torch.float32, device=dev.device)
    y_routed = torch.empty_like(dev.y)
    opts = B.make_options(path=path)
    B.pw_moe_forward_routed(dev.shape, wl.T, dev.x, wrd, dev.blocks[0], dev.q, y_routed, cnt, mass, dev.ws,
                            opts=opts)
    # the same layer fed the router's ids and weights through the two-call route
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev.device)
    w = torch.empty((wl.T, wl.k), dtype=torch.float32, device=dev.device)
    B.pw_router_topk(dev.shape, wl.T, dev.x, wrd, ids, w, None, None, dev.ws)
    B.pw_moe_forward(dev.shape, wl.T, dev.x, ids, w, dev.blocks[0], dev.q, dev.y, dev.ws, opts=opts)
    torch.cuda.synchronize()
    assert np.array_equal(y_routed.cpu().numpy().view(np.uint16), dev.y.cpu().numpy().view(np.uint16))
    assert dev.status() == 0
    gids = ids.cpu().numpy()
    oids, ow = check_route(gids, w.cpu().numpy(), L.x, wr, wl.k)
    assert np.array_equal(cnt.cpu().numpy(), np.bincount(gids.reshape(-1), minlength=wl.E))
    ref = orc.moe_forward_layer(L, ids=oids, w=ow.astype(np.float32))
    got = y_routed.float().cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mx = float(np.max(np.abs(got - ref)))
    say(f"  layer vs oracle: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel <= 1e-3 and mx <= 2e-2
