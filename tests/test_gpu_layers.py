"""Multi-layer decode (pw_moe_forward_layers): eight Qwen-shaped layers with
their own storage, page tables and routers, chained in one call.

* bit-identical to eight chained pw_moe_forward_routed calls (the combine of
  layer l is computed inside layer l + 1's router with the combine kernel's
  arithmetic), routing counts identical per layer;
* layer 0 and the last layer within the oracle's tolerance, each on its own
  input and the GPU router's ids and weights;
* one captured HIP graph of the call, replayed across a pager commit of the
  last layer: before the commit it reproduces the eager call, after it the
  eager call at the new bitwidths ("Technical summary: PagedWeight", Core
  components 3: commits at safe boundaries, q read on the device).
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
NLAYERS = 8


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


def compare(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    err = got - ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
    mx = float(np.max(np.abs(err)))
    say(f"  {what}: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert np.all(np.isfinite(got)) and rel <= REL_L2 and mx <= MAX_ABS, (what, rel, mx)


def _scale_down_tables(torch, L, dev, factor, paged):
    """Multiply every down table of layer L by `factor` (fp16, rounded on the
    host) and write the new tables to the device copies in place."""
    for e in range(L.wl.E):
        t = (L.luts[e][1].view(np.float16).astype(np.float32) * np.float32(factor)).astype(np.float16)
        L.luts[e][1] = t.view(np.uint16)
        dst = dev.luts[2 * e + 1] if paged else dev.luts[0][e][1]
        dst.copy_(torch.from_numpy(L.luts[e][1].view(np.int16)))


@pytest.fixture(scope="module")
def stack(torch):
    """Eight layers: 0..6 static device storage, 7 through the weight pager.

    A chain of SwiGLU layers without a residual path is quadratic in the
    activation scale, so the synthetic layers are normalized: after layer l is
    built, its down tables are scaled so that its output on its actual input
    has unit RMS, which keeps every layer's input O(1) (otherwise the values
    vanish after a few layers and the later layers' outputs no longer depend
    on their weights)."""
    from any_precision_bitplane_amd.device import DeviceLayer, PagedLayer
    base = synth.WORKLOADS["qwen_decode"]
    shp = B.shape(base.H, base.I, base.E, base.k)
    ws = torch.empty(B.pw_workspace_bytes(shp, base.T), dtype=torch.uint8, device="cuda")
    B.pw_workspace_init(ws)
    layers, devs, wrs = [], [], []
    x = None
    for l in range(NLAYERS):
        wl = synth.Workload(f"qwen_layer{l}", H=base.H, I=base.I, E=base.E, k=base.k, T=base.T, seed=3000 + l)
        say(f"drawing layer {l}")
        L = synth.make_layer(wl)
        layers.append(L)
        wrs.append(torch.from_numpy(synth.draw_router_weights(wl.seed, wl.E, wl.H)).cuda())
        paged = l == NLAYERS - 1
        if not paged:
            dev = DeviceLayer(L)
        else:
            full = sum(8 * (2 * wl.I * wl.H if b % 2 == 0 else wl.H * wl.I) // 8 for b in range(2 * wl.E))
            dev = PagedLayer(L, full + (1 << 20))
            dev.request(L.q)
            dev.execute()
            dev.commit()
        devs.append(dev)
        if x is None:
            x = torch.from_numpy(L.x).cuda()
        y = torch.empty((wl.T, wl.H), dtype=torch.float16, device="cuda")
        B.pw_moe_forward_routed(shp, wl.T, x, wrs[l], dev.blocks if paged else dev.blocks[0], dev.q, y, None, None, ws)
        torch.cuda.synchronize()
        rms = float(y.float().pow(2).mean().sqrt())
        assert rms > 0
        _scale_down_tables(torch, L, dev, 1.0 / rms, paged)
        B.pw_moe_forward_routed(shp, wl.T, x, wrs[l], dev.blocks if paged else dev.blocks[0], dev.q, y, None, None, ws)
        torch.cuda.synchronize()
        x = y
    yield layers, devs, wrs
    devs[-1].close()


def test_layers_equal_chained_routed_calls_and_the_oracle(torch, stack):
    layers, devs, wrs = stack
    wl = layers[0].wl
    shp = B.shape(wl.H, wl.I, wl.E, wl.k)
    T = wl.T
    ws = torch.empty(B.pw_workspace_bytes(shp, T), dtype=torch.uint8, device="cuda")
    B.pw_workspace_init(ws)
    x0 = torch.from_numpy(layers[0].x).cuda()

    say("eight chained routed layer calls")
    xs = [x0]
    cnt_chain = torch.zeros((NLAYERS, wl.E), dtype=torch.int32, device="cuda")
    mass_chain = torch.zeros((NLAYERS, wl.E), dtype=torch.float32, device="cuda")
    for l in range(NLAYERS):
        y = torch.empty((T, wl.H), dtype=torch.float16, device="cuda")
        B.pw_moe_forward_routed(shp, T, xs[-1], wrs[l], devs[l].blocks if l == NLAYERS - 1 else devs[l].blocks[0],
                                devs[l].q, y, cnt_chain[l], mass_chain[l], ws)
        xs.append(y)
    say("one multi-layer call")
    y_ml = torch.empty((T, wl.H), dtype=torch.float16, device="cuda")
    cnt_ml = torch.zeros_like(cnt_chain)
    mass_ml = torch.zeros_like(mass_chain)
    blocks = [d.blocks if i == NLAYERS - 1 else d.blocks[0] for i, d in enumerate(devs)]
    B.pw_moe_forward_layers(shp, T, x0, wrs, blocks, [d.q for d in devs], y_ml, cnt_ml, mass_ml, ws)
    torch.cuda.synchronize()
    assert torch.equal(y_ml, xs[-1]), "multi-layer call differs from the chained calls"
    assert torch.equal(cnt_ml, cnt_chain)
    assert torch.allclose(mass_ml, mass_chain, rtol=1e-5, atol=1e-6)
    assert int(cnt_ml.sum()) == NLAYERS * T * wl.k
    assert B.pw_get_device_status(ws) == 0

    for l in (0, NLAYERS - 1):
        ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
        B.pw_router_topk(shp, T, xs[l], wrs[l], ids, w, None, None, ws)
        torch.cuda.synchronize()
        x_np = xs[l].cpu().numpy()
        L = layers[l]
        ref = orc.moe_forward(x_np, ids.cpu().numpy(), w.cpu().numpy(), L.planes, L.luts, L.q, wl.H, wl.I, wl.E)
        assert np.sqrt(np.mean(ref ** 2)) > 0.3, "the layer's output should be O(1)"
        compare(xs[l + 1].float().cpu().numpy(), ref, f"layer {l} vs oracle")


def test_layers_graph_replays_follow_a_pager_commit(torch, stack):
    layers, devs, wrs = stack
    wl = layers[0].wl
    shp = B.shape(wl.H, wl.I, wl.E, wl.k)
    T = wl.T
    ws = torch.empty(B.pw_workspace_bytes(shp, T), dtype=torch.uint8, device="cuda")
    B.pw_workspace_init(ws)
    x0 = torch.from_numpy(layers[0].x).cuda()
    blocks = [d.blocks if i == NLAYERS - 1 else d.blocks[0] for i, d in enumerate(devs)]
    qs = [d.q for d in devs]
    y_graph = torch.empty((T, wl.H), dtype=torch.float16, device="cuda")

    def eager():
        y = torch.empty_like(y_graph)
        B.pw_moe_forward_layers(shp, T, x0, wrs, blocks, qs, y, None, None, ws)
        torch.cuda.synchronize()
        return y

    say("capture one multi-layer call in a HIP graph")
    before = eager()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.pw_moe_forward_layers(shp, T, x0, wrs, blocks, qs, y_graph, None, None, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        B.pw_moe_forward_layers(shp, T, x0, wrs, blocks, qs, y_graph, None, None, ws)
    for rep in range(3):
        y_graph.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph, before), f"replay {rep} before the commit"
        assert torch.equal(eager(), before)

    say("pager: last layer's blocks lowered to 3 bits, committed between replays")
    P = devs[-1]
    P.request(np.full(layers[-1].q.shape, 3, np.uint8))
    P.execute()
    assert P.commit() > 0
    torch.cuda.synchronize()
    after = eager()
    assert not torch.equal(after, before)
    for rep in range(3):
        y_graph.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph, after), f"replay {rep} after the commit"
    del g
    P.request(layers[-1].q)
    P.execute()
    P.commit()
    torch.cuda.synchronize()
    assert torch.equal(eager(), before)
