"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Bars: dequantized weights bit-exact; layer output within relative L2 error
1e-3 and max abs error 2e-2 of the oracle (fp32 accumulation, fp16 h and y).
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

_ORACLE_CACHE = {}
_LAYERS = {}


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


def layer_for(name, T=None, routed_only=True):
    wl = synth.WORKLOADS[name] if T is None else synth.WORKLOADS[name].with_T(T)
    key = (wl.name, routed_only)
    if key not in _LAYERS:
        _LAYERS[key] = synth.make_routed_layer(wl) if routed_only else synth.make_layer(wl)
    return _LAYERS[key]


def custom_layer(H, I, E, k, T, seed, qvals=None):
    wl = synth.Workload(f"custom{H}x{I}x{E}x{k}x{T}", H=H, I=I, E=E, k=k, T=T, seed=seed)
    L = synth.make_layer(wl)
    if qvals is not None:
        L.q[:] = np.asarray(qvals, np.uint8)
    return L


def oracle_y(L, tokens=None, q=None, ids=None, w=None):
    return orc.moe_forward_layer(L, tokens=tokens, cache=_ORACLE_CACHE, q=q, ids=ids, w=w)


def compare(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    err = got - ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
    mx = float(np.max(np.abs(err))) if err.size else 0.0
    say(f"  {what}: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert np.all(np.isfinite(got)), what
    assert rel <= REL_L2, (what, rel)
    assert mx <= MAX_ABS, (what, mx)


def run_forward(torch, L, path=B.PW_PATH_AUTO, mfma_min_tokens=0, dev=None):
    from any_precision_bitplane_amd.device import DeviceLayer
    dev = dev or DeviceLayer(L)
    dev.forward(B.make_options(path=path, mfma_min_tokens=mfma_min_tokens))
    torch.cuda.synchronize()
    return dev, dev.y.float().cpu().numpy()


# ---------------------------------------------------------------------------
# dequantization: bit-exact
# ---------------------------------------------------------------------------
def _pack(torch, planes, module, nplanes=8):
    """Canonical planes -> device layout on the GPU (pw_pack_planes)."""
    N, W = planes.shape[1], planes.shape[2]
    src = torch.from_numpy(np.ascontiguousarray(planes[:nplanes]).view(np.int32)).cuda()
    out = torch.empty(B.pw_planes_bytes(N, 32 * W, nplanes) // 4, dtype=torch.int32, device="cuda")
    B.pw_pack_planes(src, N, 32 * W, nplanes, module, out)
    return out


def _dequant_checks(torch, planes, lut, module, what, qs=range(3, 9)):
    """Pack the canonical planes, dequantize on the GPU at each q, compare bit
    for bit with the oracle's dequantization of the canonical planes."""
    N, K = planes.shape[1], planes.shape[2] * 32
    p = _pack(torch, planes, module)
    l = torch.from_numpy(lut.view(np.int16)).cuda()
    out = torch.empty((N, K), dtype=torch.int16, device="cuda")
    for q in qs:
        say(f"dequant {what} N={N} K={K} module={module} q={q}")
        B.pw_dequant_block(p, l, N, K, q, out, module=module)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint16)
        ref = orc.dequant_block(planes, lut, q)
        assert np.array_equal(got, ref), f"{what} q={q}: {np.count_nonzero(got != ref)} mismatches"


def test_dequant_bit_exact_tiny_all_blocks(torch):
    L = layer_for("tiny", routed_only=False)
    for e in range(L.wl.E):
        for m in (0, 1):
            _dequant_checks(torch, L.planes[e][m], L.luts[e][m], m, f"tiny e{e} m{m}")


@pytest.mark.parametrize("group", range(6))
def test_dequant_bit_exact_qwen_every_block(torch, group):
    """Every block of the Qwen-shaped layer (60 experts x 2 modules, ten experts
    per group) at every bitwidth 3..8."""
    wl = synth.WORKLOADS["qwen_decode"]
    for e in range(10 * group, 10 * group + 10):
        for m in (0, 1):
            N, K = wl.block_shape(m)
            planes = synth.draw_planes(wl.seed, e, m, N, K)
            lut = synth.draw_lut(wl.seed, e, m, N)
            _dequant_checks(torch, planes, lut, m, f"qwen e{e} m{m}")


@pytest.mark.parametrize("m", [0, 1])
def test_dequant_bit_exact_mixtral_full_block(torch, m):
    """One full-size Mixtral-shaped block per module (gate_up 28672 x 4096,
    down 4096 x 14336) at every bitwidth 3..8."""
    wl = synth.WORKLOADS["mixtral_prefill"]
    N, K = wl.block_shape(m)
    planes = synth.draw_planes(wl.seed, 5, m, N, K)
    lut = synth.draw_lut(wl.seed, 5, m, N)
    _dequant_checks(torch, planes, lut, m, f"mixtral e5 m{m}")


def test_dequant_ragged_shapes(torch):
    # K/32 below one 16-word tile, not a multiple of 16 (a narrower last column
    # tile: 44 and 65 words), not a multiple of 4; both row orders
    rng = np.random.default_rng(11)
    for N, K in [(16, 32), (32, 96), (48, 2080), (32, 4128), (64, 1408), (16, 544)]:
        planes = rng.integers(0, 2 ** 32, (8, N, K // 32), dtype=np.uint32)
        lut = synth.draw_lut(5, 0, 0, N)
        for m in (0, 1):
            _dequant_checks(torch, planes, lut, m, "ragged", qs=(3, 5, 8))


def _layout_ref(canon, module):
    """The device layout written out element by element from its definition
    (16-row x 16-word tiles, tile-row-major, rows inside a tile, the last
    column tile W mod 16 wide; gate_up rows interleaved 8 gate / 8 up)."""
    P, N, W = canon.shape
    I = N // 2
    d = np.arange(N)[:, None]
    c = np.arange(W)[None, :]
    n_of_d = np.where((d & 15) < 8, 8 * (d >> 4) + (d & 15), I + 8 * (d >> 4) + (d & 15) - 8) if module == 0 else d
    width = np.minimum(16, W - (c & ~15))
    off = (d >> 4) * 16 * W + (c >> 4) * 256 + (d & 15) * width + (c & 15)
    out = np.zeros(P * N * W, dtype=np.uint32)
    for p in range(P):
        out[p * N * W + off] = canon[p][np.broadcast_to(n_of_d, off.shape), np.broadcast_to(c, off.shape)]
    return out


@pytest.mark.parametrize("module", [0, 1])
def test_pack_planes_layout(torch, module):
    """pw_pack_planes writes every word where the layout puts it (bit-exact),
    for full and partial column tiles and plane counts below 8; the result is
    a permutation of the input words."""
    rng = np.random.default_rng(12 + module)
    for N, K, nplanes in [(16, 32, 8), (32, 96, 3), (48, 1408, 8), (64, 2080, 5), (2816, 2048, 8), (256, 512, 6)]:
        say(f"pack N={N} K={K} nplanes={nplanes} module={module}")
        canon = rng.integers(0, 2 ** 32, (8, N, K // 32), dtype=np.uint32)
        assert B.pw_planes_bytes(N, K, nplanes) == nplanes * N * K // 8
        got = _pack(torch, canon, module, nplanes)
        torch.cuda.synchronize()
        got = got.cpu().numpy().view(np.uint32)
        ref = _layout_ref(canon[:nplanes], module)
        assert np.array_equal(got, ref)
        assert np.array_equal(np.sort(got), np.sort(canon[:nplanes].reshape(-1)))


# ---------------------------------------------------------------------------
# layer forward vs oracle
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("path", [B.PW_PATH_GEMV, B.PW_PATH_AUTO])
def test_forward_tiny(torch, path):
    L = layer_for("tiny")
    say(f"forward tiny path={path}")
    _, y = run_forward(torch, L, path)
    compare(y, oracle_y(L), f"tiny path={path}")


def test_forward_qwen_decode(torch):
    L = layer_for("qwen_decode")
    say("forward qwen_decode T=4")
    _, y = run_forward(torch, L)
    compare(y, oracle_y(L), "qwen_decode")


@pytest.mark.parametrize("T", [1, 8])
def test_forward_mixtral_decode(torch, T):
    L = layer_for("mixtral_decode", T=T)
    say(f"forward mixtral_decode T={T}")
    _, y = run_forward(torch, L, B.PW_PATH_GEMV)
    compare(y, oracle_y(L), f"mixtral_decode T={T}")


def test_forward_ragged_shapes(torch):
    # gate_up K = 2080 (65 plane words: two slices, one-word tail); down K = 96
    for (H, I, E, k, T, seed) in [(2080, 96, 5, 3, 7, 31), (32, 32, 3, 2, 5, 32), (96, 1056, 4, 4, 3, 33)]:
        L = custom_layer(H, I, E, k, T, seed)
        say(f"forward ragged H={H} I={I} E={E} k={k} T={T}")
        _, y = run_forward(torch, L, B.PW_PATH_GEMV)
        compare(y, oracle_y(L), f"ragged H={H} I={I}")


@pytest.mark.parametrize("H,I,E,k,T,seed", [(2048, 704, 36, 6, 6, 35), (512, 256, 96, 8, 12, 36)])
def test_forward_one_token_per_expert_every_bitwidth_pair(torch, H, I, E, k, T, seed):
    # Every expert takes exactly one token, and the experts' (gate_up, down)
    # bitwidths run over all 36 pairs of 3..8: the single-token decode at
    # every Q, in both products.  S = T*k = 36 routes inside the gate_up
    # kernel; S = 96 goes through the route kernel.
    qvals = [(3 + e % 6, 3 + (e // 6) % 6) for e in range(E)]
    L = custom_layer(H, I, E, k, T, seed, qvals=qvals)
    L.ids[:] = np.arange(T * k, dtype=np.int32).reshape(T, k) % E
    say(f"forward one token per expert H={H} I={I} E={E} k={k} T={T}")
    _, y = run_forward(torch, L, B.PW_PATH_GEMV)
    compare(y, oracle_y(L), f"one token per expert E={E}")


def test_forward_gemv_three_bit_pair_tables(torch):
    """3-bit blocks run on pair tables built in LDS: every block at q=3, K not
    a multiple of the 64-word slice (several slices), several tokens per
    expert (token pairs and a single token left over)."""
    L = custom_layer(2080, 1056, 4, 2, 6, 45, qvals=np.full((4, 2), 3))
    say("forward gemv q=3 H=2080 I=1056 E=4 k=2 T=6")
    _, y = run_forward(torch, L, B.PW_PATH_GEMV)
    compare(y, oracle_y(L), "gemv q=3 pair tables")


def test_forward_many_tokens_per_expert_gemv(torch):
    # experts with 3..40 tokens take several token groups on the GEMV path
    L = custom_layer(256, 512, 4, 2, 40, 34)
    say("forward gemv many tokens per expert")
    _, y = run_forward(torch, L, B.PW_PATH_GEMV)
    compare(y, oracle_y(L), "gemv many tokens")


@pytest.mark.parametrize("T,inline", [(16, 1), (17, 0)])
def test_forward_gemv_routing_edge(torch, T, inline):
    """The bit-plane GEMV's two routing forms at their edge: 16 tokens of the
    Qwen-shaped layer fill all 64 slots the gate_up kernel routes by itself
    (one slot per lane), 17 tokens (68 slots) take the route kernel."""
    L = layer_for("qwen_decode", T=T)
    wl = L.wl
    info = B.pw_moe_path_info(B.shape(wl.H, wl.I, wl.E, wl.k), T)
    assert info.gemv == 1 and info.mgemv == 0 and info.mfma == 0 and info.inline_route == inline
    say(f"forward qwen_decode T={T} AUTO (GEMV, inline routing {inline})")
    dev, y = run_forward(torch, L)
    assert dev.status() == 0
    compare(y, oracle_y(L), f"qwen gemv T={T}, inline routing {inline}")


@pytest.mark.parametrize("k", [1, 2])
@pytest.mark.parametrize("path", [B.PW_PATH_GEMV, B.PW_PATH_MGEMV, B.PW_PATH_MFMA, B.PW_PATH_AUTO])
def test_forward_single_token_every_family(torch, path, k):
    """One token (one or two routed slots) on every kernel family: one 32-token
    matrix-core GEMV tile or one 512-token MFMA tile holding a single token."""
    L = custom_layer(256, 512, 8, k, 1, seed=70 + k)
    say(f"forward single token k={k} path={path}")
    dev, y = run_forward(torch, L, path)
    assert dev.status() == 0
    compare(y, oracle_y(L), f"single token k={k} path={path}")


def test_forward_zero_tokens_is_noop(torch):
    from any_precision_bitplane_amd.device import DeviceLayer
    L = layer_for("tiny")
    dev = DeviceLayer(L)
    dev.y.fill_(7.0)
    say("forward T=0")
    st = B.pw_moe_forward(dev.shape, 0, dev.x, dev.ids, dev.w, dev.blocks[0], dev.q, dev.y, dev.ws)
    torch.cuda.synchronize()
    assert st == B.PW_OK
    assert bool((dev.y == 7.0).all())


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_deterministic_and_relocation_invariant(torch):
    """Same inputs give the same bits; moving the blocks to other addresses and
    rewriting the page table gives the same bits too."""
    from any_precision_bitplane_amd.device import DeviceLayer
    L = layer_for("qwen_decode")
    say("determinism + relocation qwen_decode")
    dev = DeviceLayer(L, copies=2, experts=[int(e) for e in L.active_experts()])
    dev.forward()
    y0 = dev.y.clone()
    dev.forward()
    y1 = dev.y.clone()
    dev.forward(copy=1)
    y2 = dev.y.clone()
    torch.cuda.synchronize()
    assert dev.planes[1][int(L.active_experts()[0])][0].data_ptr() != dev.planes[0][int(L.active_experts()[0])][0].data_ptr()
    assert torch.equal(y0, y1) and torch.equal(y0, y2)


def test_concurrent_calls_on_two_streams(torch):
    """Two layers, each with its own workspace, enqueued alternately on two
    streams with nothing ordering one stream against the other: every output
    equals the serial result bit for bit (calls share no state beyond their
    arguments).  One layer runs the GEMV family with inline routing, the other
    the matrix-core GEMV after the route kernel."""
    from any_precision_bitplane_amd.device import DeviceLayer
    da = DeviceLayer(layer_for("qwen_decode"))
    db = DeviceLayer(layer_for("mixtral_decode", T=64))
    da.forward()
    db.forward()
    torch.cuda.synchronize()
    ya, yb = da.y.clone(), db.y.clone()
    outs_a = [torch.empty_like(ya) for _ in range(8)]
    outs_b = [torch.empty_like(yb) for _ in range(8)]
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    say("8 + 8 forwards alternating on two streams")
    for i in range(8):
        da.forward(stream=sa, y=outs_a[i])
        db.forward(stream=sb, y=outs_b[i])
    torch.cuda.synchronize()
    assert da.status() == 0 and db.status() == 0
    for i in range(8):
        assert torch.equal(outs_a[i], ya), f"stream A call {i}"
        assert torch.equal(outs_b[i], yb), f"stream B call {i}"


def test_commit_is_ordered_on_the_stream(torch):
    """A q write enqueued after a forward does not affect it; the next forward
    sees it (the page table is read on the device)."""
    from any_precision_bitplane_amd.device import DeviceLayer
    L = layer_for("qwen_decode")
    say("stream-ordered commit qwen_decode")
    dev = DeviceLayer(L)
    q_new = L.q.copy()
    q_new[:, :] = 3
    out_a = torch.empty_like(dev.y)
    out_b = torch.empty_like(dev.y)
    dev.forward(y=out_a)
    dev.set_q(q_new)
    dev.forward(y=out_b)
    torch.cuda.synchronize()
    compare(out_a.float().cpu().numpy(), oracle_y(L), "before commit")
    compare(out_b.float().cpu().numpy(), oracle_y(L, q=q_new), "after commit")
    ref = DeviceLayer(L)
    ref.forward()
    torch.cuda.synchronize()
    assert torch.equal(out_a, ref.y)


def test_block_bitwidth_only_affects_its_tokens(torch):
    """Each block is computed at its own q: changing the q of experts a token
    does not route to leaves that token's output bit-identical."""
    from any_precision_bitplane_amd.device import DeviceLayer
    L = layer_for("qwen_decode")
    say("per-block bitwidth independence qwen_decode")
    dev = DeviceLayer(L)
    dev.forward()
    base = dev.y.clone()
    mine = set(int(e) for e in L.ids[0])
    q2 = L.q.copy()
    for e in range(L.wl.E):
        if e not in mine:
            q2[e] = 3 + (q2[e] - 3 + 2) % 6
    dev.set_q(q2)
    dev.forward()
    torch.cuda.synchronize()
    assert torch.equal(base[0], dev.y[0])


def test_invalid_ids_and_bitwidths_flagged_and_zero(torch):
    from any_precision_bitplane_amd.device import DeviceLayer
    L = layer_for("tiny")
    say("invalid ids / bitwidths")
    ids = L.ids.copy()
    ids[0, 1] = L.wl.E
    ids[3, 0] = -5
    dev = DeviceLayer(L)
    dev.ids.copy_(torch.from_numpy(ids))
    dev.forward()
    torch.cuda.synchronize()
    assert dev.status() & B.PW_DEV_BAD_EXPERT_ID
    assert dev.status() == 0            # reading clears it
    compare(dev.y.float().cpu().numpy(), oracle_y(L, ids=ids), "dropped slots")

    q = L.q.copy()
    bad_e = int(L.ids[5, 0])
    q[bad_e, 1] = 11
    dev2 = DeviceLayer(L)
    dev2.set_q(q)
    dev2.forward()
    torch.cuda.synchronize()
    assert dev2.status() & B.PW_DEV_BAD_BITWIDTH
    compare(dev2.y.float().cpu().numpy(), oracle_y(L, q=q), "invalid bitwidth block")


def test_gemv_small_call_invalid_down_bitwidth_and_dropped_slots(torch):
    """Small calls on the GEMV kernels route inside gate_up, and the down kernel
    takes each routed expert's bitwidth and storage from a work descriptor:
    an invalid down bitwidth there still reads as zero rows and is flagged,
    dropped slots add nothing, and the next call on the same workspace is exact."""
    from any_precision_bitplane_amd.device import DeviceLayer
    L = layer_for("tiny")
    opts = B.make_options(path=B.PW_PATH_GEMV)
    info = B.pw_moe_path_info(B.shape(L.wl.H, L.wl.I, L.wl.E, L.wl.k), L.wl.T, opts)
    assert info.gemv == 1 and info.inline_route == 1
    ids = L.ids.copy()
    ids[1, 0] = -3
    q = L.q.copy()
    q[int(L.ids[6, 1]), 1] = 2
    say("GEMV inline call: invalid down bitwidth and a dropped slot")
    dev = DeviceLayer(L)
    dev.ids.copy_(torch.from_numpy(ids))
    dev.set_q(q)
    dev.forward(opts)
    torch.cuda.synchronize()
    st = dev.status()
    assert st & B.PW_DEV_BAD_BITWIDTH and st & B.PW_DEV_BAD_EXPERT_ID
    compare(dev.y.float().cpu().numpy(), oracle_y(L, ids=ids, q=q), "gemv inline, bad down q + dropped slot")
    say("GEMV inline call: the valid layer on the same workspace")
    dev.ids.copy_(torch.from_numpy(L.ids))
    dev.set_q(L.q)
    dev.forward(opts)
    torch.cuda.synchronize()
    assert dev.status() == 0
    compare(dev.y.float().cpu().numpy(), oracle_y(L), "gemv inline, valid after invalid")


def test_duplicate_ids_are_summed(torch):
    from any_precision_bitplane_amd.device import DeviceLayer
    L = layer_for("tiny")
    ids = L.ids.copy()
    ids[:, 1] = ids[:, 0]
    say("duplicate ids")
    dev = DeviceLayer(L)
    dev.ids.copy_(torch.from_numpy(ids))
    dev.forward()
    torch.cuda.synchronize()
    compare(dev.y.float().cpu().numpy(), oracle_y(L, ids=ids), "duplicate ids")


# ---------------------------------------------------------------------------
# MFMA (dequant-to-LDS) path and the per-expert path choice
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,T", [("tiny", None), ("qwen_decode", None), ("mixtral_decode", 64)])
def test_forward_mfma_forced(torch, name, T):
    L = layer_for(name, T=T)
    say(f"forward {name} T={L.wl.T} path=MFMA")
    _, y = run_forward(torch, L, B.PW_PATH_MFMA)
    compare(y, oracle_y(L), f"{name} mfma")


def test_forward_mfma_ragged_shapes(torch):
    # (160, 96, .., 600) gives each expert one full 512-token tile and a partial
    # one, with both K ranges ending inside a quad of eight plane words; the
    # last case runs the down product in two K parts (33 quads: 17 + 16, the
    # last one partial)
    for (H, I, E, k, T, seed) in [(2080, 96, 5, 3, 70, 41), (96, 1056, 4, 4, 45, 42), (256, 512, 2, 1, 300, 43),
                                  (160, 96, 2, 2, 260, 44), (160, 96, 2, 2, 600, 46), (256, 8224, 2, 1, 300, 47)]:
        L = custom_layer(H, I, E, k, T, seed)
        info = B.pw_moe_path_info(B.shape(H, I, E, k), T, B.make_options(path=B.PW_PATH_MFMA))
        say(f"forward mfma ragged H={H} I={I} E={E} k={k} T={T} down K parts={info.down_kparts}")
        assert info.down_kparts == (2 if I == 8224 else 1)
        _, y = run_forward(torch, L, B.PW_PATH_MFMA)
        compare(y, oracle_y(L), f"mfma ragged H={H} I={I}")


def test_forward_qwen_batched_auto_mixes_paths(torch):
    """Zipf routing: hot experts (many tokens, 8 bits) on the MFMA kernels, the
    rest on the matrix-core GEMV, in one call; then every expert on the GEMV."""
    L = layer_for("qwen_batched")
    counts = np.bincount(L.ids.reshape(-1), minlength=L.wl.E)
    assert counts.max() >= 16 and counts[counts > 0].min() < 16
    say("forward qwen_batched T=256 AUTO")
    _, y = run_forward(torch, L, B.PW_PATH_AUTO, mfma_min_tokens=16)
    ref = oracle_y(L)
    compare(y, ref, "qwen_batched auto")
    say("forward qwen_batched T=256 GEMV")
    _, y2 = run_forward(torch, L, B.PW_PATH_GEMV)
    compare(y2, ref, "qwen_batched gemv")


# Full-size prefill (T = 4096, E = 8, top-2, skewed bitwidths).  Every expert
# gets about 1000 slots, i.e. two or three 512-slot MFMA tiles, the last one
# partial (some with fewer tokens than one wave's 128).  Each pair
# test drops every slot outside two experts (ids -> -1): those experts' slots,
# their order and hence their MFMA tiles stay exactly as in the full call, and
# every token routed to them is compared with the oracle over the same ids, so
# all 16 blocks are checked at full K on all of their tiles.  The oracle
# dequantizes two experts per test, which bounds its time and memory.  The full
# call is then checked on stratified tokens: for every expert, tokens of its
# first and of its last tile, against the sum of the four pairs' references.
_C4 = {}
_C4_PAIRS = [(0, 1), (2, 3), (4, 5), (6, 7)]


def _c4_layer():
    if "layer" not in _C4:
        _C4["layer"] = layer_for("mixtral_prefill", routed_only=False)
    return _C4["layer"]


def _c4_device(torch):
    if "dev" not in _C4:
        from any_precision_bitplane_amd.device import DeviceLayer
        _C4["dev"] = DeviceLayer(_c4_layer())
    return _C4["dev"]


def _c4_pair_ids(a, b):
    ids = _c4_layer().ids.copy()
    ids[(ids != a) & (ids != b)] = -1
    return ids


def _c4_pair_ref(a, b):
    """Oracle y for all tokens with only experts a and b routed."""
    key = ("ref", a, b)
    if key not in _C4:
        L = _c4_layer()
        _C4[key] = orc.moe_forward_layer(L, ids=_c4_pair_ids(a, b))
    return _C4[key]


@pytest.mark.parametrize("pair", _C4_PAIRS)
def test_forward_mixtral_prefill_expert_pairs_all_tokens(torch, pair):
    a, b = pair
    L = _c4_layer()
    dev = _c4_device(torch)
    ids = _c4_pair_ids(a, b)
    say(f"forward mixtral_prefill T=4096 AUTO, only experts {a},{b} routed "
        f"(q gate_up {L.q[a][0]},{L.q[b][0]}; q down {L.q[a][1]},{L.q[b][1]})")
    dev.ids.copy_(torch.from_numpy(ids))
    dev.forward(B.make_options(path=B.PW_PATH_AUTO))
    torch.cuda.synchronize()
    y = dev.y.float().cpu().numpy()
    dev.ids.copy_(torch.from_numpy(L.ids))
    assert dev.status() == B.PW_DEV_BAD_EXPERT_ID     # the dropped slots, nothing else
    rows = np.nonzero((ids >= 0).any(axis=1))[0]
    assert len(rows) > 1500
    assert not np.any(y[np.setdiff1d(np.arange(L.wl.T), rows)])
    ref = _c4_pair_ref(a, b)
    compare(y[rows], ref[rows], f"mixtral_prefill experts {a},{b}: all {len(rows)} tokens")


def _c4_strata():
    """For every expert: 4 tokens from its first 512-slot tile and 4 from its last."""
    L = _c4_layer()
    flat = L.ids.reshape(-1)
    toks = set()
    for e in range(L.wl.E):
        slots = np.nonzero(flat == e)[0]          # slot order = the expert's sorted order
        ntile = (len(slots) + 511) // 512
        first = slots[:512] // L.wl.k
        last = slots[512 * (ntile - 1):] // L.wl.k
        for part in (first, last):
            pick = np.unique(part)
            toks.update(int(t) for t in pick[np.linspace(0, len(pick) - 1, 4).astype(int)])
    return sorted(toks)


def test_forward_mixtral_prefill_full_call_stratified(torch):
    """The full-size call with every expert routed, compared on tokens drawn
    from the first and the last MFMA tile of every expert."""
    L = _c4_layer()
    dev = _c4_device(torch)
    say("forward mixtral_prefill T=4096 AUTO, all experts")
    dev.forward(B.make_options(path=B.PW_PATH_AUTO))
    torch.cuda.synchronize()
    assert dev.status() == 0
    y = dev.y.float().cpu().numpy()
    assert np.all(np.isfinite(y))
    toks = _c4_strata()
    per = {e: sum(1 for t in toks if e in set(int(v) for v in L.ids[t])) for e in range(L.wl.E)}
    assert min(per.values()) >= 8, per
    ref = sum(_c4_pair_ref(a, b)[toks] for a, b in _C4_PAIRS)
    compare(y[toks], ref, f"mixtral_prefill full call, {len(toks)} stratified tokens")
    _C4.clear()


def test_forward_qwen_largest_prefill_stratified(torch):
    """A Qwen-shaped prefill of 32768 tokens (131072 routed slots, about 2200
    per expert: four or five 512-slot MFMA tiles each, the remainders of at most
    96 on the matrix-core GEMV; a 1 GB o buffer), the largest call in the
    suite.  The oracle takes tokens from every expert's first and last tile."""
    T = 32768
    L = layer_for("qwen_decode", T=T)
    wl = L.wl
    info = B.pw_moe_path_info(B.shape(wl.H, wl.I, wl.E, wl.k), T)
    assert info.mfma == 1 and info.mfma_tail > 0
    say(f"forward qwen_decode T={T} AUTO (prefill form)")
    dev, y = run_forward(torch, L)
    assert dev.status() == 0
    assert np.all(np.isfinite(y))
    flat = L.ids.reshape(-1)
    toks = set()
    for e in range(wl.E):
        slots = np.nonzero(flat == e)[0]
        if len(slots) == 0:
            continue
        ntile = (len(slots) + 511) // 512
        for part in (slots[:512] // wl.k, slots[512 * (ntile - 1):] // wl.k):
            pick = np.unique(part)
            toks.update(int(t) for t in pick[np.linspace(0, len(pick) - 1, 2).astype(int)])
    toks = sorted(toks)
    ref = orc.moe_forward_layer(L, tokens=toks)
    compare(y[toks], ref, f"qwen T={T}, {len(toks)} tokens from every expert's first and last tile")
    _LAYERS.clear()


# ---------------------------------------------------------------------------
# matrix-core GEMV (weights decoded in registers into the MFMA B operand)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,T", [("tiny", None), ("qwen_decode", None), ("mixtral_decode", 8),
                                    ("mixtral_decode", 64)])
def test_forward_mgemv_forced(torch, name, T):
    L = layer_for(name, T=T)
    say(f"forward {name} T={L.wl.T} path=MGEMV")
    _, y = run_forward(torch, L, B.PW_PATH_MGEMV)
    compare(y, oracle_y(L), f"{name} mgemv")


def test_forward_mgemv_ragged_and_many_tokens(torch):
    # K tails inside a 128-wide chunk (gate_up K = 2080: 65 words; down K = 96: 3 words), experts with more than
    # 64 tokens (second pass over K), a single token, and I not a multiple of 8 rows' pairs
    for (H, I, E, k, T, seed) in [(2080, 96, 5, 3, 70, 51), (96, 1056, 4, 4, 45, 52), (256, 512, 2, 1, 150, 53),
                                  (160, 224, 3, 2, 1, 54), (64, 40 * 32, 2, 2, 33, 55), (256, 512, 2, 1, 48, 58),
                                  (64, 4128, 3, 2, 20, 59)]:
        L = custom_layer(H, I, E, k, T, seed)
        say(f"forward mgemv ragged H={H} I={I} E={E} k={k} T={T}")
        _, y = run_forward(torch, L, B.PW_PATH_MGEMV)
        compare(y, oracle_y(L), f"mgemv ragged H={H} I={I} T={T}")


def test_forward_mgemv_every_bitwidth_pair(torch):
    H, I, E, k, T, seed = 512, 256, 36, 4, 45, 56
    qvals = [(3 + e % 6, 3 + (e // 6) % 6) for e in range(E)]
    L = custom_layer(H, I, E, k, T, seed, qvals=qvals)
    say("forward mgemv every (gate_up, down) bitwidth pair")
    _, y = run_forward(torch, L, B.PW_PATH_MGEMV)
    compare(y, oracle_y(L), "mgemv bitwidth pairs")


def test_forward_mgemv_invalid_bitwidth_flagged_and_zero(torch):
    from any_precision_bitplane_amd.device import DeviceLayer
    L = custom_layer(256, 512, 4, 2, 40, 57)
    L.q[1, 0] = 9
    L.q[2, 1] = 2
    dev = DeviceLayer(L)
    say("forward mgemv with invalid bitwidths on two blocks")
    dev.forward(B.make_options(path=B.PW_PATH_MGEMV))
    torch.cuda.synchronize()
    assert dev.status() & B.PW_DEV_BAD_BITWIDTH
    compare(dev.y.float().cpu().numpy(), oracle_y(L), "mgemv invalid bitwidths")


def test_forward_auto_three_families(torch):
    """Batched Qwen-shaped layer with AUTO bands at 4 and 64 tokens: experts
    below 4 tokens on the GEMV kernels, 4..63 on the matrix-core GEMV, 64 and
    more on the MFMA kernels, in one call; then the default per-call rule."""
    L = layer_for("qwen_batched")
    counts = np.bincount(L.ids.reshape(-1), minlength=L.wl.E)
    c = counts[counts > 0]
    assert (c < 4).any() and ((c >= 4) & (c < 64)).any() and (c >= 64).any()
    say("forward qwen_batched T=256 AUTO bands 4 / 64")
    from any_precision_bitplane_amd.device import DeviceLayer
    dev = DeviceLayer(L)
    dev.forward(B.make_options(path=B.PW_PATH_AUTO, mgemv_min_tokens=4, mfma_min_tokens=64))
    torch.cuda.synchronize()
    ref = oracle_y(L)
    compare(dev.y.float().cpu().numpy(), ref, "qwen_batched auto three families")
    say("forward qwen_batched T=256 AUTO default rule")
    _, y = run_forward(torch, L, B.PW_PATH_AUTO, dev=dev)
    compare(y, ref, "qwen_batched auto default rule")


@pytest.mark.parametrize("H,I,E,k,T,seed", [(256, 512, 1, 1, 5, 61), (256, 512, 1, 1, 300, 62),
                                            (128, 256, 4, 4, 20, 63), (96, 160, 3, 3, 260, 64)])
def test_forward_auto_edge_layers(torch, H, I, E, k, T, seed):
    """AUTO on degenerate routing: one expert (a plain SwiGLU FFN) below and
    above the MFMA band, and k = E (every expert takes every token)."""
    L = custom_layer(H, I, E, k, T, seed)
    say(f"forward AUTO edge H={H} I={I} E={E} k={k} T={T}")
    dev, y = run_forward(torch, L, B.PW_PATH_AUTO)
    assert dev.status() == 0
    compare(y, oracle_y(L), f"auto edge E={E} k={k} T={T}")


_FAMILIES = {B.PW_PATH_GEMV: "gemv", B.PW_PATH_MGEMV: "mgemv", B.PW_PATH_MFMA: "mfma"}


@pytest.mark.parametrize("T,family,launched", [(6, B.PW_PATH_GEMV, ("gemv",)), (7, B.PW_PATH_MGEMV, ("mgemv",)),
                                               (256, B.PW_PATH_MGEMV, ("mgemv",)),
                                               (257, B.PW_PATH_MGEMV, ("mgemv", "mfma"))])
def test_auto_family_at_the_mean_edges(torch, T, family, launched):
    """AUTO runs one kernel family per call, chosen from the mean routed slots
    per routed expert m = T*k / min(E, T*k): GEMV for m < 1.6, matrix-core GEMV
    for 1.6 <= m <= 64, MFMA above, where an expert's tokens past its last whole
    512-token tile take the matrix-core GEMV when there are at most 96 of them.
    With E = 8, k = 2 the batches T = 6 / 7 / 256 / 257 sit on either side of
    both edges; at T = 257 every expert holds at most 96 tokens, so all of
    them are such tails and the MFMA kernels find no tile.  Every family is
    deterministic and sums in its own order (here with the down product's K
    range in one part on both GEMV forms), so AUTO's output equals the
    computing family's forced output bit for bit and differs from the others."""
    L = custom_layer(1024, 1024, 8, 2, T, 700 + T)
    info = B.pw_moe_path_info(B.shape(1024, 1024, 8, 2), T)
    assert _families(info) == launched
    forced = B.pw_moe_path_info(B.shape(1024, 1024, 8, 2), T, B.make_options(path=family))
    assert forced.down_kparts == info.down_kparts == 1
    if "mfma" in launched:
        assert info.mfma_tail == 96
        assert np.bincount(L.ids.reshape(-1), minlength=8).max() <= 96
    say(f"forward AUTO family edge T={T} (expect {_FAMILIES[family]})")
    dev, y_auto = run_forward(torch, L, B.PW_PATH_AUTO)
    assert dev.status() == 0
    same = []
    for f, name in _FAMILIES.items():
        say(f"  forced {name}")
        _, y_f = run_forward(torch, L, f, dev=dev)
        if np.array_equal(y_auto, y_f):
            same.append(f)
    assert same == [family], [_FAMILIES[f] for f in same]
    compare(y_auto, oracle_y(L), f"auto family edge T={T}")


def _families(info):
    return tuple(n for n in ("gemv", "mgemv", "mfma") if getattr(info, n))


def _designed_ids(counts, seed):
    """k = 1 routing with the given per-expert slot counts, in seeded token order."""
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    np.random.default_rng(seed).shuffle(ids)
    return ids.reshape(-1, 1)


@pytest.mark.parametrize("H,I,counts,kparts", [
    # tails of exactly 96 (matrix-core GEMV) and 97 (a partial MFMA tile), an
    # expert of 80 tokens (all of it a tail), a whole tile, an unrouted expert
    # and a one-token expert; I = 8224 splits the down product's K range in two
    # (33 quads of eight plane words), which both families then share
    (256, 8224, [608, 609, 80, 512, 0, 1], 2),
    # K range in one part; tails of 1, 31, 32, 33 and 95 tokens behind one or two whole tiles
    (512, 1024, [513, 543, 544, 1057, 607, 700], 1),
])
def test_forward_auto_prefill_tails(torch, H, I, counts, kparts):
    """AUTO's prefill form: MFMA tiles for whole 512-token runs, the
    matrix-core GEMV for short tails, both writing the same K parts of the
    expert outputs, against the oracle on every token."""
    E, T = len(counts), int(sum(counts))
    L = custom_layer(H, I, E, 1, T, 800 + T)
    L.ids = _designed_ids(counts, 810 + T)
    L.w = np.ones((T, 1), np.float32)
    info = B.pw_moe_path_info(B.shape(H, I, E, 1), T)
    assert _families(info) == ("mgemv", "mfma") and info.mfma_tail == 96 and info.down_kparts == kparts
    say(f"forward AUTO prefill tails H={H} I={I} counts={counts} down K parts={kparts}")
    dev, y = run_forward(torch, L, B.PW_PATH_AUTO)
    assert dev.status() == 0
    compare(y, oracle_y(L), f"auto prefill tails H={H} I={I}")


@pytest.mark.parametrize("H,I,E,k,T,seed", [(128, 96, 256, 64, 1, 71), (256, 128, 256, 8, 40, 72),
                                            (64, 64, 256, 256, 2, 73)])
def test_forward_largest_expert_counts_every_path(torch, H, I, E, k, T, seed):
    """The largest expert count the layer takes (E = 256): 64 slots routed
    inside the gate_up kernel (k = 64, one token), 320 slots over 179 experts
    through the route kernel, and k = E (every expert takes both tokens); AUTO
    and each family forced.  Routing weights are 1 (the layer uses them as
    given), which keeps the outputs well inside fp16's normal range."""
    L = custom_layer(H, I, E, k, T, seed)
    L.w[:] = 1.0
    ref = oracle_y(L)
    dev = None
    for path in (B.PW_PATH_AUTO, B.PW_PATH_GEMV, B.PW_PATH_MGEMV, B.PW_PATH_MFMA):
        say(f"forward E={E} k={k} T={T} H={H} I={I} path={path}")
        dev, y = run_forward(torch, L, path, dev=dev)
        assert dev.status() == 0
        compare(y, ref, f"E={E} k={k} T={T} path={path}")


# ---------------------------------------------------------------------------
# The forward kernels' own decode, read back exactly
# ---------------------------------------------------------------------------
# Tables chosen so that the layer's output is one column of a dequantized
# block: every gate weight 32 (with a one-hot token x, gate = 32 exactly and
# SiLU(32) = 32 exactly in fp32, since exp(-32) vanishes next to 1), so
#   readout "down": up row i_e's weights all 1/32 and the other up rows 0, so
#     h is exactly one-hot at i_e and y[t] = W_down[:, i_e] of the token's expert;
#   readout "up":   the down block the identity scaled by 1/32 (code 2^(q-1)
#     at (n, n), table entries 0 except that code's 1/32), so
#     h = 32 W_up[:, k0] and y[t][n] = W_up[n, k0] for n < min(H, I).
# Every product and sum on the way is exact in fp32 and the results are fp16
# values, so the kernels must reproduce the oracle's dequantized weights
# exactly (values compared, -0 equal to +0: a weight of -0 comes out as +0
# after the combine's add).
_F16_32, _F16_1_32 = 0x5000, 0x2800


def _table(L, e, m, N):
    q = int(L.q[e][m])
    off = orc.lut_offset(N, q)
    return L.luts[e][m][off: off + N * 2 ** q].reshape(N, 2 ** q)


def _readout_layer(H, I, E, T, seed, mode):
    L = custom_layer(H, I, E, 1, T, seed)
    L.q[:, 0] = [3 + (e % 6) for e in range(E)]
    L.q[:, 1] = [3 + ((e + 1) % 6) for e in range(E)]
    L.ids = (np.arange(T, dtype=np.int32) % E).reshape(T, 1)
    L.w = np.ones((T, 1), np.float32)
    k0 = [(7 * t + 3) % H for t in range(T)]
    L.x = np.zeros((T, H), np.float16)
    L.x[np.arange(T), k0] = 1.0
    col = [(37 * e + 5) % I for e in range(E)]
    for e in range(E):
        L.luts[e][0] = L.luts[e][0].copy()
        tab = _table(L, e, 0, 2 * I)
        tab[:I] = _F16_32                       # every gate weight 32
        if mode == "down":
            tab[I:] = 0
            tab[I + col[e]] = _F16_1_32
        else:
            pl = np.zeros_like(L.planes[e][1])
            n = np.arange(min(H, I))
            pl[0, n, n // 32] = (np.uint32(1) << (n % 32).astype(np.uint32))
            L.planes[e][1] = pl
            L.luts[e][1] = np.zeros_like(L.luts[e][1])
            tab_d = _table(L, e, 1, H)
            tab_d[n, 2 ** (int(L.q[e][1]) - 1)] = _F16_1_32
    if mode == "down":
        want = np.stack([orc.fp16_bits_to_f64(orc.dequant_block(L.planes[t % E][1], L.luts[t % E][1],
                                                                int(L.q[t % E][1])))[:, col[t % E]]
                         for t in range(T)])
    else:
        want = np.zeros((T, H))
        m = min(H, I)
        for t in range(T):
            e = t % E
            wgu = orc.fp16_bits_to_f64(orc.dequant_block(L.planes[e][0], L.luts[e][0], int(L.q[e][0])))
            want[t, :m] = wgu[I: I + m, k0[t]]
    return L, want


@pytest.mark.parametrize("mode", ["down", "up"])
@pytest.mark.parametrize("H,I", [(256, 192), (128, 2112)])
def test_forward_kernels_decode_weights_exactly(torch, mode, H, I):
    """Each kernel family's decode of the up and down blocks, through the
    forward itself, equals the oracle's dequantized weights exactly, at every
    bitwidth 3..8 (six experts, two tokens each); I = 2112 splits the GEMV's
    down product into two K parts."""
    E, T = 6, 12
    L, want = _readout_layer(H, I, E, T, 900 + H + (I if mode == "up" else 0), mode)
    # the oracle's own forward on the same layer gives the same columns (its
    # fp64 SiLU(32) is 32 (1 - 1.3e-14), not 32)
    np.testing.assert_allclose(oracle_y(L), want, rtol=1e-12, atol=0)
    dev = None
    for path in (B.PW_PATH_GEMV, B.PW_PATH_MGEMV, B.PW_PATH_MFMA, B.PW_PATH_AUTO):
        say(f"decode readout {mode} H={H} I={I} path={path}")
        dev, y = run_forward(torch, L, path, dev=dev)
        assert dev.status() == 0
        bad = np.argwhere(y.astype(np.float64) != want)
        assert bad.size == 0, (mode, path, bad[:5], y[tuple(bad[0])], want[tuple(bad[0])])


@pytest.mark.parametrize("H,I,E,k,T,seed", [(256, 8224, 2, 1, 1100, 81), (512, 384, 5, 2, 2660, 82),
                                            (384, 512, 3, 3, 1580, 83), (160, 352, 7, 2, 1890, 84),
                                            (1056, 224, 4, 4, 560, 85)])
def test_forward_auto_prefill_seeded_layers(torch, H, I, E, k, T, seed):
    """AUTO's prefill form on seeded layers whose experts end in short tails
    (11 to 66 tokens past whole 512-token tiles) next to a nearly full last
    tile, with odd numbers of MFMA tiles (grouped item order) and, at
    I = 8224, a two-part K split of the down product shared by both families."""
    L = custom_layer(H, I, E, k, T, seed)
    info = B.pw_moe_path_info(B.shape(H, I, E, k), T)
    assert _families(info) == ("mgemv", "mfma") and info.mfma_tail == 96
    say(f"forward AUTO prefill seeded H={H} I={I} E={E} k={k} T={T} down K parts={info.down_kparts}")
    dev, y = run_forward(torch, L, B.PW_PATH_AUTO)
    assert dev.status() == 0
    compare(y, oracle_y(L), f"auto prefill seeded H={H} I={I} E={E} k={k} T={T}")


@pytest.mark.parametrize("H,I,E,k,T,seed", [(16384, 32, 2, 2, 5, 91), (32, 16384, 2, 2, 5, 92),
                                            (8192, 96, 3, 1, 300, 93)])
def test_forward_extreme_aspect_ratios_every_path(torch, H, I, E, k, T, seed):
    """The widest hidden size over a one-word inner size (a 64-row gate_up
    block: one partial 128-row MFMA tile), the reverse (the down product's K
    range in eight parts on both GEMV forms and four on MFMA), and an
    8192-wide layer on AUTO's prefill form with its tails; each family forced
    and AUTO."""
    L = custom_layer(H, I, E, k, T, seed)
    L.w[:] = 1.0
    ref = oracle_y(L)
    dev = None
    for path in (B.PW_PATH_AUTO, B.PW_PATH_GEMV, B.PW_PATH_MGEMV, B.PW_PATH_MFMA):
        info = B.pw_moe_path_info(B.shape(H, I, E, k), T, B.make_options(path=path))
        say(f"forward H={H} I={I} E={E} k={k} T={T} path={path} down K parts={info.down_kparts}")
        dev, y = run_forward(torch, L, path, dev=dev)
        assert dev.status() == 0
        compare(y, ref, f"H={H} I={I} path={path}")


def _random_case(seed):
    rng = np.random.default_rng(9000 + seed)
    H = 32 * int(rng.integers(1, 40))
    I = 32 * int(rng.integers(1, 40))
    E = int(rng.integers(1, 24))
    k = int(rng.integers(1, min(E, 6) + 1))
    T = int(rng.choice([1, 2, 3, 5, 8, 17, 40, 70, 130, 300]))
    L = custom_layer(H, I, E, k, T, 9100 + seed)
    L.q[:] = rng.integers(3, 9, L.q.shape).astype(np.uint8)
    if seed % 5 == 0 and k > 1:   # some tokens list one expert twice
        L.ids[::3, 1] = L.ids[::3, 0]
    path = [B.PW_PATH_AUTO, B.PW_PATH_GEMV, B.PW_PATH_MGEMV, B.PW_PATH_MFMA][seed % 4]
    return L, path


@pytest.mark.parametrize("seed", range(24))
def test_forward_random_layers_every_path(torch, seed):
    """Seeded random shapes (H, I multiples of 32 up to 1248; E up to 23; k up
    to 6; T from 1 to 300), random bitwidths, some duplicate ids, each kernel
    family forced in turn and AUTO."""
    L, path = _random_case(seed)
    wl = L.wl
    say(f"forward random seed={seed} H={wl.H} I={wl.I} E={wl.E} k={wl.k} T={wl.T} path={path}")
    _, y = run_forward(torch, L, path)
    compare(y, oracle_y(L), f"random seed={seed} path={path}")
