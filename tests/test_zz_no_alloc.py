"""The allocation-free forward (pw_moe_forward_noalloc) against pw_moe_forward:
same kernels, so the outputs must be identical bit for bit, and both within
the oracle's tolerance.  Two calls in a row, the second with a smaller input,
so the second call runs over what the first left in the static scratch."""
import sys

import numpy as np
import pytest

import oracle.pagedweight_oracle as orc
from any_precision_bitplane_amd import binding as B
from any_precision_bitplane_amd import synth

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_ABS = 2e-2


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


def _check_oracle(y, L, ids=None):
    ref = orc.moe_forward_layer(L, ids=ids)
    err = y.astype(np.float64) - ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
    mx = float(np.max(np.abs(err)))
    say(f"  vs oracle: rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert np.all(np.isfinite(y)) and rel <= REL_L2 and mx <= MAX_ABS, (rel, mx)


def _both(torch, L, ids=None, opts=None, dev=None):
    """y from pw_moe_forward (workspace) and from pw_moe_forward_noalloc, and
    the status word the latter raised."""
    from any_precision_bitplane_amd.device import DeviceLayer
    dev = dev or DeviceLayer(L)
    if ids is not None:
        dev.ids.copy_(torch.from_numpy(ids))
    dev.forward(opts)
    y_ws = dev.y.clone()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    y_na = torch.full_like(dev.y, 7.0)
    B.pw_moe_forward_noalloc(dev.shape, L.wl.T, dev.x, dev.ids, dev.w, dev.blocks[0], dev.q, y_na, status,
                             opts=opts)
    torch.cuda.synchronize()
    return y_ws.float().cpu().numpy(), y_na.float().cpu().numpy(), int(status.item()), dev


def test_noalloc_two_calls_second_smaller(torch):
    # first: Qwen-shaped layer, 64 tokens (matrix-core GEMV, route kernel);
    # second: the 4-token decode call (GEMV, routing inside gate_up)
    for T in (64, 4):
        wl = synth.WORKLOADS["qwen_decode"].with_T(T)
        L = synth.make_routed_layer(wl)
        say(f"noalloc forward qwen_decode T={T}")
        y_ws, y_na, st, _ = _both(torch, L)
        assert st == 0
        assert np.array_equal(y_ws, y_na), f"T={T}: {np.count_nonzero(y_ws != y_na)} elements differ"
        _check_oracle(y_na, L)


def test_noalloc_reports_device_errors_in_the_callers_word(torch):
    wl = synth.WORKLOADS["tiny"]
    L = synth.make_layer(wl)
    ids = L.ids.copy()
    ids[2, 1] = wl.E + 3
    say("noalloc forward tiny with one out-of-range id")
    y_ws, y_na, st, dev = _both(torch, L, ids=ids)
    assert st == B.PW_DEV_BAD_EXPERT_ID
    assert dev.status() & B.PW_DEV_BAD_EXPERT_ID     # the workspace call flagged it too
    assert np.array_equal(y_ws, y_na)
    _check_oracle(y_na, L, ids=ids)


def test_noalloc_rejects_calls_beyond_its_scratch(torch):
    wl = synth.WORKLOADS["mixtral_prefill"]
    shp = B.shape(wl.H, wl.I, wl.E, wl.k)
    need = B.pw_workspace_bytes(shp, wl.T)
    assert need > B.PW_NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(16, dtype=torch.int32, device="cuda")
    say(f"noalloc forward asked for {need} scratch bytes (host-side rejection, nothing launched)")
    st = B.pw_moe_forward_noalloc(shp, wl.T, dummy, dummy, dummy, dummy, dummy, dummy, check=False)
    assert st == B.PW_ERR_WORKSPACE


def test_noalloc_largest_call_its_scratch_holds(torch):
    # the largest Qwen-shaped call whose workspace fits the static scratch
    # (found from pw_workspace_bytes, one token more does not fit), on the
    # family AUTO picks and on the MFMA kernels forced through the options
    shp = B.shape(2048, 1408, 60, 4)
    lim = B.PW_NOALLOC_SCRATCH_BYTES
    lo, hi = 1, 1 << 16
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if B.pw_workspace_bytes(shp, mid) <= lim:
            lo = mid
        else:
            hi = mid - 1
    T = lo
    assert B.pw_workspace_bytes(shp, T + 1) > lim
    wl = synth.WORKLOADS["qwen_decode"].with_T(T)
    L = synth.make_routed_layer(wl)
    ref = orc.moe_forward_layer(L)
    dev = None
    for path in (B.PW_PATH_AUTO, B.PW_PATH_MFMA):
        opts = B.make_options(path=path)
        info = B.pw_moe_path_info(shp, T, opts)
        say(f"noalloc forward qwen_decode T={T} path={path} mgemv={info.mgemv} mfma={info.mfma} "
            f"(workspace {B.pw_workspace_bytes(shp, T)} of {lim} bytes)")
        y_ws, y_na, st, dev = _both(torch, L, opts=opts, dev=dev)
        assert st == 0
        assert np.array_equal(y_ws, y_na), f"T={T} path={path}: {np.count_nonzero(y_ws != y_na)} elements differ"
        err = y_na.astype(np.float64) - ref
        rel = np.linalg.norm(err) / np.linalg.norm(ref)
        say(f"  vs oracle: rel_l2={rel:.3e} max_abs={np.max(np.abs(err)):.3e}")
        assert rel <= REL_L2 and np.max(np.abs(err)) <= MAX_ABS
