"""Host-side byte and flop accounting behind bench.py's roofline figures,
checked against the stored arrays of synthetic layers (no GPU needed)."""
import numpy as np

from any_precision_bitplane_amd import roofline, synth


def _stored_block_bytes(L, e, m):
    """Bytes of block (e, m) a call at its committed bitwidth must read,
    counted from the arrays themselves: planes 0..q-1 and the bitwidth-q table
    (table b of a block starts at element N*(2^b - 8))."""
    q = int(L.q[e][m])
    planes = L.planes[e][m]
    N = planes.shape[1]
    plane_bytes = int(planes[:q].nbytes)
    start, stop = N * (2 ** q - 8), N * (2 ** (q + 1) - 8)
    table_bytes = int(L.luts[e][m][start:stop].nbytes)
    return plane_bytes + table_bytes


def test_module_and_layer_bytes_match_stored_arrays():
    for name in ("tiny", "qwen_decode"):
        L = synth.make_layer(synth.WORKLOADS[name])
        wl = L.wl
        routed = sorted(set(int(e) for e in L.ids.reshape(-1) if 0 <= e < wl.E))
        for m in (0, 1):
            expect = sum(_stored_block_bytes(L, e, m) for e in routed) + wl.T * wl.H * 2 + wl.T * wl.k * 4
            got = roofline.module_bytes(L.q, L.ids, wl.H, wl.I, wl.E, wl.T, wl.k, m)
            assert got == expect, (name, m, got, expect)
        expect = (sum(_stored_block_bytes(L, e, m) for e in routed for m in (0, 1))
                  + 2 * wl.T * wl.H * 2 + wl.T * wl.k * 8 + 2 * wl.E)
        assert roofline.layer_bytes(L.q, L.ids, wl.H, wl.I, wl.E, wl.T, wl.k) == expect


def test_unrouted_and_out_of_range_experts_cost_nothing():
    L = synth.make_layer(synth.WORKLOADS["tiny"])
    wl = L.wl
    ids = np.full_like(L.ids, 3)
    ids[0, 0] = -1          # dropped slot
    ids[1, 0] = wl.E        # out of range
    only3 = roofline.module_bytes(L.q, ids, wl.H, wl.I, wl.E, wl.T, wl.k, 0)
    assert only3 == _stored_block_bytes(L, 3, 0) + wl.T * wl.H * 2 + wl.T * wl.k * 4


def test_layer_flops_counts_two_per_multiply_add():
    # gate_up: 2I x H weights, down: H x I, each used once per routed slot
    T, k, H, I = 5, 3, 64, 96
    assert roofline.layer_flops(T, k, H, I) == 2 * T * k * (2 * I * H + H * I)
