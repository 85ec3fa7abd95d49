"""The C-ABI library loads, exports every function its header declares, and its
host-side checks reject bad arguments before touching a device.  No GPU needed:
none of these calls reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

from any_precision_bitplane_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedweight.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pw_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libpagedweight.so is not built (python -m any_precision_bitplane_amd.build)")
    return B.load()


def test_every_declared_function_is_exported(lib):
    declared = header_functions()
    assert len(declared) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(pw_\w+)", out))
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)
    assert sorted(B.exported_symbols()) == declared


def test_version_and_status_strings(lib):
    assert B.pw_abi_version() == 4
    for s in (B.PW_OK, B.PW_ERR_INVALID_ARG, B.PW_ERR_UNSUPPORTED_SHAPE, B.PW_ERR_BITWIDTH,
              B.PW_ERR_WORKSPACE, B.PW_ERR_ALIGNMENT, B.PW_ERR_HIP, B.PW_ERR_UNSUPPORTED, 12345):
        assert isinstance(B.pw_status_str(s), str) and B.pw_status_str(s)


def test_storage_sizes(lib):
    assert B.pw_plane_words(2816, 2048) == 8 * 2816 * 64
    assert B.pw_plane_words(10, 33) == 0
    assert B.pw_lut_elems(2048) == 504 * 2048
    for b in range(3, 9):
        assert B.pw_lut_offset(2048, b) == 2048 * (2 ** b - 8)
    assert B.pw_lut_offset(2048, 2) == 0 and B.pw_lut_offset(2048, 9) == 0


def test_shape_checks(lib):
    ok = B.shape(2048, 1408, 60, 4)
    assert B.pw_check_shape(ok, 4) == B.PW_OK
    assert B.pw_check_shape(ok, 0) == B.PW_OK
    assert B.pw_check_shape(ok, -1) == B.PW_ERR_INVALID_ARG
    assert B.pw_check_shape(B.shape(2040, 1408, 60, 4), 4) == B.PW_ERR_UNSUPPORTED_SHAPE
    assert B.pw_check_shape(B.shape(2048, 1400, 60, 4), 4) == B.PW_ERR_UNSUPPORTED_SHAPE
    assert B.pw_check_shape(B.shape(2048, 1408, 4, 5), 4) == B.PW_ERR_UNSUPPORTED_SHAPE
    assert B.pw_check_shape(B.shape(2048, 1408, 257, 4), 4) == B.PW_ERR_UNSUPPORTED_SHAPE
    assert B.pw_check_shape(B.shape(0, 1408, 60, 4), 4) == B.PW_ERR_INVALID_ARG
    # a block's planes must stay below 2^31 bytes at 8 bits (2*I*H weights)
    assert B.pw_check_shape(B.shape(32768, 32768, 8, 2), 4) == B.PW_ERR_UNSUPPORTED_SHAPE
    assert B.pw_check_shape(B.shape(32768, 32736, 8, 2), 4) == B.PW_OK
    assert B.pw_workspace_bytes(B.shape(2040, 1408, 60, 4), 4) == 0


def test_workspace_size_grows_with_tokens(lib):
    shp = B.shape(2048, 1408, 60, 4)
    a, b = B.pw_workspace_bytes(shp, 4), B.pw_workspace_bytes(shp, 256)
    assert 0 < a < b
    # h (fp16, I wide) and o (fp32, H wide) per routed slot dominate
    assert b >= 256 * 4 * (1408 * 2 + 2048 * 4)
    assert a % 256 == 0 and b % 256 == 0


def _fwd(lib, shp, T, x=1 << 20, ids=1 << 20, w=1 << 20, blocks=1 << 20, q=1 << 20, y=1 << 20,
         ws=1 << 20, ws_bytes=1 << 40, opts=None):
    return lib.pw_moe_forward(ctypes.byref(shp), T, x, ids, w, blocks, q, y, ws, ws_bytes,
                              ctypes.byref(opts) if opts else None, None)


def test_forward_rejects_bad_arguments_before_launch(lib):
    shp = B.shape(256, 512, 8, 2)
    assert _fwd(lib, shp, 0) == B.PW_OK                        # T = 0: nothing enqueued
    assert _fwd(lib, shp, 4, x=None) == B.PW_ERR_INVALID_ARG
    assert _fwd(lib, shp, 4, ids=None) == B.PW_ERR_INVALID_ARG
    assert _fwd(lib, shp, 4, ws=None) == B.PW_ERR_INVALID_ARG
    assert _fwd(lib, shp, 4, x=(1 << 20) + 2) == B.PW_ERR_ALIGNMENT
    assert _fwd(lib, shp, 4, ws=(1 << 20) + 64) == B.PW_ERR_ALIGNMENT
    assert _fwd(lib, shp, 4, ws_bytes=100) == B.PW_ERR_WORKSPACE
    assert _fwd(lib, shp, 4, opts=B.make_options(path=7)) == B.PW_ERR_INVALID_ARG
    assert _fwd(lib, B.shape(250, 512, 8, 2), 4) == B.PW_ERR_UNSUPPORTED_SHAPE
    assert _fwd(lib, shp, -3) == B.PW_ERR_INVALID_ARG


def test_dequant_rejects_bad_arguments_before_launch(lib):
    f = lib.pw_dequant_block
    p = 1 << 20
    assert f(None, p, 16, 32, 4, 0, p, None) == B.PW_ERR_INVALID_ARG
    assert f(p, p, 16, 30, 4, 0, p, None) == B.PW_ERR_UNSUPPORTED_SHAPE
    assert f(p, p, 8, 32, 4, 1, p, None) == B.PW_ERR_UNSUPPORTED_SHAPE     # rows come in 16-row tiles
    assert f(p, p, 16, 32, 2, 0, p, None) == B.PW_ERR_BITWIDTH
    assert f(p, p, 16, 32, 9, 1, p, None) == B.PW_ERR_BITWIDTH
    assert f(p, p + 2, 16, 32, 4, 0, p, None) == B.PW_ERR_ALIGNMENT
    assert f(p, p, 0, 32, 4, 0, p, None) == B.PW_ERR_INVALID_ARG
    assert f(p, p, 16, 32, 4, 2, p, None) == B.PW_ERR_INVALID_ARG          # module 0 or 1


def test_device_layout_sizes(lib):
    # a plane of the device layout holds exactly the canonical plane's words
    for N, K in [(16, 32), (2816, 2048), (2048, 1408), (28672, 4096), (4096, 14336)]:
        for n in range(1, 9):
            assert B.pw_planes_bytes(N, K, n) == n * N * K // 8
    assert B.pw_planes_bytes(24, 32, 8) == 0        # N % 16
    assert B.pw_planes_bytes(16, 48, 8) == 0        # K % 32
    assert B.pw_planes_bytes(16, 32, 0) == 0 and B.pw_planes_bytes(16, 32, 9) == 0


def test_pack_rejects_bad_arguments_before_launch(lib):
    f = lib.pw_pack_planes
    p, q = 1 << 20, 1 << 24
    assert f(None, 16, 32, 8, 0, q, None) == B.PW_ERR_INVALID_ARG
    assert f(p, 16, 32, 8, 0, None, None) == B.PW_ERR_INVALID_ARG
    assert f(p, 16, 32, 0, 0, q, None) == B.PW_ERR_INVALID_ARG
    assert f(p, 16, 32, 9, 0, q, None) == B.PW_ERR_INVALID_ARG
    assert f(p, 16, 32, 8, 3, q, None) == B.PW_ERR_INVALID_ARG
    assert f(p, 16, 32, 8, 1, p, None) == B.PW_ERR_INVALID_ARG              # not in place
    assert f(p, 24, 32, 8, 1, q, None) == B.PW_ERR_UNSUPPORTED_SHAPE
    assert f(p, 16, 40, 8, 1, q, None) == B.PW_ERR_UNSUPPORTED_SHAPE
    assert f(p + 2, 16, 32, 8, 1, q, None) == B.PW_ERR_ALIGNMENT
    assert f(p, 16, 32, 8, 1, q + 4, None) == B.PW_ERR_ALIGNMENT


def test_status_and_init_reject_bad_arguments(lib):
    flags = ctypes.c_uint32(0)
    assert lib.pw_get_device_status(None, ctypes.byref(flags), None) == B.PW_ERR_INVALID_ARG
    assert lib.pw_get_device_status(1 << 20, None, None) == B.PW_ERR_INVALID_ARG
    assert lib.pw_workspace_init(None, 1024, None) == B.PW_ERR_INVALID_ARG
    assert lib.pw_workspace_init((1 << 20) + 16, 1024, None) == B.PW_ERR_ALIGNMENT


def test_router_rejects_bad_arguments_before_launch(lib):
    p = 1 << 20

    def route(shp, T, x=p, wr=p, ids=p, w=p, cnt=None, mass=None, ws=p, ws_bytes=1 << 40):
        return lib.pw_router_topk(ctypes.byref(shp), T, x, wr, ids, w, cnt, mass, ws, ws_bytes, None)

    shp = B.shape(256, 512, 8, 2)
    assert route(shp, 0) == B.PW_OK
    assert route(shp, 4, wr=None) == B.PW_ERR_INVALID_ARG
    assert route(shp, 4, ids=None) == B.PW_ERR_INVALID_ARG
    assert route(shp, 4, x=p + 2) == B.PW_ERR_ALIGNMENT
    assert route(shp, 4, cnt=p + 2) == B.PW_ERR_ALIGNMENT
    assert route(shp, 4, ws_bytes=100) == B.PW_ERR_WORKSPACE
    assert route(B.shape(256, 512, 128, 65), 4) == B.PW_ERR_UNSUPPORTED_SHAPE   # k > 64
    assert route(B.shape(256, 512, 8, 9), 4) == B.PW_ERR_UNSUPPORTED_SHAPE      # k > E
    f = lib.pw_moe_forward_routed
    assert f(ctypes.byref(shp), 4, p, p, None, p, p, None, None, p, 1 << 40, None, None) == B.PW_ERR_INVALID_ARG
    assert f(ctypes.byref(shp), 4, p, p, p, p, p + 2, None, None, p, 1 << 40, None, None) == B.PW_ERR_ALIGNMENT
    assert f(ctypes.byref(shp), 4, p, p, p, p, p, None, None, p, 100, None, None) == B.PW_ERR_WORKSPACE
    assert f(ctypes.byref(shp), 0, p, p, p, p, p, None, None, p, 1 << 40, None, None) == B.PW_OK


def _families(info):
    return tuple(n for n in ("gemv", "mgemv", "mfma") if getattr(info, n))


# fams: the families whose kernels run; ("mgemv", "mfma") on the AUTO rule's
# prefill side means MFMA with the matrix-core GEMV taking the experts' tails
@pytest.mark.parametrize("shp,T,fams,inline,launches,kparts", [
    # E = 8, k = 2: the mean routed slots per routed expert m = T*k / min(E, T*k) crosses 1.6 at T = 7 and 64 at
    # T = 257
    ((1024, 1024, 8, 2), 1, ("gemv",), 1, 3, None),
    ((1024, 1024, 8, 2), 6, ("gemv",), 1, 3, None),
    ((1024, 1024, 8, 2), 7, ("mgemv",), 0, 4, 1),
    ((1024, 1024, 8, 2), 256, ("mgemv",), 0, 4, 1),
    ((1024, 1024, 8, 2), 257, ("mgemv", "mfma"), 0, 6, 1),
    # Qwen-shaped layer: decode, 16 tokens (64 slots, still routed inline), 17 tokens (a route kernel), batched
    ((2048, 1408, 60, 4), 4, ("gemv",), 1, 3, 1),
    ((2048, 1408, 60, 4), 16, ("gemv",), 1, 3, None),
    ((2048, 1408, 60, 4), 17, ("gemv",), 0, 4, 1),
    ((2048, 1408, 60, 4), 256, ("mgemv",), 0, 4, 1),
    # Mixtral-shaped layer: one token splits the down product's K range over 4 waves; prefill is MFMA,
    # its down product in one K part (16 token tiles x 32 row tiles fill 256 CUs twice)
    ((4096, 14336, 8, 2), 1, ("gemv",), 1, 3, 4),
    # 64 tokens: matrix-core GEMV alone, its down product in two K parts (8 tiles x 128 chunks)
    ((4096, 14336, 8, 2), 64, ("mgemv",), 0, 4, 2),
    ((4096, 14336, 8, 2), 4096, ("mgemv", "mfma"), 0, 6, 1),
    ((4096, 14336, 8, 2), 16384, ("mgemv", "mfma"), 0, 6, 1),
])
def test_path_info_auto_rule(lib, shp, T, fams, inline, launches, kparts):
    info = B.pw_moe_path_info(B.shape(*shp), T)
    assert _families(info) == fams
    assert info.inline_route == inline and info.launches == launches
    if kparts is not None:
        assert info.down_kparts == kparts
    prefill = "mfma" in fams
    assert info.mgemv_from == (1 if "mgemv" in fams and not prefill else 0)
    assert info.mfma_from == (1 if prefill else 0)
    assert info.mfma_tail == (96 if prefill else 0)


def test_path_info_forced_paths_and_bands(lib):
    s = B.shape(2048, 1408, 60, 4)
    i = B.pw_moe_path_info(s, 4096, B.make_options(path=B.PW_PATH_GEMV))
    assert _families(i) == ("gemv",) and i.launches == 4 and i.down_kparts == 1
    i = B.pw_moe_path_info(s, 1, B.make_options(path=B.PW_PATH_MFMA))
    assert _families(i) == ("mfma",) and i.mfma_from == 1 and i.inline_route == 0 and i.mfma_tail == 0
    i = B.pw_moe_path_info(s, 1, B.make_options(path=B.PW_PATH_MGEMV))
    assert _families(i) == ("mgemv",) and i.mgemv_from == 1
    # explicit bands on a batch averaging 17 slots per expert: all three families, in one call
    i = B.pw_moe_path_info(s, 256, B.make_options(mgemv_min_tokens=4, mfma_min_tokens=64))
    assert _families(i) == ("gemv", "mgemv", "mfma") and (i.mgemv_from, i.mfma_from) == (4, 64)
    assert i.launches == 1 + 2 * 3 + 1 and i.mfma_tail == 0
    # explicit bands keep every MFMA expert whole on the MFMA kernels
    i = B.pw_moe_path_info(B.shape(4096, 14336, 8, 2), 4096, B.make_options(mfma_min_tokens=1))
    assert _families(i) == ("mfma",) and i.mfma_tail == 0 and i.launches == 4
    # an MFMA band no expert can reach is not launched; below a mean of 1.6 the GEMV keeps every expert
    i = B.pw_moe_path_info(s, 4, B.make_options(mfma_min_tokens=256))
    assert _families(i) == ("gemv",) and i.inline_route == 1
    # nothing to do
    i = B.pw_moe_path_info(s, 0)
    assert _families(i) == () and i.launches == 0


def test_path_info_rejects_what_the_forward_rejects(lib):
    s = B.shape(2048, 1408, 60, 4)
    with pytest.raises(B.PwError):
        B.pw_moe_path_info(s, 4, B.make_options(path=7))
    with pytest.raises(B.PwError):
        B.pw_moe_path_info(B.shape(2048, 1408, 60, 61), 4)          # top_k > E
    with pytest.raises(B.PwError):                                     # 32-bit activation offsets
        B.pw_moe_path_info(B.shape(4096, 14336, 8, 2), 40000, B.make_options(path=B.PW_PATH_MGEMV))
    assert lib.pw_moe_path_info(ctypes.byref(s), 4, None, None) == B.PW_ERR_INVALID_ARG


def test_multi_layer_call_rejects_bad_arguments_before_launch(lib):
    p = 1 << 20
    shp = B.shape(256, 512, 8, 2)
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)

    def call(L, T=4, wr=None, bl=None, q=None, x=p, y=p, ws=p, ws_bytes=1 << 40, opts=None):
        wr = wr if wr is not None else arr(*([p] * max(L, 1)))
        bl = bl if bl is not None else arr(*([p] * max(L, 1)))
        q = q if q is not None else arr(*([p] * max(L, 1)))
        return lib.pw_moe_forward_layers(ctypes.byref(shp), L, T, x, wr, bl, q, y, None, None, ws, ws_bytes,
                                         ctypes.byref(opts) if opts is not None else None, None)

    assert call(0) == B.PW_ERR_INVALID_ARG
    assert call(2, wr=arr(p, None)) == B.PW_ERR_INVALID_ARG
    assert call(2, q=arr(None, p)) == B.PW_ERR_INVALID_ARG
    assert call(2, bl=arr(p, p + 4)) == B.PW_ERR_ALIGNMENT
    assert call(2, x=None) == B.PW_ERR_INVALID_ARG
    assert call(2, ws=None) == B.PW_ERR_INVALID_ARG
    assert call(2, ws_bytes=16) == B.PW_ERR_WORKSPACE
    assert call(2, T=0) == B.PW_OK
    ev = B.make_options(events=[p, p, p, p, p])
    assert call(2, opts=ev) == B.PW_ERR_UNSUPPORTED
    big = B.shape(32768, 64, 8, 2)
    assert lib.pw_moe_forward_layers(ctypes.byref(big), 2, 4, p, arr(p, p), arr(p, p), arr(p, p), p, None, None, p,
                                     1 << 40, None, None) == B.PW_ERR_UNSUPPORTED_SHAPE
