"""ctypes binding of libpagedweight (C ABI in include/pagedweight.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Functions carry the C names.  Tensor arguments are torch tensors on
the GPU (their data_ptr() is passed); `stream` is a torch.cuda.Stream, a raw
hipStream_t integer, or None for torch's current stream.

The library must have been built (python -m any_precision_bitplane_amd.build);
loading fails loudly otherwise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int32, c_size_t, c_uint32, c_void_p
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpagedweight.so")

PW_OK = 0
PW_ERR_INVALID_ARG = -1
PW_ERR_UNSUPPORTED_SHAPE = -2
PW_ERR_BITWIDTH = -3
PW_ERR_WORKSPACE = -4
PW_ERR_ALIGNMENT = -5
PW_ERR_HIP = -6
PW_ERR_UNSUPPORTED = -7
PW_ERR_OUT_OF_MEMORY = -8

PW_PAGE_CPU = 0
PW_PAGE_GPU = 1
PW_PAGE_IN_TRANSFER = 2

PW_DEV_BAD_EXPERT_ID = 0x1
PW_DEV_BAD_BITWIDTH = 0x2

PW_PATH_AUTO = 0
PW_PATH_GEMV = 1
PW_PATH_MFMA = 2
PW_PATH_MGEMV = 3

PW_STAGE_ROUTE = 0
PW_STAGE_GATE_UP = 1
PW_STAGE_DOWN = 2
PW_STAGE_COMBINE = 3
PW_NUM_STAGES = 4

PW_EVENTS_STAGES = 0
PW_EVENTS_KERNELS = 1


class PwMoeShape(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("inter", c_int32), ("num_experts", c_int32), ("top_k", c_int32)]


class PwBlockDesc(ctypes.Structure):
    _fields_ = [("planes", c_void_p), ("lut_all", c_void_p)]


class PwMoeOptions(ctypes.Structure):
    _fields_ = [("path", c_int32), ("mfma_min_tokens", c_int32),
                ("stage_events", c_void_p * (PW_NUM_STAGES + 1)),
                ("mgemv_min_tokens", c_int32), ("event_mode", c_int32)]


class PwPageInfo(ctypes.Structure):
    _fields_ = [("desired", c_int32), ("committed", c_int32), ("resident", c_int32), ("pending", c_int32),
                ("state", c_int32), ("reserved", c_int32), ("arena_offset", ctypes.c_uint64)]


class PwPathInfo(ctypes.Structure):
    _fields_ = [("gemv", c_int32), ("mgemv", c_int32), ("mfma", c_int32), ("mgemv_from", c_int32),
                ("mfma_from", c_int32), ("inline_route", c_int32), ("down_kparts", c_int32), ("launches", c_int32),
                ("mfma_tail", c_int32)]


class PwPlanProblem(ctypes.Structure):
    _fields_ = [("num_blocks", c_int32), ("num_experts", c_int32), ("expert_of", c_void_p),
                ("plane_bytes", c_void_p), ("sensitivity", c_void_p), ("correction", c_void_p),
                ("routing_mass", c_void_p), ("hot_fraction", ctypes.c_double), ("floor_cold", c_int32),
                ("floor_hot", c_int32), ("hot_multiplier", ctypes.c_float), ("reserved", c_int32)]


class PwError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {pw_status_str(status)} ({status})")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpagedweight.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m any_precision_bitplane_amd.build`")
    lib = ctypes.CDLL(path)
    sig = {
        "pw_abi_version": (c_int32, []),
        "pw_status_str": (c_char_p, [c_int32]),
        "pw_plane_words": (c_size_t, [c_int32, c_int32]),
        "pw_lut_elems": (c_size_t, [c_int32]),
        "pw_lut_offset": (c_size_t, [c_int32, c_int32]),
        "pw_check_shape": (c_int32, [POINTER(PwMoeShape), c_int32]),
        "pw_workspace_bytes": (c_size_t, [POINTER(PwMoeShape), c_int32]),
        "pw_workspace_init": (c_int32, [c_void_p, c_size_t, c_void_p]),
        "pw_moe_forward": (c_int32, [POINTER(PwMoeShape), c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_size_t, POINTER(PwMoeOptions), c_void_p]),
        "pw_moe_forward_noalloc": (c_int32, [POINTER(PwMoeShape), c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_void_p, POINTER(PwMoeOptions), c_void_p]),
        "pw_moe_path_info": (c_int32, [POINTER(PwMoeShape), c_int32, POINTER(PwMoeOptions), POINTER(PwPathInfo)]),
        "pw_planes_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
        "pw_pack_planes": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
        "pw_dequant_block": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                       c_void_p]),
        "pw_get_device_status": (c_int32, [c_void_p, POINTER(c_uint32), c_void_p]),
        "pw_router_topk": (c_int32, [POINTER(PwMoeShape), c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "pw_moe_forward_routed": (c_int32, [POINTER(PwMoeShape), c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                            POINTER(PwMoeOptions), c_void_p]),
        "pw_moe_forward_layers": (c_int32, [POINTER(PwMoeShape), c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                            POINTER(PwMoeOptions), c_void_p]),
        "pw_plan_bitwidths": (c_int32, [POINTER(PwPlanProblem), c_void_p, ctypes.c_int64, c_void_p,
                                        POINTER(ctypes.c_int64), POINTER(c_int32)]),
        "pw_pager_create": (c_int32, [c_int32, POINTER(c_int32), POINTER(c_int32), c_void_p, c_size_t, c_void_p,
                                      c_void_p, POINTER(c_void_p)]),
        "pw_pager_destroy": (c_int32, [c_void_p]),
        "pw_pager_set_block": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p]),
        "pw_pager_request": (c_int32, [c_void_p, c_int32, c_int32]),
        "pw_pager_execute": (c_int32, [c_void_p, c_void_p]),
        "pw_pager_commit": (c_int32, [c_void_p, c_void_p, c_int32, POINTER(c_int32)]),
        "pw_pager_info": (c_int32, [c_void_p, c_int32, POINTER(PwPageInfo)]),
        "pw_pager_arena_used": (c_size_t, [c_void_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols() -> Sequence[str]:
    return ["pw_abi_version", "pw_status_str", "pw_plane_words", "pw_lut_elems", "pw_lut_offset",
            "pw_check_shape", "pw_workspace_bytes", "pw_workspace_init", "pw_moe_forward", "pw_moe_forward_noalloc",
            "pw_moe_path_info",
            "pw_dequant_block", "pw_planes_bytes", "pw_pack_planes", "pw_get_device_status", "pw_pager_create", "pw_pager_destroy",
            "pw_pager_set_block", "pw_pager_request", "pw_pager_execute", "pw_pager_commit", "pw_pager_info",
            "pw_pager_arena_used", "pw_router_topk", "pw_moe_forward_routed", "pw_moe_forward_layers",
            "pw_plan_bitwidths"]


# ---------------------------------------------------------------------------
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != PW_OK:
        raise PwError(status, what)


def shape(H: int, I: int, E: int, k: int) -> PwMoeShape:
    return PwMoeShape(H, I, E, k)


def pw_abi_version() -> int:
    return load().pw_abi_version()


def pw_status_str(status: int) -> str:
    return load().pw_status_str(status).decode()


def pw_plane_words(N: int, K: int) -> int:
    return load().pw_plane_words(N, K)


def pw_lut_elems(N: int) -> int:
    return load().pw_lut_elems(N)


def pw_lut_offset(N: int, b: int) -> int:
    return load().pw_lut_offset(N, b)


def pw_check_shape(shp: PwMoeShape, T: int) -> int:
    return load().pw_check_shape(ctypes.byref(shp), T)


def pw_workspace_bytes(shp: PwMoeShape, T_max: int) -> int:
    return load().pw_workspace_bytes(ctypes.byref(shp), T_max)


def pw_workspace_init(workspace, stream=None) -> None:
    _check(load().pw_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "pw_workspace_init")


def make_options(path: int = PW_PATH_AUTO, mfma_min_tokens: int = 0, events=None,
                 mgemv_min_tokens: int = 0, event_mode: int = 0) -> PwMoeOptions:
    o = PwMoeOptions()
    o.path = path
    o.mfma_min_tokens = mfma_min_tokens
    o.mgemv_min_tokens = mgemv_min_tokens
    o.event_mode = event_mode
    if events is not None:
        for i, ev in enumerate(events):
            o.stage_events[i] = ev
    return o


def pw_moe_forward(shp: PwMoeShape, T: int, x, ids, w, blocks, q, y, workspace,
                   opts: Optional[PwMoeOptions] = None, stream=None, check: bool = True) -> int:
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().pw_moe_forward(ctypes.byref(shp), T, _ptr(x), _ptr(ids), _ptr(w), _ptr(blocks), _ptr(q),
                               _ptr(y), _ptr(workspace), ws_bytes,
                               ctypes.byref(opts) if opts is not None else None, _stream(stream))
    if check:
        _check(st, "pw_moe_forward")
    return st


PW_NOALLOC_SCRATCH_BYTES = 64 << 20


def pw_moe_forward_noalloc(shp: PwMoeShape, T: int, x, ids, w, blocks, q, y, status=None,
                           opts: Optional[PwMoeOptions] = None, stream=None, check: bool = True) -> int:
    st = load().pw_moe_forward_noalloc(ctypes.byref(shp), T, _ptr(x), _ptr(ids), _ptr(w), _ptr(blocks), _ptr(q),
                                       _ptr(y), _ptr(status), ctypes.byref(opts) if opts is not None else None,
                                       _stream(stream))
    if check:
        _check(st, "pw_moe_forward_noalloc")
    return st


def pw_moe_path_info(shp: PwMoeShape, T: int, opts: Optional[PwMoeOptions] = None) -> PwPathInfo:
    info = PwPathInfo()
    _check(load().pw_moe_path_info(ctypes.byref(shp), T, ctypes.byref(opts) if opts is not None else None,
                                   ctypes.byref(info)), "pw_moe_path_info")
    return info


def pw_planes_bytes(N: int, K: int, nplanes: int) -> int:
    return load().pw_planes_bytes(N, K, nplanes)


def pw_pack_planes(canon, N: int, K: int, nplanes: int, module: int, dev_layout, stream=None,
                   check: bool = True) -> int:
    st = load().pw_pack_planes(_ptr(canon), N, K, nplanes, module, _ptr(dev_layout), _stream(stream))
    if check:
        _check(st, "pw_pack_planes")
    return st


def pw_dequant_block(planes, lut_all, N: int, K: int, q: int, w_out, module: int = 0, stream=None,
                     check: bool = True) -> int:
    st = load().pw_dequant_block(_ptr(planes), _ptr(lut_all), N, K, q, module, _ptr(w_out), _stream(stream))
    if check:
        _check(st, "pw_dequant_block")
    return st


def pw_get_device_status(workspace, stream=None) -> int:
    flags = c_uint32(0)
    _check(load().pw_get_device_status(_ptr(workspace), ctypes.byref(flags), _stream(stream)),
           "pw_get_device_status")
    return flags.value


# --- router ----------------------------------------------------------------
def pw_router_topk(shp: PwMoeShape, T: int, x, router_w, ids, w, stat_count=None, stat_mass=None, workspace=None,
                   stream=None, check: bool = True) -> int:
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().pw_router_topk(ctypes.byref(shp), T, _ptr(x), _ptr(router_w), _ptr(ids), _ptr(w), _ptr(stat_count),
                               _ptr(stat_mass), _ptr(workspace), ws_bytes, _stream(stream))
    if check:
        _check(st, "pw_router_topk")
    return st


def pw_moe_forward_routed(shp: PwMoeShape, T: int, x, router_w, blocks, q, y, stat_count, stat_mass, workspace,
                          opts: Optional[PwMoeOptions] = None, stream=None, check: bool = True) -> int:
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().pw_moe_forward_routed(ctypes.byref(shp), T, _ptr(x), _ptr(router_w), _ptr(blocks), _ptr(q), _ptr(y),
                                      _ptr(stat_count), _ptr(stat_mass), _ptr(workspace), ws_bytes,
                                      ctypes.byref(opts) if opts is not None else None, _stream(stream))
    if check:
        _check(st, "pw_moe_forward_routed")
    return st


def pw_moe_forward_layers(shp: PwMoeShape, T: int, x, router_ws, blocks, qs, y, stat_count, stat_mass, workspace,
                          opts: Optional[PwMoeOptions] = None, stream=None, check: bool = True) -> int:
    """router_ws, blocks, qs: sequences of device tensors, one per layer."""
    L = len(router_ws)
    arr = lambda ts: (c_void_p * L)(*[_ptr(t) for t in ts])
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().pw_moe_forward_layers(ctypes.byref(shp), L, T, _ptr(x), arr(router_ws), arr(blocks), arr(qs), _ptr(y),
                                      _ptr(stat_count), _ptr(stat_mass), _ptr(workspace), ws_bytes,
                                      ctypes.byref(opts) if opts is not None else None, _stream(stream))
    if check:
        _check(st, "pw_moe_forward_layers")
    return st


# --- planner ----------------------------------------------------------------
def pw_plan_bitwidths(q_cur, plane_bytes, expert_of, sensitivity, correction=None, routing_mass=None,
                      hot_fraction: float = 0.0, floor_cold: int = 3, floor_hot: int = 3,
                      hot_multiplier: float = 1.0, budget_bytes: int = 0, check: bool = True):
    """Host arrays (numpy) in, (status, q_out int32 [B], plane bytes, fits) out."""
    import numpy as np
    q_cur = np.ascontiguousarray(q_cur, dtype=np.int32)
    pb = np.ascontiguousarray(plane_bytes, dtype=np.int64)
    eo = np.ascontiguousarray(expert_of, dtype=np.int32)
    S = np.ascontiguousarray(sensitivity, dtype=np.float32).reshape(len(q_cur), 6)
    R = None if correction is None else np.ascontiguousarray(correction, dtype=np.float32).reshape(len(q_cur), 6)
    M = None if routing_mass is None else np.ascontiguousarray(routing_mass, dtype=np.float32)
    E = int(eo.max()) + 1 if M is None else len(M)
    prob = PwPlanProblem(len(q_cur), E, eo.ctypes.data, pb.ctypes.data, S.ctypes.data,
                         None if R is None else R.ctypes.data, None if M is None else M.ctypes.data,
                         float(hot_fraction), int(floor_cold), int(floor_hot), float(hot_multiplier), 0)
    out = np.zeros(len(q_cur), dtype=np.int32)
    used = ctypes.c_int64(0)
    fits = c_int32(0)
    st = load().pw_plan_bitwidths(ctypes.byref(prob), q_cur.ctypes.data, int(budget_bytes), out.ctypes.data,
                                  ctypes.byref(used), ctypes.byref(fits))
    if check:
        _check(st, "pw_plan_bitwidths")
    return st, out, used.value, bool(fits.value)


# --- weight pager ----------------------------------------------------------
def pw_pager_create(rows: Sequence[int], cols: Sequence[int], arena, arena_bytes: int, blocks, q) -> int:
    n = len(rows)
    r = (c_int32 * n)(*rows)
    c = (c_int32 * n)(*cols)
    out = c_void_p(0)
    _check(load().pw_pager_create(n, r, c, _ptr(arena), arena_bytes, _ptr(blocks), _ptr(q), ctypes.byref(out)),
           "pw_pager_create")
    return out.value


def pw_pager_destroy(pager: int) -> None:
    _check(load().pw_pager_destroy(pager), "pw_pager_destroy")


def pw_pager_set_block(pager: int, b: int, host_planes, lut_all) -> None:
    _check(load().pw_pager_set_block(pager, b, _ptr(host_planes), _ptr(lut_all)), "pw_pager_set_block")


def pw_pager_request(pager: int, b: int, desired: int, check: bool = True) -> int:
    st = load().pw_pager_request(pager, b, desired)
    if check:
        _check(st, "pw_pager_request")
    return st


def pw_pager_execute(pager: int, copy_stream=None, check: bool = True) -> int:
    st = load().pw_pager_execute(pager, _stream(copy_stream))
    if check:
        _check(st, "pw_pager_execute")
    return st


def pw_pager_commit(pager: int, stream=None, wait: bool = True) -> int:
    n = c_int32(0)
    _check(load().pw_pager_commit(pager, _stream(stream), 1 if wait else 0, ctypes.byref(n)), "pw_pager_commit")
    return n.value


def pw_pager_info(pager: int, b: int) -> PwPageInfo:
    info = PwPageInfo()
    _check(load().pw_pager_info(pager, b, ctypes.byref(info)), "pw_pager_info")
    return info


def pw_pager_arena_used(pager: int) -> int:
    return load().pw_pager_arena_used(pager)
