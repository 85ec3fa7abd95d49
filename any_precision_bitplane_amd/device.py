"""Device-memory plumbing: place a layer's storage, page table and activations
in GPU memory (torch tensors) and call the library on them.

Nothing here computes any part of the layer; it allocates, copies and passes
pointers.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from . import binding


def pack_to_device(planes: np.ndarray, module: int, device, nplanes: int = 8):
    """Canonical planes uint32 [8][N][K/32] (host) -> the device layout the
    kernels read (a torch int32 tensor of pw_planes_bytes(N, K, nplanes)
    bytes), through pw_pack_planes on the GPU."""
    import torch
    _, N, W = planes.shape
    canon = _to_dev(np.ascontiguousarray(planes[:nplanes]), device)
    out = torch.empty(binding.pw_planes_bytes(N, 32 * W, nplanes) // 4, dtype=torch.int32, device=device)
    binding.pw_pack_planes(canon, N, 32 * W, nplanes, module, out)
    return out


def pack_to_host(planes: np.ndarray, module: int, device) -> np.ndarray:
    """Canonical planes -> device layout, returned as a host uint32 array of
    the same shape (for pinned host copies the pager reloads from)."""
    import torch
    dev = pack_to_device(planes, module, device)
    torch.cuda.synchronize()
    return dev.cpu().numpy().view(np.uint32).reshape(planes.shape)


def _to_dev(a: np.ndarray, device):
    import torch
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceLayer:
    """One MoE layer resident on the GPU.

    ``copies`` > 1 keeps that many copies of the expert storage at different
    addresses (each with its own page table), so that a benchmark can rotate
    between them and read weights from HBM rather than from on-chip caches.
    Only the blocks listed in ``experts`` (default: all) get their own storage
    in the extra copies; the others keep pointing at copy 0.
    """

    def __init__(self, layer, device: str = "cuda:0", copies: int = 1, experts: Optional[List[int]] = None):
        import torch
        wl = layer.wl
        self.wl = wl
        self.device = device
        self.shape = binding.shape(wl.H, wl.I, wl.E, wl.k)
        self.T = wl.T
        self.planes = [[[None, None] for _ in range(wl.E)] for _ in range(copies)]
        self.luts = [[[None, None] for _ in range(wl.E)] for _ in range(copies)]
        for e in range(wl.E):
            for m in (0, 1):
                self.planes[0][e][m] = pack_to_device(layer.planes[e][m], m, device)
                self.luts[0][e][m] = _to_dev(layer.luts[e][m], device)
        sel = set(range(wl.E)) if experts is None else set(experts)
        for c in range(1, copies):
            for e in range(wl.E):
                for m in (0, 1):
                    if e in sel:
                        self.planes[c][e][m] = self.planes[0][e][m].clone()
                        self.luts[c][e][m] = self.luts[0][e][m].clone()
                    else:
                        self.planes[c][e][m] = self.planes[0][e][m]
                        self.luts[c][e][m] = self.luts[0][e][m]
        self.blocks = [self._page_table(c) for c in range(copies)]
        self.q = _to_dev(layer.q, device)
        self.x = torch.from_numpy(layer.x).to(device)
        self.ids = _to_dev(layer.ids, device)
        self.w = _to_dev(layer.w, device)
        self.y = torch.empty((wl.T, wl.H), dtype=torch.float16, device=device)
        self.ws_bytes = binding.pw_workspace_bytes(self.shape, wl.T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        binding.pw_workspace_init(self.ws)

    def _page_table(self, c: int):
        wl = self.wl
        desc = np.zeros((wl.E, 2, 2), dtype=np.uint64)
        for e in range(wl.E):
            for m in (0, 1):
                desc[e, m, 0] = self.planes[c][e][m].data_ptr()
                desc[e, m, 1] = self.luts[c][e][m].data_ptr()
        return _to_dev(desc.view(np.int64), self.device)

    def set_tokens(self, layer) -> None:
        """Point the layer at another batch (x, ids, w of ``layer``, which must
        share this layer's shape and storage); the expert storage stays."""
        import torch
        wl = layer.wl
        assert (wl.H, wl.I, wl.E, wl.k) == (self.wl.H, self.wl.I, self.wl.E, self.wl.k)
        self.wl = wl
        self.T = wl.T
        self.x = torch.from_numpy(layer.x).to(self.device)
        self.ids = _to_dev(layer.ids, self.device)
        self.w = _to_dev(layer.w, self.device)
        self.y = torch.empty((wl.T, wl.H), dtype=torch.float16, device=self.device)
        self.ws_bytes = binding.pw_workspace_bytes(self.shape, wl.T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        binding.pw_workspace_init(self.ws)

    def set_q(self, q: np.ndarray):
        """Commit new bitwidths: a stream-ordered write of the q table."""
        self.q.copy_(_to_dev(np.asarray(q, dtype=np.uint8), self.device))

    def forward(self, opts=None, copy: int = 0, stream=None, check: bool = True, y=None) -> int:
        return binding.pw_moe_forward(self.shape, self.T, self.x, self.ids, self.w, self.blocks[copy], self.q,
                                      self.y if y is None else y, self.ws, opts=opts, stream=stream, check=check)

    def status(self) -> int:
        return binding.pw_get_device_status(self.ws)


class PagedLayer:
    """One MoE layer whose plane storage the library's weight pager manages.

    The host keeps every block's eight planes in pinned memory; the GPU keeps
    the committed prefix of each block in one device arena.  The tables stay
    resident.  Bitwidth changes go through ``request`` / ``execute`` /
    ``commit`` (the pager calls of the C ABI); ``forward`` reads the page table
    the pager maintains.
    """

    def __init__(self, layer, arena_bytes: int, device: str = "cuda:0"):
        import torch
        wl = layer.wl
        self.wl = wl
        self.device = device
        self.shape = binding.shape(wl.H, wl.I, wl.E, wl.k)
        self.T = wl.T
        self.nblocks = 2 * wl.E
        self.rows = [2 * wl.I if b % 2 == 0 else wl.H for b in range(self.nblocks)]
        self.cols = [wl.H if b % 2 == 0 else wl.I for b in range(self.nblocks)]
        self.host_planes = []
        self.luts = []
        for e in range(wl.E):
            for m in (0, 1):
                src = torch.from_numpy(pack_to_host(layer.planes[e][m], m, device).view(np.int32))
                hp = torch.empty(src.shape, dtype=torch.int32, pin_memory=True)
                hp.copy_(src)
                self.host_planes.append(hp)
                self.luts.append(_to_dev(layer.luts[e][m], device))
        self.blocks = torch.zeros((self.nblocks, 2), dtype=torch.int64, device=device)
        self.q = torch.zeros(self.nblocks, dtype=torch.uint8, device=device)
        self.arena_bytes = int(arena_bytes)
        self.arena = torch.empty(self.arena_bytes, dtype=torch.uint8, device=device)
        torch.cuda.synchronize()
        self.pager = binding.pw_pager_create(self.rows, self.cols, self.arena, self.arena_bytes, self.blocks, self.q)
        for b in range(self.nblocks):
            binding.pw_pager_set_block(self.pager, b, self.host_planes[b].data_ptr(), self.luts[b])
        self.x = torch.from_numpy(layer.x).to(device)
        self.ids = _to_dev(layer.ids, device)
        self.w = _to_dev(layer.w, device)
        self.y = torch.empty((wl.T, wl.H), dtype=torch.float16, device=device)
        self.ws_bytes = binding.pw_workspace_bytes(self.shape, wl.T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        binding.pw_workspace_init(self.ws)

    def plane_bytes(self, b: int) -> int:
        return self.rows[b] * self.cols[b] // 8

    def request(self, q: np.ndarray) -> None:
        """Desired bitwidths for every block, q [E][2] (host bookkeeping)."""
        q = np.asarray(q).reshape(-1)
        for b in range(self.nblocks):
            binding.pw_pager_request(self.pager, b, int(q[b]))

    def execute(self, copy_stream=None, check: bool = True) -> int:
        return binding.pw_pager_execute(self.pager, copy_stream, check=check)

    def commit(self, stream=None, wait: bool = True) -> int:
        return binding.pw_pager_commit(self.pager, stream, wait)

    def info(self, b: int):
        return binding.pw_pager_info(self.pager, b)

    def committed(self) -> np.ndarray:
        return np.array([self.info(b).committed for b in range(self.nblocks)], dtype=np.uint8).reshape(-1, 2)

    def forward(self, opts=None, stream=None, check: bool = True, y=None) -> int:
        return binding.pw_moe_forward(self.shape, self.T, self.x, self.ids, self.w, self.blocks, self.q,
                                      self.y if y is None else y, self.ws, opts=opts, stream=stream, check=check)

    def status(self) -> int:
        return binding.pw_get_device_status(self.ws)

    def close(self) -> None:
        if getattr(self, "pager", None):
            binding.pw_pager_destroy(self.pager)
            self.pager = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
