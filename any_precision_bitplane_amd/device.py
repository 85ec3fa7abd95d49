"""Device-memory plumbing: place a layer's storage, page table and activations
in GPU memory (torch tensors) and call the library on them.

Nothing here computes any part of the layer; it allocates, copies and passes
pointers.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from . import binding


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
                self.planes[0][e][m] = _to_dev(layer.planes[e][m], device)
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

    def set_q(self, q: np.ndarray):
        """Commit new bitwidths: a stream-ordered write of the q table."""
        self.q.copy_(_to_dev(np.asarray(q, dtype=np.uint8), self.device))

    def forward(self, opts=None, copy: int = 0, stream=None, check: bool = True, y=None) -> int:
        return binding.pw_moe_forward(self.shape, self.T, self.x, self.ids, self.w, self.blocks[copy], self.q,
                                      self.y if y is None else y, self.ws, opts=opts, stream=stream, check=check)

    def status(self) -> int:
        return binding.pw_get_device_status(self.ws)
