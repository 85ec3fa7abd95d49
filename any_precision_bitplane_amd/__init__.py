"""MI355X-native fused mixed-precision MoE expert layer (PagedWeight-style
bit-plane storage with per-block committed bitwidths).

Modules:
  binding  -- ctypes binding of libpagedweight (the C ABI in include/pagedweight.h)
  device   -- GPU-resident layer storage and page tables (torch for memory only)
  synth    -- seeded synthetic inputs
  build    -- in-tree hipcc build of libpagedweight.so
"""
__all__ = ["binding", "device", "synth", "build"]
