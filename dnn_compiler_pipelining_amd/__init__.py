"""libattn: fused grouped-query softmax attention forward for AMD MI355X (gfx950).

Submodules:
  binding  -- ctypes binding of the C ABI in include/attn.h (loads libattn.so)
  inputs   -- seeded synthetic workloads (no attention arithmetic)
  build    -- hipcc build of libattn.so
"""
