"""MI355X-native routed MoE FFN layer (Kimi-K2 shape): HIP kernels behind a C ABI.

Submodules:
  binding -- ctypes binding of libmoe.so (moe_route, moe_permute, moe_expert_ffn,
             moe_combine, moe_layer_forward); loads the library on first use.
  inputs  -- seeded synthetic inputs (shapes and distributions of the workloads).
  build   -- compiles libmoe.so for gfx950 with hipcc.
"""
