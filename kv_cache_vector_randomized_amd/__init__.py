"""TurboQuant-style KV-cache quantization and decode attention for MI355X (gfx950).

The compute lives in the HIP library libtq.so (C ABI in include/tq.h); `tq` is
its thin ctypes binding, `torch_api` a convenience layer that allocates the
paged cache and workspaces with PyTorch, and `synth` the seeded input recipes.
"""
