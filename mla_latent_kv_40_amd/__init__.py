"""libmla: Multi-head Latent Attention decode over a paged latent cache, for AMD MI355X (gfx950).

The compute lives in hand-written HIP kernels behind a C ABI (``include/mla.h``,
``libmla.so`` built in this directory).  ``mla_latent_kv_40_amd.binding`` is a thin
ctypes layer with the same entry-point names; importing this package does not load
the library.
"""
__all__ = ["workloads", "binding"]
