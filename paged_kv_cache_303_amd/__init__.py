"""Paged-KV decode attention for MI355X (gfx950): HIP kernels behind a C ABI.

The product is ``libpa.so`` (built from ``csrc/``): slot-mapped cache writes,
single-pass and split-sequence paged decode attention with a log-sum-exp
reduce, whole-block copies for copy-on-write, and a host-side block pool.
``paged_kv_cache_303_amd.binding`` is a thin ctypes layer with the same
names, taking torch tensors for device memory and the current HIP stream.
``workloads`` draws seeded synthetic inputs.

Submodules are imported on first use so that ``workloads`` can be used
without loading the native library; the binding raises if ``libpa.so`` is
missing -- there is no CPU fallback.
"""

import importlib

__all__ = ["binding", "workloads", "build", "runner"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
