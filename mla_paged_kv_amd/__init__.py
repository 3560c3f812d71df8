"""MLA decode over a paged KV cache for AMD Instinct MI355X (gfx950).

The compute lives in ``libmla_paged_kv.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/mla_paged_kv.h``).  ``mla_paged_kv_amd.ops`` is a
thin ctypes binding with the same names; it raises if the library is missing
rather than computing anything on the host.  Submodules load lazily so that
``mla_paged_kv_amd.workloads`` (seeded inputs) imports without the library.
"""

import importlib

__version__ = "0.1.0"

__all__ = ["ops", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(__name__ + "." + name)
    raise AttributeError(name)
