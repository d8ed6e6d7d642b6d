"""MI355X-native DeepSeek Sparse Attention (DSA) layer.

The compute path is the HIP library ``libdsa.so`` (hand-written gfx950 kernels behind a C
ABI, declared in ``include/dsa.h``).  ``binding`` marshals torch device tensors into that
ABI; torch provides device memory and streams only.  Importing this package loads nothing;
the library is loaded on the first call and a missing library raises an error.
"""

from . import workloads  # noqa: F401

__all__ = ["workloads", "inputs", "binding"]


def __getattr__(name):
    if name in ("inputs", "binding"):
        import importlib
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
