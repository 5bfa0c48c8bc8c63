"""Fused Conv2d + folded BatchNorm + activation for AMD MI355X (gfx950).

The compute path is the HIP library ``libcvx.so`` behind the C ABI declared in
``include/cvx.h``; ``conv2d_batchnorm_activation_amd.cvx`` is its thin ctypes
binding (argument marshalling only).  Importing the binding raises if the
library has not been built: there is no CPU fallback.

``accounting`` (pure Python FLOP/byte counts for throughput reporting) does
not load the library.
"""
__all__ = ["cvx", "accounting"]


def __getattr__(name):
    if name == "cvx":
        import importlib
        return importlib.import_module(".cvx", __name__)
    if name.startswith("cvx_") or name in ("CvxError", "Status"):
        import importlib
        return getattr(importlib.import_module(".cvx", __name__), name)
    raise AttributeError(name)
