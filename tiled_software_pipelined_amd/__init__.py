"""Tiled, software-pipelined GEMM for AMD MI355X (gfx950).

The product is the C-ABI library ``libtgemm.so`` built from ``csrc/``; this
package is its thin Python binding.  Importing the package loads nothing: the
library is opened on first use by :mod:`tiled_software_pipelined_amd.lib`,
which raises if it is missing (there is no CPU fallback).
"""

__all__ = ["gemm", "Plan", "Variant"]


def __getattr__(name):
    if name in ("gemm", "Plan", "Variant"):
        from . import lib
        return getattr(lib, name)
    raise AttributeError(name)
