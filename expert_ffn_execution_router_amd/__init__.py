"""Routed MoE-layer forward over an HBM expert slot pool, MI355X (gfx950).

libmoe.so (HIP kernels + host C++) implements the layer behind the C ABI of
include/moe.h; `binding` exposes those calls under the same names and
`runtime` holds the torch-allocated device buffers around one context.
"""
from . import binding  # noqa: F401


def build():
    from .build import build as _build
    return _build()
