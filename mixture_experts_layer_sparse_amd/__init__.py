"""Sparse Mixture-of-Experts layer forward for AMD MI355X (gfx950).

The compute path is the HIP library ``libmoe.so`` (C ABI in include/moe.h);
``moe`` is its Python binding.  Build with
``python -m mixture_experts_layer_sparse_amd.build``.
"""
from . import moe  # noqa: F401
from .moe import Layer, Shape, make_shape, shape_of  # noqa: F401
