"""MI355X-native AFD expert-parallel dispatch/combine on one GPU.

The path is a C-ABI library (``include/afd.h``) of hand-written gfx950 HIP
kernels; ``Buffer`` is its thin Python binding.  Importing this package does
not load the library; creating a Buffer does, and fails loudly when it has
not been built (``python -m combine_layout_amd.build``).
"""
from .buffer import Buffer, Received, topk_idx_dtype  # noqa: F401
from ._native import AfdError  # noqa: F401
