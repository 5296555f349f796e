"""MassAlloc Attention (MALA) for AMD MI355X (gfx950).

The operator lives in libmala.so (hand-written HIP kernels behind a C ABI,
``include/mala.h``); ``contribution_gated_sparse_amd.mala`` is its thin ctypes
binding. Importing this package does not load the library; the first call
does, and fails loudly if it has not been built.
"""
from .mala import (MalaError, mala_bwd, mala_decode, mala_fwd, mala_get_tiling,  # noqa: F401
                   load_library, version)
from .autograd import MalaAttentionFunction, mala_attention  # noqa: F401
