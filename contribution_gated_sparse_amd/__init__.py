"""MassAlloc Attention (MALA) for AMD MI355X (gfx950).

The operator lives in libmala.so (hand-written HIP kernels behind a C ABI,
``include/mala.h``); ``contribution_gated_sparse_amd.mala`` is its thin ctypes
binding. Importing this package does not load the library; the first call
does, and fails loudly if it has not been built.
"""
from .mala import (DECODE_SPLIT_AUTO, MalaError, decode_split_keys, mala_bwd,  # noqa: F401
                   mala_decode, mala_fwd, mala_get_tiling, load_library, make_decode_problem,
                   version)
from .autograd import MalaAttentionFunction, mala_attention  # noqa: F401
