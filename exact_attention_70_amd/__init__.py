"""libfa: exact scaled-dot-product attention for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI shared library ``libfa.so`` (hand-written HIP
kernels) declared in ``include/fa.h``; this package only loads it and
marshals arguments.  Build with ``python -m exact_attention_70_amd.build``.
"""
from .binding import (FA_DT_BF16, FA_DT_F16, FA_DT_F32, LibfaError, bwd, bwd_workspace_size, fwd,  # noqa: F401
                    fwd_offset, load_library, merge, paged_decode, paged_decode_workspace_size,
                    paged_kv_append, paged_prefill, status_string)

__all__ = ["fwd", "fwd_offset", "merge", "bwd", "paged_decode", "paged_kv_append", "paged_prefill",
           "bwd_workspace_size",
           "paged_decode_workspace_size", "load_library", "status_string", "LibfaError",
           "FA_DT_BF16", "FA_DT_F16", "FA_DT_F32"]
