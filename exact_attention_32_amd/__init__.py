"""MI355X (gfx950) exact attention forward and backward pass.

O = softmax(scale * Q K^T [+ causal mask]) V and the per-row log-sum-exp,
and the gradients dQ, dK, dV, computed tile by tile in hand-written HIP
kernels behind the C ABI of ``include/fa.h``.  This package is the thin Python
binding of that library (``fa_fwd``, ``fa_fwd_ex``, ``fa_fwd_f32``, ``fa_fwd_kv_outer``,
``fa_bwd``, ``fa_bwd_ex``, ``fa_decode``, ``fa_decode_ex``, ``fa_decode_noalloc`` and the
workspace-size queries, ``fa_strerror``,
with the C names, plus the torch conveniences ``forward``,
``forward_kv_outer``, ``backward`` and ``decode``) and the seeded input
generators in ``inputs``.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    FA_ERR_ALIAS,
    FA_ERR_ALIGN,
    FA_ERR_HEADDIM,
    FA_ERR_HIP,
    FA_ERR_NULL,
    FA_ERR_SCALE,
    FA_DTYPE_BF16,
    FA_DTYPE_FP16,
    FA_ERR_DTYPE,
    FA_ERR_SHAPE,
    FA_ERR_STRIDE,
    FA_ERR_SCRATCH,
    FA_ERR_WORKSPACE,
    FA_DECODE_SCRATCH_BYTES,
    FA_OK,
    LIB_PATH,
    FAError,
    backward,
    decode,
    fa_bwd,
    fa_bwd_ex,
    fa_decode,
    fa_decode_ex,
    fa_decode_noalloc,
    fa_decode_workspace_size,
    fa_fwd,
    fa_fwd_ex,
    fa_fwd_f32,
    fa_fwd_kv_outer,
    fa_fwd_kv_outer_workspace_size,
    fa_strerror,
    forward,
    forward_kv_outer,
    load_library,
)
