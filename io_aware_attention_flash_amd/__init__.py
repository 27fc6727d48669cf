"""MI355X (gfx950) FlashAttention forward and backward: a C-ABI HIP library
and its binding.

The compute lives in ``libattn_fwd.so`` (hand-written HIP kernels behind the
C functions declared in ``include/attn.h``). ``attn_fwd`` and ``attn_bwd``
only marshal torch tensors into those C calls; they raise if the library is
missing. ``flash_attn_func`` is the differentiable torch operator over both
(``ops.py``). Importing this package loads nothing; the library is opened on
first use.
"""


def attn_fwd(*args, **kwargs):
    from .binding import attn_fwd as _f
    return _f(*args, **kwargs)


def attn_bwd(*args, **kwargs):
    from .binding import attn_bwd as _f
    return _f(*args, **kwargs)


def flash_attn_func(*args, **kwargs):
    from .ops import flash_attn_func as _f
    return _f(*args, **kwargs)


__all__ = ["attn_fwd", "attn_bwd", "flash_attn_func"]
