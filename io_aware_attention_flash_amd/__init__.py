"""MI355X (gfx950) FlashAttention forward: a C-ABI HIP library and its binding.

The compute lives in ``libattn_fwd.so`` (hand-written HIP kernels behind the
C functions declared in ``include/attn.h``). ``attn_fwd`` below only
marshals torch tensors into that C call; it raises if the library is missing.
Importing this package loads nothing; the library is opened on first use.
"""


def attn_fwd(*args, **kwargs):
    from .binding import attn_fwd as _f
    return _f(*args, **kwargs)


__all__ = ["attn_fwd"]
