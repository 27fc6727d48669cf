"""torch operators over the C ABI: the attention forward with its backward
attached, for training.

"4.4 Writing GPU Kernels with Triton" wires its kernels into autograd with
an ``autograd.Function`` that saves (q, k, v, O, L) in the forward and calls
the backward kernel with them (section "Wiring it into torch.autograd"). It
then recommends registering a custom operator so that the op is visible to
torch.compile and torch.export (section on custom operators). Here both
directions are ``torch.library`` custom ops:

  io_aware_attention_flash::fwd(q, k, v, causal, scale) -> (o, lse)
  io_aware_attention_flash::bwd(q, k, v, o, lse, do, causal, scale) -> (dq, dk, dv)

with fake (meta) implementations for shape inference and the backward
registered as fwd's autograd formula. ``flash_attn_func`` is the user-facing
call. O is kept in the input dtype (as the page's forward returns it) and the
backward's D = rowsum(dO * O) is formed from it. LSE is an auxiliary output
without a gradient. All compute runs in the HIP library; these wrappers only
marshal tensors.
"""
import torch

from . import binding

_NS = "io_aware_attention_flash"


def _usable(x):
    """x itself when the kernels can read it in place (unit last stride, rows
    16-byte aligned), else a contiguous copy."""
    e = x.element_size()
    if x.stride(-1) == 1 and x.data_ptr() % 16 == 0 and all((st * e) % 16 == 0
                                                            for st in x.stride()[:-1]):
        return x
    return x.contiguous()


@torch.library.custom_op(_NS + "::fwd", mutates_args=())
def _fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool,
         scale: float) -> tuple[torch.Tensor, torch.Tensor]:
    o, lse = binding.attn_fwd(_usable(q), _usable(k), _usable(v), causal=causal, scale=scale)
    return o, lse


@_fwd.register_fake
def _fwd_fake(q, k, v, causal, scale):
    # The real op returns fresh contiguous tensors whatever the input strides
    # (empty_like would copy the strides of a transposed view).
    return q.new_empty(q.shape), q.new_empty(q.shape[:3], dtype=torch.float32)


@torch.library.custom_op(_NS + "::bwd", mutates_args=())
def _bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
         dout: torch.Tensor, causal: bool,
         scale: float) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    return tuple(binding.attn_bwd(_usable(q), _usable(k), _usable(v), _usable(o), lse.contiguous(),
                                  _usable(dout), causal=causal, scale=scale))


@_bwd.register_fake
def _bwd_fake(q, k, v, o, lse, dout, causal, scale):
    return q.new_empty(q.shape), k.new_empty(k.shape), v.new_empty(v.shape)


def _setup_context(ctx, inputs, output):
    q, k, v, causal, scale = inputs
    o, lse = output
    ctx.save_for_backward(q, k, v, o, lse)
    ctx.causal = causal
    ctx.scale = scale
    ctx.mark_non_differentiable(lse)


def _backward(ctx, do, dlse):
    q, k, v, o, lse = ctx.saved_tensors
    dq, dk, dv = _bwd(q, k, v, o, lse, do, ctx.causal, ctx.scale)
    return dq, dk, dv, None, None


_fwd.register_autograd(_backward, setup_context=_setup_context)


def flash_attn_func(q, k, v, causal=False, scale=None):
    """softmax(scale q k^T [+ causal mask]) v for [B, H, N, d] bf16, fp16 or
    fp32 tensors on the GPU, differentiable in q, k and v. scale defaults to
    1/sqrt(d)."""
    if scale is None:
        scale = 1.0 / q.shape[-1] ** 0.5
    o, _ = torch.ops.io_aware_attention_flash.fwd(q, k, v, bool(causal), float(scale))
    return o
