"""The torch operators (ops.py) on a host without a GPU: they register under
their namespace and their fake implementations give the right shapes, so
torch's tracing can see through them."""
import torch
from torch._subclasses.fake_tensor import FakeTensorMode

import io_aware_attention_flash_amd as pkg
from io_aware_attention_flash_amd import ops  # noqa: F401  (registers the ops)


def test_ops_are_registered():
    assert hasattr(torch.ops.io_aware_attention_flash, "fwd")
    assert hasattr(torch.ops.io_aware_attention_flash, "bwd")
    assert callable(pkg.flash_attn_func)


def test_fake_shapes():
    with FakeTensorMode():
        q = torch.empty(2, 3, 17, 64, dtype=torch.bfloat16)
        o, lse = torch.ops.io_aware_attention_flash.fwd(q, q, q, True, 0.125)
        assert o.shape == q.shape and o.dtype == q.dtype
        assert lse.shape == (2, 3, 17) and lse.dtype == torch.float32
        dq, dk, dv = torch.ops.io_aware_attention_flash.bwd(q, q, q, o, lse, q, True, 0.125)
        assert dq.shape == dk.shape == dv.shape == q.shape


def test_fake_outputs_are_contiguous_for_strided_inputs():
    """The real ops return fresh contiguous tensors, so the fakes must too:
    a [B, N, H, d] tensor seen as [B, H, N, d] (a transposed view) must not
    hand its strides to the outputs."""
    with FakeTensorMode():
        x = torch.empty(2, 17, 3, 64, dtype=torch.bfloat16)
        q = x.transpose(1, 2)
        assert not q.is_contiguous()
        o, lse = torch.ops.io_aware_attention_flash.fwd(q, q, q, False, 0.125)
        assert o.is_contiguous() and o.stride() == (3264, 1088, 64, 1)
        assert lse.is_contiguous()
        grads = torch.ops.io_aware_attention_flash.bwd(q, q, q, o, lse, q, False, 0.125)
        for g in grads:
            assert g.shape == q.shape and g.is_contiguous()


def test_export_sees_the_operator():
    """torch.export traces a module that calls flash_attn_func into a graph
    holding the registered operator (the fake implementation gives the shapes;
    nothing runs on a GPU)."""
    class Attn(torch.nn.Module):
        def forward(self, q, k, v):
            return pkg.flash_attn_func(q, k, v, causal=True)

    q = torch.randn(1, 2, 16, 64, dtype=torch.bfloat16)
    ep = torch.export.export(Attn(), (q, q, q))
    targets = [str(n.target) for n in ep.graph.nodes if n.op == "call_function"]
    assert any("io_aware_attention_flash.fwd" in t for t in targets), targets
    out = [n for n in ep.graph.nodes if n.op == "output"][0]
    assert out is not None
