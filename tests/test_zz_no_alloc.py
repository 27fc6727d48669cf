"""The allocation-free backward (attn_bwd_noalloc) against attn_bwd_qk.

attn_bwd_noalloc keeps the per-row (L log2 e, D) values in the library's
static device scratch instead of a caller's workspace and runs the same
kernels, so its gradients must equal attn_bwd_qk's bit for bit (stronger
than the parity bar). Two calls run in a row, the second on a smaller
problem, so the second reads the scratch after the first left its rows
there; a third case is cross-attention."""
import pytest
import torch

from io_aware_attention_flash_amd import binding
from io_aware_attention_flash_amd import build as hipbuild
from io_aware_attention_flash_amd.inputs import make_dout, make_qkv

pytestmark = pytest.mark.gpu

DT = {"bf16": (torch.bfloat16, binding.ATTN_BF16), "f16": (torch.float16, binding.ATTN_F16)}


def setup_module(module):
    hipbuild.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _problem(B, H, Nq, Nk, d, dt, causal, seed):
    tdt, _ = DT[dt]
    dev = torch.device("cuda:0")
    q, _, _ = make_qkv(B, H, Nq, d, dt, 1.0, seed=seed)
    _, k, v = make_qkv(B, H, Nk, d, dt, 1.0, seed=seed + 1)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    dout = make_dout(B, H, Nq, d, dt, seed=seed).to(dev)
    scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    o, lse = binding.attn_fwd(q, k, v, causal=causal, scale=scale, out_dtype=torch.float32)
    return q, k, v, o, lse, dout, scale


def _grads(shape_q, shape_k, dev):
    return [torch.full(s, float("nan"), dtype=torch.float32, device=dev)
            for s in (shape_q, shape_k, shape_k)]


def _run_both(case):
    B, H, Nq, Nk, d, dt, causal, seed = case
    print("no-alloc case", case, flush=True)
    q, k, v, o, lse, dout, scale = _problem(B, H, Nq, Nk, d, dt, causal, seed)
    dev = q.device
    stream = torch.cuda.current_stream().cuda_stream
    in_t = DT[dt][1]
    ptrs = [x.data_ptr() for x in (q, k, v, o, lse, dout)]
    want = _grads(q.shape, k.shape, dev)
    ws_bytes = binding.bwd_workspace_bytes(B, H, Nq, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = binding.attn_bwd_qk_raw(*ptrs, *[g.data_ptr() for g in want], B, H, Nq, Nk, d, causal,
                                 scale, in_t, binding.ATTN_F32, binding.ATTN_F32, ws.data_ptr(),
                                 ws_bytes, stream)
    assert st == 0, binding.status_string(st)
    got = _grads(q.shape, k.shape, dev)
    st = binding.attn_bwd_noalloc_raw(*ptrs, *[g.data_ptr() for g in got], B, H, Nq, Nk, d, causal,
                                      scale, in_t, binding.ATTN_F32, binding.ATTN_F32, stream)
    assert st == 0, binding.status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        assert torch.isfinite(b).all(), name
        assert torch.equal(a, b), "%s: max diff %.3e" % (name, float((a - b).abs().max()))


def test_two_calls_in_a_row_second_smaller():
    # (B, H, Nq, Nk, d, dtype, causal, seed)
    _run_both((2, 8, 1000, 1000, 128, "bf16", True, 51))
    _run_both((1, 3, 200, 200, 64, "f16", False, 52))


def test_cross_attention():
    _run_both((2, 2, 300, 517, 64, "bf16", False, 53))
