"""The differentiable operator (flash_attn_func) on the GPU: forward output
and the gradients autograd produces through the registered backward, against
the fp64 oracles. O and the gradients are in the input dtype here, so the
tolerances are those of the input-dtype checks: the forward's 1e-2 plus half
an ulp of the output, and the backward's rounding bound with the input-type O
and gradient roundings added (see test_bwd_gpu.py)."""
import os

import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_flash_amd import binding
from io_aware_attention_flash_amd import build as hipbuild
from io_aware_attention_flash_amd.inputs import make_dout, make_qkv
from io_aware_attention_flash_amd.ops import flash_attn_func
from test_bwd_gpu import U, _terms, check_grads

pytestmark = pytest.mark.gpu


def setup_module(module):
    hipbuild.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


@pytest.mark.parametrize("B,H,N,d,dt,causal", [
    (2, 4, 256, 64, "f16", False), (2, 4, 256, 64, "f16", True),
    (1, 3, 200, 128, "bf16", True), (1, 2, 129, 128, "bf16", False),
    # head dims the forward's general kernel and the padded backward take
    (1, 2, 150, 96, "bf16", True), (2, 2, 100, 40, "f16", False),
])
def test_autograd_matches_oracles(B, H, N, d, dt, causal):
    print("case", B, H, N, d, dt, causal, flush=True)
    q, k, v = make_qkv(B, H, N, d, dt, 1.0, seed=21)
    dout = make_dout(B, H, N, d, dt, seed=21)
    scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    dev = torch.device("cuda:0")
    qg, kg, vg = (x.to(dev).requires_grad_() for x in (q, k, v))
    o = flash_attn_func(qg, kg, vg, causal=causal, scale=scale)
    o.backward(dout.to(dev))
    torch.cuda.synchronize()
    ro, rl = oracle.attn_oracle(q, k, v, causal=causal, scale=scale)
    ulp = np.abs(ro) * U[dt] + 1e-30
    err = np.abs(o.detach().cpu().double().numpy() - ro)
    assert np.all(err <= 1e-2 + 0.5 * ulp + 2 ** -24), "forward O"
    ref = oracle.attn_bwd_oracle(q, k, v, dout, causal=causal, scale=scale)
    # D is formed from the forward's input-dtype O: its error is at most
    # sum_c |dO_ic| (1e-2 + half an ulp of O_ic) by the forward's tolerance.
    dD = (dout.double().abs() * (1e-2 + 0.5 * torch.from_numpy(ulp))).sum(-1)
    dL = torch.full((B, H, N), 1e-3, dtype=torch.float64)
    terms, extra = _terms(q, k, v, dout, causal, scale, dD=dD, dL=dL)
    got = [x.grad.float().cpu() for x in (qg, kg, vg)]
    check_grads(got, ref, terms, extra, U[dt], "autograd", grad_rounding=U[dt])


def test_autograd_cross_attention():
    """Queries and keys of different lengths through the operator: the
    forward takes the general-layout kernel, the backward attn_bwd_qk."""
    B, H, Nq, Nk, d, dt = 2, 2, 150, 333, 128, "bf16"
    q = make_qkv(B, H, Nq, d, dt, 1.0, seed=23)[0]
    _, k, v = make_qkv(B, H, Nk, d, dt, 1.0, seed=24)
    dout = make_dout(B, H, Nq, d, dt, seed=23)
    scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    dev = torch.device("cuda:0")
    qg, kg, vg = (x.to(dev).requires_grad_() for x in (q, k, v))
    o = flash_attn_func(qg, kg, vg, causal=False, scale=scale)
    o.backward(dout.to(dev))
    torch.cuda.synchronize()
    ro, _ = oracle.attn_oracle(q, k, v, causal=False, scale=scale)
    ulp = np.abs(ro) * U[dt] + 1e-30
    assert np.all(np.abs(o.detach().cpu().double().numpy() - ro) <= 1e-2 + 0.5 * ulp + 2 ** -24)
    ref = oracle.attn_bwd_oracle(q, k, v, dout, causal=False, scale=scale)
    dD = (dout.double().abs() * (1e-2 + 0.5 * torch.from_numpy(ulp))).sum(-1)
    dL = torch.full((B, H, Nq), 1e-3, dtype=torch.float64)
    terms, extra = _terms(q, k, v, dout, False, scale, dD=dD, dL=dL)
    got = [x.grad.float().cpu() for x in (qg, kg, vg)]
    check_grads(got, ref, terms, extra, U[dt], "autograd cross", grad_rounding=U[dt])


def test_opcheck():
    """torch's operator checks: schema, fake tensors, autograd registration."""
    q, k, v = (x.cuda() for x in make_qkv(1, 2, 64, 64, "bf16", 1.0, seed=22))
    torch.library.opcheck(torch.ops.io_aware_attention_flash.fwd.default, (q, k, v, True, 0.125),
                          test_utils=("test_schema", "test_faketensor",
                                      "test_autograd_registration"))


def test_opcheck_transposed_views():
    """The same checks on [B, N, H, d] tensors seen as [B, H, N, d]: the fake
    outputs must carry the real outputs' (contiguous) strides."""
    q, k, v = (x.cuda().transpose(1, 2).contiguous().transpose(1, 2)
               for x in make_qkv(1, 2, 64, 64, "bf16", 1.0, seed=23))
    assert not q.is_contiguous()
    torch.library.opcheck(torch.ops.io_aware_attention_flash.fwd.default, (q, k, v, False, 0.125),
                          test_utils=("test_schema", "test_faketensor",
                                      "test_autograd_registration"))
    o, lse = torch.ops.io_aware_attention_flash.fwd(q, k, v, False, 0.125)
    dout = torch.randn_like(o)
    torch.library.opcheck(torch.ops.io_aware_attention_flash.bwd.default,
                          (q, k, v, o, lse, dout, False, 0.125),
                          test_utils=("test_schema", "test_faketensor"))


def test_training_step_runs():
    """A tiny attention layer trains through the operator: finite gradients
    on every parameter and a loss that falls over a few SGD steps on a fixed
    batch."""
    torch.manual_seed(0)
    dev = torch.device("cuda:0")
    B, H, N, d = 2, 4, 128, 64
    proj = torch.nn.Linear(H * d, 3 * H * d).to(dev).to(torch.bfloat16)
    x = torch.randn(B, N, H * d, device=dev, dtype=torch.bfloat16)
    target = torch.randn(B, H, N, d, device=dev, dtype=torch.bfloat16)
    opt = torch.optim.SGD(proj.parameters(), lr=0.5)
    losses = []
    for _ in range(5):
        qkv = proj(x).view(B, N, 3, H, d).permute(2, 0, 3, 1, 4)
        o = flash_attn_func(qkv[0], qkv[1], qkv[2], causal=True)
        loss = (o.float() - target.float()).pow(2).mean()
        opt.zero_grad()
        loss.backward()
        assert all(torch.isfinite(p.grad).all() for p in proj.parameters())
        opt.step()
        losses.append(loss.item())
    print("losses", losses, flush=True)
    assert losses[-1] < losses[0]


def test_torch_compile_fullgraph():
    """torch.compile(fullgraph=True) over the operator and its registered
    backward (aot_eager backend: the graph is traced through the fake
    implementations and replayed with the real ones, no code generation):
    the same output and gradients as eager, bit for bit."""
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in make_qkv(1, 4, 300, 128, "bf16", 1.0, seed=71))

    def step(q, k, v):
        o = flash_attn_func(q, k, v, causal=True)
        return (o.float() * o.float()).sum()

    compiled = torch.compile(step, fullgraph=True, backend="aot_eager")
    grads = []
    for fn in (step, compiled):
        qq, kk, vv = (x.clone().requires_grad_() for x in (q, k, v))
        loss = fn(qq, kk, vv)
        loss.backward()
        torch.cuda.synchronize()
        grads.append((loss.detach(), qq.grad, kk.grad, vv.grad))
    for a, b in zip(*grads):
        assert torch.equal(a, b)
