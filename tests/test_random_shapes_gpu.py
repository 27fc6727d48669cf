"""Randomised parity: seeded draws of problem shapes, layouts and dtypes for
the forward (contiguous, [B, N, H, d] views, cross-attention, K/V heads
shared through stride-0 views) and the backward (contiguous and [B, N, H, d]
views), each against the fp64 oracles with the tolerances of the targeted
tests. The draws come from a fixed seed, so every run checks the same cases;
the case id names each one."""
import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_flash_amd import binding
from io_aware_attention_flash_amd import build as hipbuild
from io_aware_attention_flash_amd.inputs import make_dout, make_qkv
from test_bwd_gpu import U, _terms, check_grads

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3
DEV = torch.device("cuda:0")
KINDS = ["fwd", "fwd_bnhd", "fwd_cross", "fwd_shared_kv", "bwd", "bwd_bnhd"]
HEAD_DIMS = [8, 16, 24, 32, 40, 48, 56, 64, 72, 80, 96, 112, 128]


def _draw(n, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kind = KINDS[i % len(KINDS)]  # every kind equally often
        dt = str(rng.choice(["bf16", "f16", "f32"]))
        d = int(rng.choice(HEAD_DIMS))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        if kind == "fwd_shared_kv":
            H = 2 * H
        N = int(round(np.exp(rng.uniform(0.0, np.log(1500.0)))))
        Nk = int(round(np.exp(rng.uniform(0.0, np.log(1500.0))))) if kind == "fwd_cross" else N
        causal = kind != "fwd_cross" and bool(rng.integers(0, 2))
        cases.append((i, kind, dt, B, H, N, Nk, d, causal))
    return cases


CASES = _draw(96)


def setup_module(module):
    hipbuild.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _scale(d):
    return float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))


def _bnhd(x):
    """The same values as a [B, H, N, d] view of a [B, N, H, d] tensor."""
    return x.to(DEV).transpose(1, 2).contiguous().transpose(1, 2)


def _check_fwd(o, lse, q, k, v, causal, scale, what):
    ro, rl = oracle.attn_oracle(q, k, v, causal=causal, scale=scale)
    err = np.abs(o.cpu().double().numpy() - ro)
    lerr = np.abs(lse.cpu().double().numpy() - rl)
    print("%s: O max %.2e mean %.2e | LSE max %.2e" % (what, err.max(), err.mean(), lerr.max()),
          flush=True)
    assert np.all(np.isfinite(err)) and np.all(np.isfinite(lerr)), what
    assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr.max() <= LSE_MAX, what


def _id(c):
    i, kind, dt, B, H, N, Nk, d, causal = c
    return "%02d_%s_%s_B%dH%dN%dNk%dd%d_%s" % (i, kind, dt, B, H, N, Nk, d,
                                                 "causal" if causal else "full")


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_random_case(case):
    i, kind, dt, B, H, N, Nk, d, causal = case
    print("case", _id(case), flush=True)
    scale = _scale(d)
    if kind == "fwd_cross":
        q = make_qkv(B, H, N, d, dt, 1.0, seed=100 + i)[0]
        _, k, v = make_qkv(B, H, Nk, d, dt, 1.0, seed=200 + i)
    elif kind == "fwd_shared_kv":
        Hkv = 1 if (i // len(KINDS)) % 2 == 0 else H // 2  # multi-query, or pairs of query heads
        G = H // Hkv
        q = make_qkv(B, H, N, d, dt, 1.0, seed=100 + i)[0]
        _, kk, vv = make_qkv(B, Hkv, N, d, dt, 1.0, seed=200 + i)
        q4 = q.to(DEV).view(B * Hkv, G, N, d)
        k4, v4 = (x.to(DEV).reshape(B * Hkv, 1, N, d).expand(B * Hkv, G, N, d) for x in (kk, vv))
        o, lse = binding.attn_fwd(q4, k4, v4, causal=causal, scale=scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        k, v = (x.repeat_interleave(G, dim=1) for x in (kk, vv))
        _check_fwd(o.view(B, H, N, d), lse.view(B, H, N), q, k, v, causal, scale, _id(case))
        return
    else:
        q, k, v = make_qkv(B, H, N, d, dt, 1.0, seed=100 + i)
    if kind.startswith("fwd"):
        if kind == "fwd_bnhd":
            qd, kd, vd = (_bnhd(x) for x in (q, k, v))
        else:
            qd, kd, vd = (x.to(DEV) for x in (q, k, v))
        o, lse = binding.attn_fwd(qd, kd, vd, causal=causal, scale=scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _check_fwd(o, lse, q, k, v, causal, scale, _id(case))
        return
    # backward, after the GPU forward (the tolerance adds that forward's measured errors)
    dout = make_dout(B, H, N, d, dt, seed=100 + i)
    view = _bnhd if kind == "bwd_bnhd" else (lambda x: x.to(DEV))
    qd, kd, vd, dd = (view(x) for x in (q, k, v, dout))
    o, lse = binding.attn_fwd(qd, kd, vd, causal=causal, scale=scale, out_dtype=torch.float32)
    got = binding.attn_bwd(qd, kd, vd, o, lse, dd, causal=causal, scale=scale,
                           grad_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_oracle(q, k, v, causal=causal, scale=scale)
    dD = (dout.double() * (o.cpu().double() - torch.from_numpy(ro))).sum(-1)
    dL = lse.cpu().double() - torch.from_numpy(rl)
    ref = oracle.attn_bwd_oracle(q, k, v, dout, causal=causal, scale=scale)
    terms, extra = _terms(q, k, v, dout, causal, scale, dD=dD, dL=dL)
    check_grads([g.cpu() for g in got], ref, terms, extra, U[dt], _id(case))
