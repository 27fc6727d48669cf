"""bf16 V of any finite magnitude against the fp64 oracle.

The P.V product runs in fp16 for bf16 inputs (fp16 P, V converted to fp16).
bf16 covers magnitudes far outside fp16's range, so two cases need care:
  - |v| > 65504 becomes +-inf in fp16. The kernels detect the non-finite
    accumulator and recompute the affected rows with bf16 P against the
    given V (the page's own precision for P). Scaling V by c scales O by c,
    so the parity bar is applied relative to max|V|: max |err| <= 1e-2 max|V|
    and mean |err| <= 1e-3 max|V|; LSE does not depend on V (1e-3).
  - |v| < 2^-14 falls in fp16's subnormal range, where the conversion rounds
    to a multiple of 2^-24. The weights of a row are non-negative and sum to
    one, so each output element moves by at most the largest such rounding
    in its column: the bar adds max_j |fp16(v_jc) - v_jc| per column.
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_flash_amd import binding
from io_aware_attention_flash_amd import build as hipbuild
from io_aware_attention_flash_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu


def setup_module(module):
    hipbuild.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _scale(d):
    return float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))


def _check(q, k, v, causal, scale, o, lse, what):
    ref_o, ref_l = oracle.attn_oracle(q, k, v, causal=causal, scale=scale)
    o = o.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    vmax = float(v.double().abs().max())
    # largest fp16 rounding of V per (head, column), for the subnormal range
    rnd = (v.to(torch.float16).double() - v.double()).abs()
    rnd = torch.where(torch.isinf(rnd), torch.zeros_like(rnd), rnd)
    col = rnd.amax(dim=2, keepdim=True).numpy()
    err = np.abs(o - ref_o)
    lerr = np.abs(lse - ref_l)
    print("%s: max|V| %.3g | O max %.3e mean %.3e (relative to max|V|: %.3e / %.3e) | LSE max %.3e"
          % (what, vmax, err.max(), err.mean(), err.max() / vmax, err.mean() / vmax, lerr.max()),
          flush=True)
    assert np.all(np.isfinite(o)), what + ": non-finite output"
    assert np.all(err <= 1e-2 * vmax + col), "%s: O max err %.3e" % (what, err.max())
    assert err.mean() <= 1e-3 * vmax + col.mean(), "%s: O mean err %.3e" % (what, err.mean())
    assert lerr.max() <= 1e-3, "%s: LSE max err %.3e" % (what, lerr.max())


CASES = [
    # (B, H, N, d, causal, V scale): overflow in fp16 (1e5, 1e30), subnormal (1e-6)
    (1, 2, 300, 128, True, 1e5),
    (1, 2, 300, 128, False, 1e30),
    (2, 1, 257, 64, True, 1e5),
    (1, 2, 200, 64, False, 1e30),
    (1, 2, 300, 128, True, 1e-6),
    (1, 2, 333, 64, False, 1e-6),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dN%dd%d_%s_v%g" % (
    c[0], c[1], c[2], c[3], "causal" if c[4] else "full", c[5]))
def test_v_magnitude_tuned(case):
    B, H, N, d, causal, vs = case
    print("case", case, flush=True)
    q, k, v = make_qkv(B, H, N, d, "bf16", 1.0, seed=41)
    v = (v.float() * vs).to(torch.bfloat16)
    sc = _scale(d)
    o, lse = binding.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=sc,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(q, k, v, causal, sc, o, lse, "tuned %s" % (case,))


def test_one_large_value_in_one_head():
    """A single V element beyond fp16's range: only the waves that meet it
    take the bf16 recomputation; every other row keeps the fp16 path's bits."""
    B, H, N, d = 1, 3, 600, 128
    q, k, v = make_qkv(B, H, N, d, "bf16", 1.0, seed=42)
    sc = _scale(d)
    base_o, base_l = binding.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=sc,
                                      out_dtype=torch.float32)
    v2 = v.clone()
    v2[0, 1, 300, 7] = 3.0e5
    o, lse = binding.attn_fwd(q.cuda(), k.cuda(), v2.cuda(), causal=True, scale=sc,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(q, k, v2, True, sc, o, lse, "one large value")
    # heads 0 and 2, and head 1's rows before key 300 (their waves end below it), unchanged
    assert torch.equal(o[:, 0], base_o[:, 0]) and torch.equal(o[:, 2], base_o[:, 2])
    assert torch.equal(o[0, 1, :256], base_o[0, 1, :256])
    assert torch.equal(lse, base_l)


def test_v_magnitude_first_pass():
    """Long bf16 sequences convert V in a first pass into the workspace; an
    overflowing V still takes the recomputation from the given V."""
    B, H, N, d = 1, 1, 8192, 128
    q, k, v = make_qkv(B, H, N, d, "bf16", 1.0, seed=43)
    v = (v.float() * 1e6).to(torch.bfloat16)
    sc = _scale(d)
    assert binding.workspace_bytes(B, H, N, d, binding.ATTN_BF16) > 0
    o, lse = binding.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=sc,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(q, k, v, True, sc, o, lse, "first pass, V x 1e6")


@pytest.mark.parametrize("d,vs", [(96, 1e5), (40, 1e30), (128, 1e-6)])
def test_v_magnitude_general(d, vs):
    """The general-layout kernel (strided [B, N, H, d] views, padded head dims)."""
    B, H, N = 1, 2, 190
    q, k, v = make_qkv(B, H, N, d, "bf16", 1.0, seed=44)
    v = (v.float() * vs).to(torch.bfloat16)
    sc = _scale(d)
    qs, ks_, vs_ = (x.cuda().transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    o, lse = binding.attn_fwd_general(qs, ks_, vs_, causal=True, scale=sc, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(q, k, v, True, sc, o, lse, "general d=%d V x %g" % (d, vs))
