"""GPU parity of the backward (attn_bwd): the HIP path against the fp64
backward oracle on the same seeded inputs.

Tolerance, derived from the arithmetic. The kernels round P and dS once to
the operand type before each matrix product (unit roundoff u = 2^-8 for
bf16, 2^-11 for fp16) and accumulate in fp32. An element G = sum_t x_t y_t
of dQ, dK or dV therefore differs from the exact sum by at most about
u * T, where T = sum_t |x_t y_t| is the sum of the magnitudes of its terms:
  dV_jc : T = sum_i P_ij |dO_ic|
  dK_jc : T = scale sum_i |dS_ij| |q_ic|
  dQ_ic : T = scale sum_j |dS_ij| |k_jc|
T is computed in fp64 on the CPU. The test allows
  |err| <= 2 u T + 1e-5 max|G_ref| + 1e-6.
The factor 2 covers fp32 rounding and second-order terms. dP - D, a
difference of two fp32 sums of d products, gets its own allowance of
d 2^-22 times their magnitudes, and the floor covers elements whose exact
value is 0. The relative RMS error must also be at most
u. When the gradients are stored in the input type, u |G_ref| is added for
the final rounding.

The primary cases give the backward the oracle's O and LSE rounded to fp32,
so they measure the backward alone. The end-to-end cases use the GPU
forward's O and LSE, and add the first-order effect of that forward's
measured error: an error dO_i . dO_err in D_i, or dL_i in LSE_i, moves dS_ij
by P_ij dD_i or dS_ij dL_i.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_flash_amd import binding
from io_aware_attention_flash_amd import build as hipbuild
from io_aware_attention_flash_amd.inputs import WORKLOADS, make_dout, make_qkv

pytestmark = pytest.mark.gpu

U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11,
     # fp32 inputs round nothing to a narrower type; the unit covers fp32
     # accumulation over up to a few thousand terms and exp2 of scores whose
     # own fp32 error is amplified by their size (|s * scale| up to ~10)
     "f32": 2.0 ** -16}
DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def setup_module(module):
    hipbuild.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _say(*a):
    print(*a, flush=True)


def _scale(d):
    return float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))


def _inputs(B, H, N, d, dt, sigma, seed):
    q, k, v = make_qkv(B, H, N, d, dt, sigma, seed=seed)
    return q, k, v, make_dout(B, H, N, d, dt, seed=seed)


def _terms(q, k, v, dout, causal, scale, dD=None, dL=None):
    """fp64 magnitudes T of the terms of every dQ, dK, dV element (see the
    module docstring), plus the first-order effect of errors dD and dL in the
    backward's D and LSE inputs. Used for the tolerance only."""
    q, k, v, dout = (x.double() for x in (q, k, v, dout))
    N = q.shape[2]
    s = (q @ k.transpose(-2, -1).contiguous()) * scale
    if causal:
        s = s.masked_fill(~torch.tril(torch.ones(N, N, dtype=torch.bool)), float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = p @ v
    dp = dout @ v.transpose(-2, -1).contiguous()
    ds = p * (dp - (dout * o).sum(-1, keepdim=True))
    tq = scale * (ds.abs() @ k.abs())
    tk = scale * (ds.abs().transpose(-2, -1).contiguous() @ q.abs())
    tv = p.transpose(-2, -1).contiguous() @ dout.abs()
    # dP - D is a difference of two fp32 sums of d products each (the matrix
    # core's and the first pass's): allow d * 2^-22 of their magnitudes.
    a = dout.abs() @ v.abs().transpose(-2, -1).contiguous() + \
        (dout.abs() * o.abs()).sum(-1, keepdim=True)
    e32 = p * a * (q.shape[-1] * 2.0 ** -22)
    eq = scale * (e32 @ k.abs())
    ek = scale * (e32.transpose(-2, -1).contiguous() @ q.abs())
    ev = torch.zeros_like(tv)
    if dD is not None:
        dD = dD.double().abs().unsqueeze(-1)
        eq += scale * dD * (p @ k.abs())
        ek += scale * (p.transpose(-2, -1).contiguous() @ (dD * q.abs()))
    if dL is not None:
        dL = dL.double().abs().unsqueeze(-1)
        eq += scale * dL * (ds.abs() @ k.abs())
        ek += scale * ((ds.abs() * dL).transpose(-2, -1).contiguous() @ q.abs())
        ev += (p * dL).transpose(-2, -1).contiguous() @ dout.abs()
    return [t.numpy() for t in (tq, tk, tv)], [e.numpy() for e in (eq, ek, ev)]


def check_grads(got, ref, terms, extra, u, what, grad_rounding=0.0):
    for name, g, r, t, e in zip(("dQ", "dK", "dV"), got, ref, terms, extra):
        g = np.asarray(g, dtype=np.float64)
        assert np.all(np.isfinite(g)), "%s %s: non-finite" % (what, name)
        err = np.abs(g - r)
        tol = 2.0 * u * t + 1.5 * e + grad_rounding * np.abs(r) + 1e-5 * np.abs(r).max() + 1e-6
        worst = float((err / tol).max())
        rms = float(np.sqrt((err ** 2).mean()) / max(np.sqrt((r ** 2).mean()), 1e-30))
        _say("%s %s: max|err| %.2e (max|ref| %.2e) worst err/tol %.3f rel rms %.2e" %
             (what, name, err.max(), np.abs(r).max(), worst, rms))
        assert worst <= 1.0, "%s %s: error %.3f times the tolerance" % (what, name, worst)
        assert rms <= u or np.abs(r).max() == 0.0, "%s %s: relative rms %.2e > u" % (what, name, rms)


def gpu_bwd(q, k, v, o, lse, dout, causal, scale, grad_dtype=torch.float32):
    dev = torch.device("cuda:0")
    dq, dk, dv = binding.attn_bwd(q.to(dev), k.to(dev), v.to(dev), o.to(dev), lse.to(dev),
                                  dout.to(dev), causal=causal, scale=scale, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


# ------------------------------------------------------------- full compare

CASES = [
    # (B, H, N, d, dtype, causal, sigma)
    (2, 4, 256, 64, "f16", False, 1.0),   # the chapter's own backward test shape
    (2, 4, 256, 64, "f16", True, 1.0),
    (1, 2, 1, 64, "bf16", False, 1.0),
    (1, 2, 1, 128, "f16", True, 1.0),
    (1, 2, 31, 128, "bf16", True, 1.0),
    (1, 2, 32, 64, "bf16", True, 1.0),
    (1, 2, 33, 128, "f16", False, 1.0),
    (1, 1, 127, 64, "f16", True, 1.0),
    (1, 2, 128, 128, "bf16", True, 1.0),
    (1, 2, 129, 128, "bf16", False, 1.0),
    (1, 3, 200, 64, "bf16", True, 2.0),
    (2, 1, 255, 128, "f16", True, 1.0),
    (1, 1, 257, 128, "bf16", True, 1.0),
    (3, 5, 97, 128, "bf16", False, 1.0),
    (1, 2, 300, 128, "bf16", True, 1.0),
    (1, 1, 513, 64, "f16", False, 1.0),
    (1, 1, 1000, 128, "bf16", True, 3.0),
    (2, 8, 160, 128, "bf16", True, 1.0),
    (1, 16, 70, 64, "f16", False, 1.0),
]


def _case_id(c):
    return "B%dH%dN%dd%d_%s_%s_s%g" % (c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full",
                                      c[6])


def _oracle_o_lse(q, k, v, causal, scale):
    ro, rl = oracle.attn_oracle(q, k, v, causal=causal, scale=scale)
    return torch.from_numpy(ro).float(), torch.from_numpy(rl).float()


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_bwd_matches_oracle(case):
    """Backward alone: O and LSE are the oracle's, rounded to fp32."""
    B, H, N, d, dt, causal, sigma = case
    _say("case", _case_id(case))
    q, k, v, dout = _inputs(B, H, N, d, dt, sigma, seed=11)
    scale = _scale(d)
    o, lse = _oracle_o_lse(q, k, v, causal, scale)
    got = gpu_bwd(q, k, v, o, lse, dout, causal, scale)
    ref = oracle.attn_bwd_oracle(q, k, v, dout, causal=causal, scale=scale)
    terms, extra = _terms(q, k, v, dout, causal, scale)
    check_grads(got, ref, terms, extra, U[dt], _case_id(case))


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[8], CASES[14], CASES[16]],
                         ids=_case_id)
def test_bwd_end_to_end(case):
    """GPU forward then GPU backward, against the oracle's exact gradients;
    the tolerance adds the first-order effect of the forward's measured
    O and LSE errors."""
    B, H, N, d, dt, causal, sigma = case
    _say("case", _case_id(case))
    q, k, v, dout = _inputs(B, H, N, d, dt, sigma, seed=12)
    scale = _scale(d)
    dev = torch.device("cuda:0")
    o, lse = binding.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale,
                              out_dtype=torch.float32)
    got = gpu_bwd(q, k, v, o, lse, dout, causal, scale)
    ro, rl = oracle.attn_oracle(q, k, v, causal=causal, scale=scale)
    dD = (dout.double() * (o.cpu().double() - torch.from_numpy(ro))).sum(-1)
    dL = lse.cpu().double() - torch.from_numpy(rl)
    ref = oracle.attn_bwd_oracle(q, k, v, dout, causal=causal, scale=scale)
    terms, extra = _terms(q, k, v, dout, causal, scale, dD=dD, dL=dL)
    check_grads(got, ref, terms, extra, U[dt], "end-to-end " + _case_id(case))


@pytest.mark.parametrize("case", [CASES[1], CASES[9], CASES[10]], ids=_case_id)
def test_bwd_input_dtype_o_and_grads(case):
    """O handed over in the input type (rounded, so D moves by up to
    u sum_c |dO_ic O_ic|) and gradients stored in the input type."""
    B, H, N, d, dt, causal, sigma = case
    _say("case", _case_id(case))
    q, k, v, dout = _inputs(B, H, N, d, dt, sigma, seed=13)
    scale = _scale(d)
    o, lse = _oracle_o_lse(q, k, v, causal, scale)
    o_in = o.to(DT[dt])
    got = gpu_bwd(q, k, v, o_in, lse, dout, causal, scale, grad_dtype=DT[dt])
    ref = oracle.attn_bwd_oracle(q, k, v, dout, causal=causal, scale=scale)
    dD = U[dt] * (dout.double().abs() * o.double().abs()).sum(-1)
    terms, extra = _terms(q, k, v, dout, causal, scale, dD=dD)
    check_grads([g.float() for g in got], ref, terms, extra, U[dt], _case_id(case) + " in-dtype",
                grad_rounding=U[dt])


def test_bwd_exercise5_embedded():
    """Exercise 5 ("4.4 Writing GPU Kernels with Triton", section
    "Exercises") differentiated in closed form, embedded at d = 64 in fp16
    (every value exact): q = e0, keys 2 e0 and 4 e0, values e0 and 3 e0,
    scale 1, upstream gradient e0 on the query that sees both keys."""
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "exercise5_online_softmax.json")))
    p1, p2 = g["weights"]
    o_ex = g["O_normalised"]
    d = 64
    q = torch.zeros(1, 1, 2, d, dtype=torch.float16)
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    dout = torch.zeros_like(q)
    q[0, 0, :, 0] = 1.0
    k[0, 0, :, 0] = torch.tensor(g["scores"])
    v[0, 0, :, 0] = torch.tensor(g["values"])
    dout[0, 0, 1, 0] = 1.0
    o, lse = _oracle_o_lse(q, k, v, False, 1.0)
    dq, dk, dv = gpu_bwd(q, k, v, o, lse, dout, False, 1.0)
    (k1, k2), (v1, v2) = g["scores"], g["values"]
    tol = 4 * U["f16"] * 8  # largest term magnitudes here are below 8
    assert abs(dq[0, 0, 1, 0].item() - p1 * p2 * (v2 - v1) * (k2 - k1)) <= tol
    assert abs(dk[0, 0, 0, 0].item() - p1 * (v1 - o_ex)) <= tol
    assert abs(dk[0, 0, 1, 0].item() - p2 * (v2 - o_ex)) <= tol
    assert abs(dv[0, 0, 0, 0].item() - p1) <= tol and abs(dv[0, 0, 1, 0].item() - p2) <= tol
    assert torch.count_nonzero(dq[0, 0, 0]) == 0 and torch.count_nonzero(dq[0, 0, 1, 1:]) == 0


def test_bwd_deterministic():
    """No atomics: two calls give the same bits."""
    q, k, v, dout = _inputs(1, 4, 700, 128, "bf16", 1.0, seed=14)
    scale = _scale(128)
    o, lse = _oracle_o_lse(q, k, v, True, scale)
    a = gpu_bwd(q, k, v, o, lse, dout, True, scale)
    b = gpu_bwd(q, k, v, o, lse, dout, True, scale)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


CROSS = [
    # (B, H, Nq, Nk, d, dtype, sigma): query and key lengths that differ
    (1, 1, 1, 10, 64, "f16", 1.0), (1, 1, 5, 15, 64, "bf16", 1.0),
    (2, 3, 300, 77, 128, "bf16", 1.0), (1, 2, 64, 1000, 64, "f16", 1.0),
    (1, 1, 129, 257, 128, "bf16", 3.0), (1, 2, 700, 33, 128, "f16", 1.0),
]


@pytest.mark.parametrize("case", CROSS, ids=lambda c: "B%dH%dNq%dNk%dd%d_%s_s%g" % c)
def test_bwd_cross_attention(case):
    """attn_bwd_qk with Nq != Nk; O and LSE from the oracle (fp32)."""
    B, H, Nq, Nk, d, dt, sigma = case
    _say("case", case)
    q = make_qkv(B, H, Nq, d, dt, sigma, seed=15)[0]
    _, k, v = make_qkv(B, H, Nk, d, dt, sigma, seed=16)
    dout = make_dout(B, H, Nq, d, dt, seed=15)
    scale = _scale(d)
    o, lse = _oracle_o_lse(q, k, v, False, scale)
    got = gpu_bwd(q, k, v, o, lse, dout, False, scale)
    assert got[0].shape == q.shape and got[1].shape == k.shape and got[2].shape == v.shape
    ref = oracle.attn_bwd_oracle(q, k, v, dout, causal=False, scale=scale)
    terms, extra = _terms(q, k, v, dout, False, scale)
    check_grads(got, ref, terms, extra, U[dt], "cross %s" % (case,))


# ------------------------------------------- head dims reached by padding
ODD_D = [
    # (B, H, Nq, Nk, d, dtype, causal): the kernels run at 64 or 128 columns
    # and read the columns past d as zeros
    (1, 2, 200, 200, 96, "bf16", True),
    (2, 1, 130, 130, 80, "f16", False),
    (1, 2, 97, 97, 40, "bf16", True),
    (1, 1, 64, 300, 112, "f16", False),
    (1, 1, 33, 33, 8, "bf16", True),
]


@pytest.mark.parametrize("case", ODD_D, ids=lambda c: "B%dH%dNq%dNk%dd%d_%s_%s" % (
    c[:6] + ("causal" if c[6] else "full",)))
def test_bwd_padded_head_dim(case):
    """d outside {64, 128}: gradients of the unpadded problem, in tensors
    of the caller's shape; O and LSE from the oracle (fp32)."""
    B, H, Nq, Nk, d, dt, causal = case
    _say("case", case)
    q = make_qkv(B, H, Nq, d, dt, 1.0, seed=17)[0]
    _, k, v = make_qkv(B, H, Nk, d, dt, 1.0, seed=18)
    dout = make_dout(B, H, Nq, d, dt, seed=17)
    scale = _scale(d)
    o, lse = _oracle_o_lse(q, k, v, causal, scale)
    got = gpu_bwd(q, k, v, o, lse, dout, causal, scale)
    assert got[0].shape == q.shape and got[1].shape == k.shape and got[2].shape == v.shape
    ref = oracle.attn_bwd_oracle(q, k, v, dout, causal=causal, scale=scale)
    terms, extra = _terms(q, k, v, dout, causal, scale)
    check_grads(got, ref, terms, extra, U[dt], "padded d %s" % (case,))


# ------------------------------------------------------------- fp32 inputs
F32_CASES = [
    # (B, H, Nq, Nk, d, causal): the page's test shape, a larger head dim,
    # padded head dims, cross-attention
    (2, 4, 256, 256, 64, False), (2, 4, 256, 256, 64, True), (1, 2, 300, 300, 128, True),
    (1, 1, 97, 97, 40, True), (1, 2, 130, 130, 96, False), (1, 2, 64, 200, 128, False),
    (1, 1, 1, 1, 64, True),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "B%dH%dNq%dNk%dd%d_%s" % (
    c[:5] + ("causal" if c[5] else "full",)))
def test_bwd_f32(case):
    """fp32 inputs run in fp32 throughout: within the rounding bound above
    (u = 2^-16) and within the page's ~1e-3 for fp32 ("4.4 Writing GPU
    Kernels with Triton", section "Kernel 5: FlashAttention Backward", its
    test notes); O and LSE from the oracle (fp32)."""
    B, H, Nq, Nk, d, causal = case
    _say("case", case)
    q = make_qkv(B, H, Nq, d, "f32", 1.0, seed=19)[0]
    _, k, v = make_qkv(B, H, Nk, d, "f32", 1.0, seed=20)
    dout = make_dout(B, H, Nq, d, "f32", seed=19)
    scale = _scale(d)
    o, lse = _oracle_o_lse(q, k, v, causal, scale)
    got = gpu_bwd(q, k, v, o, lse, dout, causal, scale)
    ref = oracle.attn_bwd_oracle(q, k, v, dout, causal=causal, scale=scale)
    terms, extra = _terms(q, k, v, dout, causal, scale)
    check_grads(got, ref, terms, extra, U["f32"], "f32 %s" % (case,))
    for g, r in zip(got, ref):
        assert float(np.abs(g.double().numpy() - r).max()) <= 1e-3


def test_bwd_f32_end_to_end():
    """fp32 forward then fp32 backward."""
    B, H, N, d = 1, 2, 257, 128
    q, k, v, dout = _inputs(B, H, N, d, "f32", 1.0, seed=21)
    scale = _scale(d)
    dev = torch.device("cuda:0")
    o, lse = binding.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=True, scale=scale)
    got = gpu_bwd(q, k, v, o, lse, dout, True, scale)
    ref = oracle.attn_bwd_oracle(q, k, v, dout, causal=True, scale=scale)
    for g, r in zip(got, ref):
        assert float(np.abs(g.double().numpy() - r).max()) <= 1e-3


# ----------------------------------------------------------- strided views
@pytest.mark.parametrize("dt,d,causal", [("bf16", 128, True), ("f16", 64, False),
                                         ("bf16", 80, False), ("f32", 128, True)])
def test_bwd_strided_views(dt, d, causal):
    """q, k, v, dout, o and the gradients as [B, N, H, d] tensors seen as
    [B, H, N, d] (the layout of a fused projection): the same kernels with
    other addresses, so the gradients equal the contiguous call's bit for
    bit, and meet the oracle."""
    B, H, N = 2, 3, 203
    q, k, v, dout = _inputs(B, H, N, d, dt, 1.0, seed=22)
    scale = _scale(d)
    o, lse = _oracle_o_lse(q, k, v, causal, scale)
    dev = torch.device("cuda:0")

    def bnhd(x):
        return x.to(dev).transpose(1, 2).contiguous().transpose(1, 2)

    want = binding.attn_bwd(*(x.to(dev) for x in (q, k, v, o, lse, dout)), causal=causal,
                            scale=scale, grad_dtype=torch.float32)
    gbuf = [torch.full((B, N, H, d), float("nan"), device=dev) for _ in range(3)]
    grads = [g.transpose(1, 2) for g in gbuf]
    got = binding.attn_bwd(bnhd(q), bnhd(k), bnhd(v), bnhd(o), lse.to(dev), bnhd(dout),
                           causal=causal, scale=scale, grad_dtype=torch.float32, grads=grads)
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        assert not a.is_contiguous()
        assert torch.equal(a, b)
    ref = oracle.attn_bwd_oracle(q, k, v, dout, causal=causal, scale=scale)
    terms, extra = _terms(q, k, v, dout, causal, scale)
    check_grads([g.cpu() for g in got], ref, terms, extra, U[dt], "strided %s d=%d" % (dt, d))


def test_bwd_head_dim_out_of_range():
    """Head dims that padding cannot serve are refused before any launch."""
    for d in (4, 100, 136):
        x = torch.zeros(1, 1, 8, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.zeros(1, 1, 8, dtype=torch.float32, device="cuda")
        with pytest.raises(ValueError):
            binding.attn_bwd(x, x, x, x, lse, x)


# ------------------------------------------------ full-size, sampled rows

FULL = ["b2h32_n4096_d128_bf16_causal", "b8h12_n3000_d64_f16", "b4h16_n1024_d64_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_bwd_full_size_sampled(name):
    """The full workloads (GPU forward then backward, as a training step
    would run them): sampled query rows (dQ) and key rows (dK, dV) of two
    heads against the oracle, plus the Jacobian invariants on every head:
    the dK rows of a head sum to 0 and the dV rows to the dO rows' sum."""
    w = WORKLOADS[name]
    _say("workload", name)
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.sigma, seed=0)
    dout = make_dout(w.B, w.H, w.N, w.d, w.dtype, seed=0)
    dev = torch.device("cuda:0")
    o, lse = binding.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=w.causal, scale=w.scale,
                              out_dtype=torch.float32)
    dq, dk, dv = binding.attn_bwd(q.to(dev), k.to(dev), v.to(dev), o, lse, dout.to(dev),
                                  causal=w.causal, scale=w.scale, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    u = U[w.dtype]
    for x in (dq, dk, dv):
        assert bool(torch.isfinite(x).all())
    # invariants on every head (fp64 sums on the GPU of the fp32 gradients)
    sk = dk.double().sum(2)
    sv = dv.double().sum(2) - dout.to(dev).double().sum(2)
    mag_k = dk.double().abs().sum(2)
    mag_v = dv.double().abs().sum(2)
    assert bool((sk.abs() <= 16 * u * mag_k + 1e-4).all()), "dK rows do not sum to 0"
    assert bool((sv.abs() <= 16 * u * mag_v + 1e-4).all()), "dV rows do not sum to sum dO"
    # sampled rows of two heads
    rng = np.random.default_rng(0)
    N = w.N
    heads = [0, w.B * w.H - 1]
    for bh in heads:
        b, h = divmod(bh, w.H)
        rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, N // 2, N - 2, N - 1],
                                         rng.integers(0, N, 7)]))
        qh, kh, vh, dh = (x[b:b + 1, h:h + 1] for x in (q, k, v, dout))
        rq, rk, rv = oracle.attn_bwd_oracle(qh, kh, vh, dh, causal=w.causal, scale=w.scale,
                                            qrows=rows, krows=rows)
        ro, rl = oracle.attn_oracle(qh, kh, vh, causal=w.causal, scale=w.scale)
        dD = (dh.double() * (o[b:b + 1, h:h + 1].cpu().double() - torch.from_numpy(ro))).sum(-1)
        dL = lse[b:b + 1, h:h + 1].cpu().double() - torch.from_numpy(rl)
        terms, extra = _terms(qh, kh, vh, dh, w.causal, w.scale, dD=dD, dL=dL)
        got = [dq[b, h].cpu()[rows], dk[b, h].cpu()[rows], dv[b, h].cpu()[rows]]
        terms = [t[0, 0][rows] for t in terms]
        extra = [e[0, 0][rows] for e in extra]
        check_grads(got, (rq, rk, rv), terms, extra, u, "%s head %d" % (name, bh))


# ---------------------------------------------------- offsets past 2^31

def test_bwd_offsets_past_2_31():
    """B2^12 H2^8 N64 d64 bf16 causal: 2^32 elements per tensor, so element
    offsets pass 2^31 (byte offsets 2^32) in every input and gradient, with
    2^20 workgroups per launch. GPU forward then backward; whole heads on both
    sides of the crossing, and the first and last head, against the oracle.
    Inputs come from torch's seeded generator on the GPU; only the compared
    heads are copied back."""
    B, H, N, d, dt, causal = 4096, 256, 64, 64, "bf16", True
    _say("backward, offsets past 2^31")
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(32)
    q, k, v, dout = (torch.randn((B, H, N, d), generator=gen, device=dev, dtype=DT[dt])
                     for _ in range(4))
    scale = _scale(d)
    o, lse = binding.attn_fwd(q, k, v, causal=causal, scale=scale, out_dtype=torch.float32)
    dq, dk, dv = binding.attn_bwd(q, k, v, o, lse, dout, causal=causal, scale=scale,
                                  grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for x in (dq, dk, dv):
        assert bool(torch.isfinite(x).all())
    cross = (1 << 31) // (N * d)
    for bh in (0, cross - 1, cross, B * H - 1):
        b, h = divmod(bh, H)
        qh, kh, vh, dh = (x[b:b + 1, h:h + 1].cpu() for x in (q, k, v, dout))
        ref = oracle.attn_bwd_oracle(qh, kh, vh, dh, causal=causal, scale=scale)
        ro, rl = oracle.attn_oracle(qh, kh, vh, causal=causal, scale=scale)
        dD = (dh.double() * (o[b:b + 1, h:h + 1].cpu().double() - torch.from_numpy(ro))).sum(-1)
        dL = lse[b:b + 1, h:h + 1].cpu().double() - torch.from_numpy(rl)
        terms, extra = _terms(qh, kh, vh, dh, causal, scale, dD=dD, dL=dL)
        got = [x[b:b + 1, h:h + 1].cpu() for x in (dq, dk, dv)]
        check_grads(got, ref, terms, extra, U[dt], "head %d of %d" % (bh, B * H))
    del q, k, v, dout, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_bwd_shared_kv_heads():
    """Grouped-query attention through stride-0 views: Q as [B*Hkv, G, N, d],
    K and V as [B*Hkv, G, N, d] views of [B, Hkv, N, d] tensors with head
    stride 0. The backward reads the shared K and V in place and writes dK
    and dV per query head (disjoint outputs), which must equal the oracle's
    gradients for materialised copies of K and V; through autograd, the
    expand's own backward then sums them over each group."""
    B, H, Hkv, N, d, dt, causal = 2, 8, 2, 193, 128, "bf16", True
    G = H // Hkv
    q = make_qkv(B, H, N, d, dt, 1.0, seed=37)[0]
    _, kk, vv = make_qkv(B, Hkv, N, d, dt, 1.0, seed=38)
    dout = make_dout(B, H, N, d, dt, seed=37)
    scale = _scale(d)
    dev = torch.device("cuda:0")
    q4, do4 = (x.to(dev).view(B * Hkv, G, N, d) for x in (q, dout))
    k4, v4 = (x.to(dev).reshape(B * Hkv, 1, N, d).expand(B * Hkv, G, N, d) for x in (kk, vv))
    o, lse = binding.attn_fwd(q4, k4, v4, causal=causal, scale=scale, out_dtype=torch.float32)
    dq, dk, dv = binding.attn_bwd(q4, k4, v4, o, lse, do4, causal=causal, scale=scale,
                                  grad_dtype=torch.float32)
    torch.cuda.synchronize()
    kr, vr = (x.repeat_interleave(G, dim=1) for x in (kk, vv))
    ref = oracle.attn_bwd_oracle(q, kr, vr, dout, causal=causal, scale=scale)
    ro, rl = oracle.attn_oracle(q, kr, vr, causal=causal, scale=scale)
    dD = (dout.double() * (o.view(B, H, N, d).cpu().double() - torch.from_numpy(ro))).sum(-1)
    dL = lse.view(B, H, N).cpu().double() - torch.from_numpy(rl)
    terms, extra = _terms(q, kr, vr, dout, causal, scale, dD=dD, dL=dL)
    got = [x.view(B, H, N, d).cpu() for x in (dq, dk, dv)]
    check_grads(got, ref, terms, extra, U[dt], "shared K/V heads")
    # autograd over the stride-0 views: the group sums land in the shared tensors
    from io_aware_attention_flash_amd.ops import flash_attn_func
    kg, vg = (x.to(dev).reshape(B * Hkv, 1, N, d).clone().requires_grad_() for x in (kk, vv))
    qg = q4.clone().requires_grad_()
    flash_attn_func(qg, kg.expand(B * Hkv, G, N, d), vg.expand(B * Hkv, G, N, d),
                    causal=causal, scale=scale).backward(do4)
    torch.cuda.synchronize()
    for name, g, per_head in (("dK", kg.grad, dk), ("dV", vg.grad, dv)):
        want = per_head.double().sum(1, keepdim=True)
        rel = float((g.double() - want).norm() / want.norm())
        print("shared K/V heads, autograd %s: relative error %.2e" % (name, rel), flush=True)
        # bf16 gradients per head, summed: a few units of bf16 rounding
        assert torch.isfinite(g).all() and rel <= 4 * U[dt], name
