"""GPU parity of the general-layout forward (attn_fwd_strided): cross-attention,
head dims other than 64 / 128 and strided tensors, against the fp64 oracle
on the same seeded inputs. Tolerances are the forward's: O max |err| <= 1e-2
and mean |err| <= 1e-3 (fp32 output), LSE max |err| <= 1e-3."""
import os

import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_flash_amd import binding
from io_aware_attention_flash_amd import build as hipbuild
from io_aware_attention_flash_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3
DEV = torch.device("cuda:0")


def setup_module(module):
    hipbuild.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _scale(d):
    return float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))


def _qkv(B, H, Nq, Nk, d, dt, sigma, seed):
    q = make_qkv(B, H, Nq, d, dt, sigma, seed=seed)[0]
    _, k, v = make_qkv(B, H, Nk, d, dt, sigma, seed=seed + 1)
    return q, k, v


def _check(o, lse, q, k, v, causal, scale, what):
    ro, rl = oracle.attn_oracle(q, k, v, causal=causal, scale=scale)
    err = np.abs(o.detach().cpu().double().numpy() - ro)
    lerr = np.abs(lse.detach().cpu().double().numpy() - rl)
    print("%s: O max %.3e mean %.3e | LSE max %.3e" % (what, err.max(), err.mean(), lerr.max()),
          flush=True)
    assert np.all(np.isfinite(err)) and np.all(np.isfinite(lerr)), what
    assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr.max() <= LSE_MAX, what


CROSS = [
    # (B, H, Nq, Nk, d, dtype, sigma): the page's two shapes first
    (1, 1, 5, 15, 32, "f32", 1.0), (1, 1, 1, 10, 64, "f32", 1.0),
    (1, 1, 5, 15, 32, "bf16", 1.0), (1, 1, 1, 10, 64, "f16", 1.0),
    (2, 3, 300, 77, 128, "bf16", 1.0), (1, 2, 64, 1000, 64, "f16", 1.0),
    (1, 1, 129, 257, 128, "bf16", 3.0), (2, 2, 1, 1, 8, "f16", 1.0),
    (1, 2, 200, 130, 96, "f32", 1.0),
    # d <= 64 takes 128-key tiles up to 1024 keys and 64-key tiles past that
    (1, 2, 100, 1024, 64, "bf16", 1.0), (1, 2, 100, 1025, 64, "f16", 1.0),
    (1, 1, 70, 1500, 48, "bf16", 2.0),
    # d = 64 / 128 in bf16/fp16 run on the tuned kernels: few keys, one query, many query
    # tiles against few keys, a ragged key tail
    (1, 2, 257, 1, 128, "bf16", 1.0), (1, 3, 1, 5000, 128, "bf16", 1.0),
    (2, 2, 700, 129, 64, "f16", 1.0), (1, 4, 2048, 333, 128, "bf16", 1.0),
]


@pytest.mark.parametrize("case", CROSS, ids=lambda c: "B%dH%dNq%dNk%dd%d_%s_s%g" % c)
def test_cross_attention(case):
    B, H, Nq, Nk, d, dt, sigma = case
    print("case", case, flush=True)
    q, k, v = _qkv(B, H, Nq, Nk, d, dt, sigma, seed=31)
    scale = _scale(d)
    o, lse = binding.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(o, lse, q, k, v, False, scale, "cross %s" % (case,))


HEAD_DIMS = [(8, "bf16", False), (32, "f16", True), (48, "bf16", True), (72, "f16", False),
             (80, "bf16", True), (96, "f16", True), (112, "bf16", False), (24, "f32", True)]


@pytest.mark.parametrize("d,dt,causal", HEAD_DIMS)
def test_head_dims(d, dt, causal):
    print("case d", d, dt, causal, flush=True)
    for (B, H, N) in ((1, 2, 100), (2, 1, 300)):
        q, k, v = make_qkv(B, H, N, d, dt, 1.0, seed=32)
        scale = _scale(d)
        o, lse = binding.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale,
                                  out_dtype=torch.float32)
        torch.cuda.synchronize()
        _check(o, lse, q, k, v, causal, scale, "d=%d %s causal=%s N=%d" % (d, dt, causal, N))


@pytest.mark.parametrize("dt,causal", [("bf16", True), ("f16", False), ("f32", True)])
def test_strided_layouts(dt, causal):
    """Q, K, V from a [B, N, H, d] projection (strides (N H d, d, H d)); V a
    column slice of a wider tensor (row stride > d); O written into a
    [B, N, H, d] buffer through its transposed view."""
    B, H, N, d = 2, 3, 190, 80
    print("case strided", dt, causal, flush=True)
    g = torch.Generator().manual_seed(33)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
    qkv = torch.randn(B, N, 3, H, d, generator=g).to(tdt)
    wide = torch.randn(B, H, N, 128, generator=g).to(tdt)
    q, k = qkv[:, :, 0].transpose(1, 2), qkv[:, :, 1].transpose(1, 2)
    v = wide[..., :d]
    scale = _scale(d)
    qkv_g = qkv.to(DEV)
    qg, kg = qkv_g[:, :, 0].transpose(1, 2), qkv_g[:, :, 1].transpose(1, 2)
    vg = wide.to(DEV)[..., :d]
    assert not (qg.is_contiguous() or kg.is_contiguous() or vg.is_contiguous())
    obuf = torch.zeros(B, N, H, d, dtype=torch.float32, device=DEV)
    o, lse = binding.attn_fwd(qg, kg, vg, causal=causal, scale=scale, out_dtype=torch.float32,
                              out=obuf.transpose(1, 2))
    torch.cuda.synchronize()
    assert o.data_ptr() == obuf.data_ptr()
    _check(obuf.transpose(1, 2), lse, q.contiguous(), k.contiguous(), v.contiguous(), causal,
           scale, "strided %s causal=%s" % (dt, causal))


TUNED_STRIDED = [
    # (B, H, N, d, dtype, causal, out_dtype, V scale): tile shapes 8x64 and 4x32 (d=128),
    # 8x128 and 4x64 (d=64); bf16 V beyond fp16's range (recomputed rows)
    (2, 4, 1000, 128, "bf16", True, "f32", 1.0),
    (1, 8, 2048, 128, "bf16", True, "f32", 1.0),
    (4, 16, 1024, 64, "bf16", False, "in", 1.0),
    (2, 3, 777, 64, "f16", False, "f32", 1.0),
    (1, 2, 300, 128, "bf16", True, "f32", 1e5),
]


@pytest.mark.parametrize("case", TUNED_STRIDED, ids=lambda c: "B%dH%dN%dd%d_%s_c%d_%s_v%g" % c)
def test_tuned_kernels_on_strided_views(case):
    """attn_fwd_strided on self-attention at d = 64 or 128 runs the tuned
    kernels with the tensors' own strides: Q and K as [B, N, H, d] views of
    a fused projection, V a column slice of a wider [B, N, H, 2d] tensor (row
    stride 2 H d), O into a [B, N, H, d] buffer. Only the addressing differs
    from the contiguous call, so O and LSE must equal it bit for bit; the
    contiguous call is itself held to the oracle on a few rows."""
    B, H, N, d, dt, causal, out, vscale = case
    print("case tuned strided", case, flush=True)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    odt = torch.float32 if out == "f32" else tdt
    q, k, v = make_qkv(B, H, N, d, dt, 1.0, seed=36)
    v = (v.float() * vscale).to(tdt)
    scale = _scale(d)
    qkv = torch.empty(B, N, 3, H, d, dtype=tdt, device=DEV)
    wide = torch.zeros(B, N, H, 2 * d, dtype=tdt, device=DEV)
    qs, ks = qkv[:, :, 0].transpose(1, 2), qkv[:, :, 1].transpose(1, 2)
    vs = wide.transpose(1, 2)[..., d:]
    qs.copy_(q.to(DEV)), ks.copy_(k.to(DEV)), vs.copy_(v.to(DEV))
    assert not (qs.is_contiguous() or ks.is_contiguous() or vs.is_contiguous())
    assert vs.stride(2) == 2 * H * d
    obuf = torch.full((B, N, H, d), float("nan"), dtype=odt, device=DEV)
    o_s, lse_s = binding.attn_fwd(qs, ks, vs, causal=causal, scale=scale, out_dtype=odt,
                                  out=obuf.transpose(1, 2))
    o_c, lse_c = binding.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale,
                                  out_dtype=odt)
    torch.cuda.synchronize()
    assert o_s.data_ptr() == obuf.data_ptr()
    assert torch.isfinite(o_c).all()
    assert torch.equal(o_s, o_c), "O: max diff %.3e" % float((o_s.float() - o_c.float()).abs().max())
    assert torch.equal(lse_s, lse_c), "LSE differs"
    rows = np.array([0, 1, N // 2, N - 1])
    ro, rl = oracle.attn_oracle(q[:1, :1], k[:1, :1], v[:1, :1], causal=causal, scale=scale,
                                rows=rows)
    vmax = max(1.0, float(v[:1, :1].float().abs().max()))
    err = np.abs(o_c[0, 0].cpu().double().numpy()[rows] - ro).max()
    bar = (1e-2 + (2.0 ** -9 if out == "in" else 0.0) * np.abs(ro).max()) * vmax
    assert err <= bar, "O rows: %.3e" % err
    assert np.abs(lse_c[0, 0].cpu().double().numpy()[rows] - rl).max() <= 1e-3


def test_tuned_strided_full_headline_shape():
    """The strided instance at the full B2 H32 N4096 d128 causal bf16 shape on
    [B, N, H, d] views (what bench.py --pass fwd_general times): every element
    of O and LSE equals the contiguous call's."""
    B, H, N, d = 2, 32, 4096, 128
    q, k, v = (x.to(DEV) for x in make_qkv(B, H, N, d, "bf16", 1.0, seed=0))
    qs, ks, vs = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    scale = _scale(d)
    obuf = torch.empty(B, N, H, d, dtype=torch.float32, device=DEV)
    o_s, lse_s = binding.attn_fwd(qs, ks, vs, causal=True, scale=scale, out_dtype=torch.float32,
                                  out=obuf.transpose(1, 2))
    o_c, lse_c = binding.attn_fwd(q, k, v, causal=True, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_c) and torch.equal(lse_s, lse_c)


def test_tuned_cross_attention_large():
    """Cross-attention at B2 H16 Nq 4096 Nk 1024 d128 bf16 on the tuned
    kernels: sampled rows of every head against the oracle (the forward's
    bar), properties over every output."""
    B, H, Nq, Nk, d = 2, 16, 4096, 1024, 128
    q, k, v = _qkv(B, H, Nq, Nk, d, "bf16", 1.0, seed=38)
    scale = _scale(d)
    o, lse = binding.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    oc, lc = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.all(np.isfinite(oc)) and np.all(np.isfinite(lc))
    vmin = v.double().numpy().min(axis=2, keepdims=True)
    vmax = v.double().numpy().max(axis=2, keepdims=True)
    assert np.all(oc >= vmin - 1e-6) and np.all(oc <= vmax + 1e-6)
    rng = np.random.default_rng(38)
    rows_in_head = np.unique(np.concatenate([[0, 1, 255, 256, Nq - 1], rng.integers(0, Nq, 12)]))
    rows = np.concatenate([bh * Nq + rows_in_head for bh in range(B * H)])
    ro, rl = oracle.attn_oracle(q, k, v, causal=False, scale=scale, rows=rows)
    go = oc.reshape(B * H * Nq, d)[rows]
    gl = lc.reshape(B * H * Nq)[rows]
    err, lerr = np.abs(go - ro), np.abs(gl - rl)
    print("cross large: O max %.3e mean %.3e | LSE max %.3e over %d rows" % (
        err.max(), err.mean(), lerr.max(), len(rows)), flush=True)
    assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr.max() <= LSE_MAX


PADDED = [
    # (B, H, Nq, Nk, d, dtype, causal): computed at D = 128 (d > 64) or 64 (Nk >= 256)
    (2, 3, 1000, 1000, 80, "bf16", True), (1, 4, 700, 700, 96, "f16", False),
    (2, 2, 513, 513, 112, "bf16", True), (1, 3, 600, 600, 40, "bf16", True),
    (2, 2, 300, 1100, 24, "f16", False), (1, 2, 77, 2000, 72, "bf16", False),
]


@pytest.mark.parametrize("case", PADDED, ids=lambda c: "B%dH%dNq%dNk%dd%d_%s_c%d" % c)
def test_tuned_kernels_on_padded_head_dims(case):
    """Head dims other than 64 and 128 on the tuned kernels (strided
    instances): the columns d .. D-1 are read as zeros, so the result equals,
    bit for bit, the contiguous call on the same tensors zero-padded to D
    columns (O's first d columns, LSE); the padded call is held to the
    oracle on a few rows."""
    B, H, Nq, Nk, d, dt, causal = case
    print("case padded", case, flush=True)
    D = 64 if d <= 64 else 128
    q, k, v = _qkv(B, H, Nq, Nk, d, dt, 1.0, seed=37)
    scale = _scale(d)
    o, lse = binding.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale,
                              out_dtype=torch.float32)
    pad = lambda x: torch.nn.functional.pad(x, (0, D - d)).to(DEV)
    if Nq == Nk:
        o_p, lse_p = binding.attn_fwd(pad(q), pad(k), pad(v), causal=causal, scale=scale,
                                      out_dtype=torch.float32)
    else:  # the contiguous tuned call needs Nq == Nk: the strided entry on padded tensors
        o_p, lse_p = binding.attn_fwd_general(pad(q), pad(k), pad(v), causal=causal, scale=scale,
                                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o_p[..., :d]), "O: max diff %.3e" % float((o - o_p[..., :d]).abs().max())
    assert torch.equal(lse, lse_p)
    assert not o_p[..., d:].abs().max() > 0
    _check(o, lse, q, k, v, causal, scale, "padded %s" % (case,))


@pytest.mark.parametrize("d,dt,causal", [(128, "bf16", True), (64, "f16", False)])
def test_general_kernel_on_fast_shapes(d, dt, causal):
    """attn_fwd_strided on contiguous shapes the tuned kernels take: it runs
    them too, so its result equals attn_fwd's bit for bit; both within the
    forward's tolerance of the oracle."""
    B, H, N = 2, 2, 513
    q, k, v = make_qkv(B, H, N, d, dt, 1.0, seed=34)
    scale = _scale(d)
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = binding.attn_fwd_general(qg, kg, vg, causal=causal, scale=scale,
                                      out_dtype=torch.float32)
    o2, lse2 = binding.attn_fwd(qg, kg, vg, causal=causal, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    _check(o, lse, q, k, v, causal, scale, "general d=%d" % d)
    _check(o2, lse2, q, k, v, causal, scale, "tuned d=%d" % d)


def test_input_dtype_output():
    """bf16 output of a cross-attention call: within 1e-2 plus half an ulp."""
    q, k, v = _qkv(1, 2, 150, 260, 96, "bf16", 1.0, seed=35)
    scale = _scale(96)
    o, lse = binding.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    ro, _ = oracle.attn_oracle(q, k, v, causal=False, scale=scale)
    err = np.abs(o.cpu().double().numpy() - ro)
    assert np.all(err <= 1e-2 + 0.5 * np.abs(ro) * 2.0 ** -8 + 1e-30)


# Shared key/value heads through stride-0 views: multi-query attention (one
# K/V head for all H query heads) and grouped-query attention (Hkv K/V heads,
# each shared by G = H / Hkv query heads, by viewing Q as [B*Hkv, G, N, d] and
# K, V as [B*Hkv, G, N, d] with head stride 0). The kernels only read K and V,
# so aliased inputs need no copy; the oracle gets materialised copies.
SHARED_KV = [
    # (B, H, Hkv, Nq, Nk, d, dtype, causal)
    (2, 8, 1, 300, 300, 128, "bf16", True),
    (2, 8, 2, 257, 257, 64, "f16", False),
    (1, 12, 4, 200, 517, 128, "bf16", False),
    (2, 6, 3, 190, 190, 96, "bf16", True),
    (1, 4, 1, 100, 100, 64, "f32", True),
]


@pytest.mark.parametrize("case", SHARED_KV, ids=lambda c: "B%dH%dHkv%dNq%dNk%dd%d_%s_%s" % (
    c[:7] + ("causal" if c[7] else "full",)))
def test_shared_kv_heads(case):
    B, H, Hkv, Nq, Nk, d, dt, causal = case
    G = H // Hkv
    print("case shared K/V heads", case, flush=True)
    q = make_qkv(B, H, Nq, d, dt, 1.0, seed=35)[0]
    _, kk, vv = make_qkv(B, Hkv, Nk, d, dt, 1.0, seed=36)
    scale = _scale(d)
    qd, kd, vd = q.to(DEV), kk.to(DEV), vv.to(DEV)
    # [B*Hkv, G, n, d] views; K and V repeat each of their heads G times (stride 0)
    q4 = qd.view(B * Hkv, G, Nq, d)
    k4, v4 = (x.reshape(B * Hkv, 1, Nk, d).expand(B * Hkv, G, Nk, d) for x in (kd, vd))
    assert k4.stride(1) == 0 and v4.stride(1) == 0
    o, lse = binding.attn_fwd(q4, k4, v4, causal=causal, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    kr, vr = (x.repeat_interleave(G, dim=1) for x in (kk, vv))  # [B, H, Nk, d] copies
    _check(o.view(B, H, Nq, d), lse.view(B, H, Nq), q, kr, vr, causal, scale,
           "shared K/V %s" % (case,))
