"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Tolerances (fixed for this method, bf16/fp16 in with fp32 accumulation):
  O   : max |err| <= 1e-2 and mean |err| <= 1e-3 over the compared elements
  LSE : max |err| <= 1e-3
O is compared as fp32 output; the input-dtype output is checked separately
(within 1e-2 plus half an ulp of the output type).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_flash_amd import binding
from io_aware_attention_flash_amd import build as hipbuild
from io_aware_attention_flash_amd.inputs import WORKLOADS, make_qkv, workload_qkv

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def setup_module(module):
    hipbuild.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _say(*a):
    print(*a, flush=True)


def gpu_attn(q, k, v, causal, scale, out_dtype=torch.float32):
    dev = torch.device("cuda:0")
    o, lse = binding.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale,
                              out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _scale(d):
    return float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))


def check_close(o, lse, ref_o, ref_lse, what):
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    err = np.abs(o - ref_o)
    lerr = np.abs(lse - ref_lse)
    _say("%s: O max %.3e mean %.3e | LSE max %.3e" % (what, err.max(), err.mean(), lerr.max()))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what + ": non-finite output"
    assert err.max() <= O_MAX, "%s: O max abs err %.3e" % (what, err.max())
    assert err.mean() <= O_MEAN, "%s: O mean abs err %.3e" % (what, err.mean())
    assert lerr.max() <= LSE_MAX, "%s: LSE max abs err %.3e" % (what, lerr.max())


# ---------------------------------------------------------------- full compare
SMALL_CASES = [
    # (B, H, N, d, dtype, causal, sigma)
    (2, 4, 256, 64, "f16", False, 1.0),   # the chapter's own test shape
    (2, 4, 256, 64, "f16", True, 1.0),
    (1, 1, 128, 64, "f32", False, 1.0),   # the single-head fp32 workload
    (1, 2, 300, 128, "f32", True, 1.0),
    (1, 2, 1, 64, "bf16", False, 1.0),
    (1, 2, 1, 128, "f16", True, 1.0),
    (2, 2, 63, 64, "bf16", True, 1.0),
    (1, 3, 65, 128, "bf16", False, 1.0),
    (1, 2, 127, 64, "f16", True, 1.0),
    (1, 2, 129, 128, "bf16", True, 1.0),
    (1, 2, 200, 64, "bf16", False, 1.0),
    (2, 1, 333, 128, "f16", False, 1.0),
    (1, 2, 517, 128, "bf16", True, 3.0),
    (1, 2, 640, 64, "f16", True, 1.0),
    (1, 1, 1000, 128, "bf16", False, 3.0),
    # key-tile edges (d=128: 32 or 64 keys per tile, d=64: 64 or 128)
    (1, 2, 64, 128, "f16", False, 1.0),
    (1, 2, 128, 64, "bf16", True, 1.0),
    (1, 2, 129, 64, "bf16", False, 1.0),
    (1, 1, 191, 128, "bf16", True, 1.0),
    (1, 1, 192, 128, "f16", True, 1.0),
    (1, 1, 385, 64, "f16", True, 2.0),
    (3, 5, 97, 128, "bf16", True, 1.0),
    # query-tile edges (128 or 256 rows per workgroup)
    (1, 1, 255, 128, "bf16", True, 1.0),
    (1, 1, 256, 128, "f16", True, 1.0),
    (1, 2, 257, 128, "bf16", False, 1.0),
    (1, 1, 511, 128, "f16", False, 1.0),
    (2, 1, 513, 128, "bf16", True, 2.0),
    # enough heads that the 256-row tiles fill whole rounds of workgroups, so
    # the library takes them (d=128: 64-key tiles, d=64: 128-key), with
    # ragged last query and key tiles; the cases above take the 128-row ones
    (4, 16, 2000, 128, "bf16", True, 1.0),
    (8, 32, 1000, 128, "f16", False, 1.0),
    (8, 16, 1000, 64, "bf16", True, 2.0),
    (4, 16, 1000, 64, "f16", False, 1.0),
    # B*H a multiple of 8: workgroup ids run head-major within each XCD
    (2, 8, 700, 128, "bf16", True, 1.0),
    (1, 16, 777, 128, "f16", False, 1.0),
    (3, 8, 200, 64, "f16", False, 1.0),
    (2, 12, 400, 64, "bf16", True, 1.0),
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: "B%dH%dN%dd%d_%s_%s_s%g" % (
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full", c[6]))
def test_parity_full(case):
    B, H, N, d, dt, causal, sigma = case
    _say("case", case)
    q, k, v = make_qkv(B, H, N, d, dt, sigma, seed=1)
    sc = _scale(d)
    ref_o, ref_l = oracle.attn_oracle(q, k, v, causal=causal, scale=sc)
    o, lse = gpu_attn(q, k, v, causal, sc)
    check_close(o.numpy(), lse.numpy(), ref_o, ref_l, str(case))


# ------------------------------------------- the named workloads, every element
FULL_WORKLOAD_CASES = [(name, 0) for name in WORKLOADS] + [
    ("b2h32_n4096_d128_bf16_causal", 1), ("b2h32_n4096_d128_bf16_causal", 2)]


def _log_parity(record):
    """Append one JSON line per compared workload to $ATTN_PARITY_LOG, when set."""
    path = os.environ.get("ATTN_PARITY_LOG")
    if path:
        import json
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")


@pytest.mark.parametrize("name,seed", FULL_WORKLOAD_CASES,
                         ids=["%s_seed%d" % c for c in FULL_WORKLOAD_CASES])
def test_parity_workload_full(name, seed):
    """Every element of O (fp32 output) and of LSE of a named workload against
    the oracle: max and mean |err| over all B*H*N*d outputs, max |err| over
    all B*H*N log-sum-exps, at the launch configuration bench.py times."""
    w = WORKLOADS[name]
    _say("full workload", name, "seed", seed)
    q, k, v = workload_qkv(w, seed=seed)
    o, lse = gpu_attn(q, k, v, w.causal, w.scale)
    ref_o, ref_l = oracle.attn_oracle(q, k, v, causal=w.causal, scale=w.scale)
    o = o.numpy().astype(np.float64)
    lse = lse.numpy().astype(np.float64)
    err = np.abs(o - ref_o)
    lerr = np.abs(lse - ref_l)
    rec = {"workload": name, "seed": seed, "elements": int(err.size), "rows": int(lerr.size),
           "o_max_abs": float(err.max()), "o_mean_abs": float(err.mean()),
           "lse_max_abs": float(lerr.max())}
    _log_parity(rec)
    check_close(o, lse, ref_o, ref_l, "%s seed %d (all %d elements)" % (name, seed, err.size))


# ---------------------------------------------- the named workloads, sampled
def _sample_rows(B, H, N, n_heads=6, n_rand=40, seed=0):
    rng = np.random.default_rng(seed)
    heads = sorted(set([0, B * H - 1] + list(rng.integers(0, B * H, n_heads - 2))))
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, N // 2, N - 129, N - 128, N - 65,
             N - 64, N - 2, N - 1]
    rows = []
    for bh in heads:
        ii = sorted(set([i for i in fixed if 0 <= i < N] + list(rng.integers(0, N, n_rand))))
        rows += [bh * N + i for i in ii]
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("seed", [0, 1])
def test_parity_workload_sampled(name, seed):
    w = WORKLOADS[name]
    _say("workload", name, "seed", seed)
    q, k, v = workload_qkv(w, seed=seed)
    o, lse = gpu_attn(q, k, v, w.causal, w.scale)
    rows = _sample_rows(w.B, w.H, w.N, seed=seed)
    ref_o, ref_l = oracle.attn_oracle(q, k, v, causal=w.causal, scale=w.scale, rows=rows)
    check_close(o.reshape(-1, w.d).numpy()[rows], lse.reshape(-1).numpy()[rows], ref_o, ref_l,
                "%s seed %d (%d sampled rows)" % (name, seed, len(rows)))
    # Properties over every output: finite, inside the per-column hull of V
    # (causal rows only see a prefix, whose hull lies inside the full one).
    of = o.double()
    assert torch.isfinite(of).all() and torch.isfinite(lse).all()
    vf = v.double()
    lo = vf.min(dim=2, keepdim=True).values - 1e-3
    hi = vf.max(dim=2, keepdim=True).values + 1e-3
    assert bool(((of >= lo) & (of <= hi)).all()), "output outside the hull of V"
    # LSE >= max visible score; a loose lower bound that holds for every row:
    # LSE_i >= s_ii (causal) -- cheap to check on the diagonal.
    if w.causal:
        diag = (q.double() * k.double()).sum(-1) * w.scale
        assert bool((lse.double() >= diag - 1e-3).all())


# ------------------------------------------------------------ long sequences
LONG_CASES = [
    # (B, H, N, d, dtype, causal): one head at a million keys (row and key
    # indices past 2^19, 4096 query tiles), and a non-causal fp16 d=64 head
    # at 2^18
    (1, 1, 1 << 20, 128, "bf16", True),
    (1, 1, 1 << 18, 64, "f16", False),
]


@pytest.mark.parametrize("case", LONG_CASES, ids=lambda c: "N%d_d%d_%s_%s" % (
    c[2], c[3], c[4], "causal" if c[5] else "full"))
def test_long_sequence_sampled(case):
    """Sampled rows of one very long head against the oracle: the first and
    last rows, rows on both sides of query-tile and pairing boundaries, and
    random rows."""
    B, H, N, d, dt, causal = case
    _say("long sequence", case)
    q, k, v = make_qkv(B, H, N, d, dt, 1.0, seed=5)
    sc = _scale(d)
    o, lse = gpu_attn(q, k, v, causal, sc)
    rng = np.random.default_rng(5)
    fixed = [0, 1, 127, 128, 255, 256, 257, N // 2 - 1, N // 2, N - 257, N - 256, N - 129, N - 1]
    rows = np.array(sorted(set(fixed + list(rng.integers(0, N, 8)))), dtype=np.int64)
    ref_o, ref_l = oracle.attn_oracle(q, k, v, causal=causal, scale=sc, rows=rows)
    check_close(o.reshape(-1, d).numpy()[rows], lse.reshape(-1).numpy()[rows], ref_o, ref_l,
                "N=%d d=%d (%d sampled rows)" % (N, d, len(rows)))
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


# ---------------------------------------------------- offsets past 2^31
BIG_CASES = [
    # (B, H, N, d, dtype, causal, layout): 2^32 elements per tensor, so the
    # element offsets of the later heads pass 2^31 (byte offsets 2^32) and the
    # grid has 2^20 workgroups; "bnhd" passes [B, N, H, d] tensors as
    # transposed views
    (4096, 256, 64, 64, "bf16", True, "bhnd"),
    (2048, 512, 32, 128, "f16", False, "bhnd"),
    (4096, 256, 64, 64, "bf16", False, "bnhd"),
    (4096, 256, 64, 64, "f32", True, "bhnd"),    # the fp32 kernel
    (4096, 256, 64, 64, "f32", False, "bnhd"),   # the general kernel (fp32 views)
]


@pytest.mark.parametrize("case", BIG_CASES, ids=lambda c: "B%dH%dN%d_d%d_%s_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full", c[6]))
def test_offsets_past_2_31(case):
    """Whole heads on both sides of element offset 2^31, the first and the
    last head against the oracle. Inputs come from torch's seeded generator
    on the GPU (2^32 values per tensor); only the compared heads are copied
    back for the oracle."""
    B, H, N, d, dt, causal, layout = case
    _say("offsets past 2^31", case)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(31)
    shape = (B, H, N, d) if layout == "bhnd" else (B, N, H, d)
    q, k, v = (torch.randn(shape, generator=gen, device=dev, dtype=DT[dt]) for _ in range(3))
    if layout == "bnhd":
        q, k, v = (x.transpose(1, 2) for x in (q, k, v))
    sc = _scale(d)
    o, lse = binding.attn_fwd(q, k, v, causal=causal, scale=sc, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    cross = (1 << 31) // (N * d)  # first head whose elements start at offset 2^31
    for bh in (0, cross - 1, cross, B * H - 1):
        b, h = divmod(bh, H)
        qh, kh, vh = (x[b:b + 1, h:h + 1].cpu() for x in (q, k, v))
        ref_o, ref_l = oracle.attn_oracle(qh, kh, vh, causal=causal, scale=sc)
        check_close(o[b:b + 1, h:h + 1].cpu().numpy(), lse[b:b + 1, h:h + 1].cpu().numpy(),
                    ref_o, ref_l, "head %d of %d" % (bh, B * H))
    del q, k, v, o, lse
    torch.cuda.empty_cache()


# ------------------------------------------------------------- special cases
def test_exercise5_embedded():
    """Exercise 5 of the Triton chapter inside a d=64 head: q0 = e0,
    keys 2 e0 and 4 e0, values 1 e0 and 3 e0, scale 1."""
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "exercise5_online_softmax.json")))
    for dt in ("bf16", "f16", "f32"):
        q = torch.zeros(1, 1, 2, 64)
        k = torch.zeros(1, 1, 2, 64)
        v = torch.zeros(1, 1, 2, 64)
        q[0, 0, :, 0] = 1.0
        k[0, 0, :, 0] = torch.tensor(g["scores"])
        v[0, 0, :, 0] = torch.tensor(g["values"])
        o, lse = gpu_attn(q.to(DT[dt]), k.to(DT[dt]), v.to(DT[dt]), False, 1.0)
        assert abs(float(o[0, 0, 1, 0]) - g["O_normalised"]) <= 1e-3, dt
        assert abs(float(lse[0, 0, 1]) - g["lse"]) <= 1e-4, dt
        assert float(o[0, 0, 1, 1:].abs().max()) == 0.0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_zero_scale_is_mean_of_v(causal, dt):
    B, H, N, d = 1, 2, 150, 64
    q, k, v = make_qkv(B, H, N, d, dt, 1.0, seed=3)
    o, lse = gpu_attn(q, k, v, causal, 0.0)
    vf = v.double()
    cnt = torch.arange(1, N + 1, dtype=torch.float64).view(1, 1, N, 1)
    want = vf.cumsum(2) / cnt if causal else vf.mean(2, keepdim=True).expand_as(vf)
    n_vis = cnt.view(1, 1, N) if causal else torch.full((1, 1, N), float(N), dtype=torch.float64)
    assert float((o.double() - want).abs().max()) <= 2e-3
    assert float((lse.double() - n_vis.log()).abs().max()) <= 1e-4


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_causal_first_row_is_v0(dt):
    q, k, v = make_qkv(2, 3, 200, 128, dt, 1.0, seed=4)
    o, lse = gpu_attn(q, k, v, True, _scale(128))
    # p = exp2(0) = 1 exactly, l = 1, so O_0 = V_0 exactly in fp32.
    assert torch.equal(o[:, :, 0, :], v[:, :, 0, :].float())


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_input_dtype_output(dt):
    B, H, N, d = 2, 2, 333, 128
    q, k, v = make_qkv(B, H, N, d, dt, 1.0, seed=5)
    sc = _scale(d)
    ref_o, _ = oracle.attn_oracle(q, k, v, causal=True, scale=sc)
    o, _ = gpu_attn(q, k, v, True, sc, out_dtype=DT[dt])
    assert o.dtype == DT[dt]
    half_ulp = np.abs(ref_o) * (2.0 ** -8 if dt == "bf16" else 2.0 ** -11)
    err = np.abs(o.double().numpy() - ref_o)
    assert np.all(err <= 1e-2 + half_ulp), float(err.max())


def test_deterministic_bitwise():
    w = WORKLOADS["b4h16_n1024_d64_bf16"]
    q, k, v = (x.cuda() for x in workload_qkv(w, seed=7))
    o1, l1 = binding.attn_fwd(q, k, v, causal=True, scale=w.scale, out_dtype=torch.float32)
    o2, l2 = binding.attn_fwd(q, k, v, causal=True, scale=w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_head_dim_zero_padding(dt):
    """d=64 data zero-padded to d=128 at the same scale: same O and LSE
    (exact in the math). The two head dims run with different key-tile
    widths, so p is rounded to fp16 against different running maxima and the
    results agree to the parity tolerance, not bitwise."""
    q, k, v = make_qkv(1, 2, 257, 64, dt, 1.0, seed=8)
    pad = lambda x: torch.cat([x, torch.zeros_like(x)], dim=-1)  # noqa: E731
    o64, l64 = gpu_attn(q, k, v, True, 0.125)
    o128, l128 = gpu_attn(pad(q), pad(k), pad(v), True, 0.125)
    assert float(o128[..., 64:].abs().max()) == 0.0
    assert float((o128[..., :64] - o64).abs().max()) <= 2e-3
    assert float((l128 - l64).abs().max()) <= LSE_MAX


def test_out_and_lse_buffers_untouched_outside():
    """Writes stay inside O and LSE: guard regions around them keep their fill."""
    B, H, N, d = 1, 2, 130, 64
    q, k, v = (x.cuda() for x in make_qkv(B, H, N, d, "bf16", 1.0, seed=9))
    n = B * H * N * d
    big = torch.full((n + 2048,), 7.0, device="cuda")
    lbig = torch.full((B * H * N + 2048,), 7.0, device="cuda")
    o = big[1024:1024 + n].view(B, H, N, d)
    lse = lbig[1024:1024 + B * H * N].view(B, H, N)
    binding.attn_fwd(q, k, v, causal=False, scale=0.125, out_dtype=torch.float32, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((big[:1024] == 7.0).all() and (big[1024 + n:] == 7.0).all())
    assert bool((lbig[:1024] == 7.0).all() and (lbig[1024 + B * H * N:] == 7.0).all())


# ------------------------------------------- the workspace (first-pass) path
WS_CASES = [
    # (B, H, N, d, causal): long bf16 sequences take the first pass
    (1, 2, 8192, 128, True),
    (1, 1, 8200, 64, False),
]


def _raw(q, k, v, causal, scale, ws=None, ws_bytes=0):
    B, H, N, d = q.shape
    o = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream().cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
            causal, scale, binding.ATTN_BF16, binding.ATTN_F32)
    if ws is None:
        st = binding.attn_fwd_raw(*args, stream)
    else:
        st = binding.attn_fwd_ws_raw(*args, ws, ws_bytes, stream)
    assert st == 0, binding.status_string(st)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("case", WS_CASES, ids=lambda c: "B%dH%dN%dd%d_%s" % (
    c[0], c[1], c[2], c[3], "causal" if c[4] else "full"))
def test_workspace_path(case):
    """attn_fwd_ws gives attn_fwd's bits whether or not it uses the
    workspace; the workspace then holds V in fp16 (torch's rounding) and
    nothing past it is written; the results meet the oracle."""
    B, H, N, d, causal = case
    _say("workspace case", case)
    qc, kc, vc = make_qkv(B, H, N, d, "bf16", 1.0, seed=11)
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    sc = _scale(d)
    need = binding.workspace_bytes(B, H, N, d, binding.ATTN_BF16)
    assert need == B * H * N * d * 2
    base_o, base_l = _raw(q, k, v, causal, sc)
    ws = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    o, lse = _raw(q, k, v, causal, sc, ws.data_ptr(), need)
    assert torch.equal(o, base_o) and torch.equal(lse, base_l)
    assert torch.equal(ws[:need].view(torch.float16).view(v.shape), v.to(torch.float16))
    assert bool((ws[need:] == 0x5A).all())
    # Too small or misaligned: ignored, same bits.
    for ptr, nbytes in ((ws.data_ptr(), need - 16), (ws.data_ptr() + 8, need)):
        o2, l2 = _raw(q, k, v, causal, sc, ptr, nbytes)
        assert torch.equal(o2, base_o) and torch.equal(l2, base_l)
    ref_o, ref_l = oracle.attn_oracle(qc, kc, vc, causal=causal, scale=sc)
    check_close(o.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "workspace " + str(case))
