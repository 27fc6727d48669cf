"""GPU parity of attn_row_softmax against the fp64 oracle (the pages' Kernel 2).

Tolerance from the arithmetic: fp32 throughout (exp on v_exp_f32, one
reciprocal per row), so each output is within a few fp32 roundings of the
exact value relative to its size: |err| <= 1e-5 |y| + 1e-7 (the page reports
~1e-7 absolute on its test). Outputs stored in bf16/fp16 add their rounding:
the unit roundoff u |y| (2^-8 bf16, 2^-11 fp16), and half the fp16 subnormal
spacing. Inputs are the seeded draws rounded to the input dtype; the
oracle receives the same rounded values."""
import os

import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_flash_amd import binding
from io_aware_attention_flash_amd import build as hipbuild

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
# Rounding to the output type: at most the unit roundoff u times |y| (RNE),
# plus half the subnormal spacing for fp16 (outputs below 2^-14).
ROUND = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}
SUBNORMAL = {"f32": 0.0, "bf16": 0.0, "f16": 2.0 ** -25}


def setup_module(module):
    hipbuild.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _x(M, N, dt, sigma, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(M, N, generator=g) * sigma).to(DT[dt])


def _check(y, x, out, what):
    ref = oracle.row_softmax(x)
    got = y.cpu().double().numpy()
    err = np.abs(got - ref)
    tol = 1e-5 * np.abs(ref) + 1e-7 + ROUND[out] * np.abs(ref) + SUBNORMAL[out]
    worst = float((err / tol).max())
    print("%s: max|err| %.2e worst err/tol %.3f" % (what, err.max(), worst), flush=True)
    assert np.all(np.isfinite(got)) and worst <= 1.0, what


SHAPES = [
    # (M, N, dtype, sigma): the page's test shape and the 2000-column bug case first
    (1823, 781, "f32", 1.0), (4, 5, "f32", 1.0), (3, 2000, "f32", 1.0),
    (7, 1, "bf16", 1.0), (33, 63, "f16", 2.0), (64, 512, "bf16", 1.0),
    (17, 4096, "bf16", 3.0), (9, 4097, "f16", 1.0), (5, 16384, "f32", 1.0),
    (3, 16385, "bf16", 1.0), (2, 70001, "f16", 1.0), (300, 1024, "f16", 1.0),
    # one 16-wave row per workgroup: 16-byte loads up to 65536, element loads up to 32768
    (4, 20000, "f16", 1.0), (2, 65536, "bf16", 2.0), (3, 32767, "f32", 1.0),
    # two passes, 16-byte loads
    (2, 70000, "bf16", 1.0),
    # one wave up to 2048 16-bit / 1024 fp32 columns, four waves up to 8192 / 4096
    (6, 2048, "bf16", 1.0), (5, 2056, "bf16", 1.0), (7, 2049, "f16", 1.0),
    (3, 8192, "f16", 1.0), (3, 8200, "bf16", 1.0), (9, 1024, "f32", 1.0),
    (9, 1028, "f32", 1.0), (4, 4096, "f32", 2.0), (4, 4100, "f32", 1.0),
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "M%dN%d_%s_s%g" % c)
def test_row_softmax(case):
    M, N, dt, sigma = case
    print("case", case, flush=True)
    x = _x(M, N, dt, sigma, seed=41)
    for out in sorted({dt, "f32"}):
        y = binding.row_softmax(x.to(DEV), out_dtype=DT[out])
        torch.cuda.synchronize()
        _check(y, x, out, "%s -> %s" % (case, out))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_strided_rows(dt):
    """Rows further apart than N (a column slice of a wider matrix), with odd
    N (element loads) and with N a multiple of the 16-byte piece."""
    for N, pad in ((781, 13), (1024, 64)):
        x = _x(40, N, dt, 1.0, seed=42)
        xg = torch.zeros(40, N + pad, dtype=DT[dt], device=DEV)
        xg[:, :N] = x.to(DEV)
        xv = xg[:, :N]
        ybuf = torch.zeros(40, N + 8, dtype=DT[dt], device=DEV)
        y = binding.row_softmax(xv, out=ybuf[:, :N])
        torch.cuda.synchronize()
        _check(y, x, dt, "strided N=%d pad=%d %s" % (N, pad, dt))
        assert torch.count_nonzero(ybuf[:, N:]) == 0, "wrote past the row"


def test_large_logits_and_inf():
    """Entries of -inf get 0, a dominant entry gets 1, and +-1e4 shifts do
    not overflow."""
    x = torch.zeros(3, 300)
    x[0, 7] = 1e4
    x[1, :] = -1e4
    x[1, 5] = 0.0
    x[2, 100:] = float("-inf")
    y = binding.row_softmax(x.to(DEV)).cpu()
    assert y[0, 7].item() == 1.0 and torch.count_nonzero(y[0]) == 1
    assert y[1, 5].item() == 1.0
    assert torch.all(y[2, 100:] == 0) and abs(y[2, :100].sum().item() - 1.0) <= 1e-6


@pytest.mark.parametrize("M,N,dt", [(1 << 19, 8192, "bf16"), (1 << 18, 16384, "f32")],
                         ids=["M524288N8192_bf16", "M262144N16384_f32"])
def test_offsets_past_2_31(M, N, dt):
    """2^32 elements in one matrix: the element offsets of the later rows pass
    2^31 (byte offsets 2^32). Rows on both sides of the crossing and the last
    row against the oracle; inputs come from torch's seeded generator on the
    GPU and only the compared rows are copied back. (Offsets within a row stay
    below N <= 2^30; the row base is 64-bit.)"""
    print("offsets past 2^31", (M, N, dt), flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(43)
    x = torch.randn((M, N), generator=gen, device=DEV, dtype=DT[dt])
    y = binding.row_softmax(x, out_dtype=DT[dt])
    torch.cuda.synchronize()
    cross = (1 << 31) // N
    for r in sorted({0, max(cross - 1, 0), min(cross, M - 1), M - 1}):
        _check(y[r:r + 1], x[r:r + 1].cpu(), dt, "row %d of %d" % (r, M))
    del x, y
    torch.cuda.empty_cache()


def _random_cases(n, seed=2027):
    rng = np.random.default_rng(seed)
    pairs = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"), ("f16", "f32")]
    cases = []
    for i in range(n):
        M = int(rng.integers(1, 300))
        N = int(round(np.exp(rng.uniform(0.0, np.log(150000.0)))))
        if N * M > (1 << 25):
            M = max(1, (1 << 25) // N)
        tin, tout = pairs[int(rng.integers(0, len(pairs)))]
        pad = int(rng.choice([0, 0, 8, 13]))  # extra row stride (elements) of x and y
        cases.append((i, M, N, tin, tout, pad, float(rng.choice([1.0, 3.0]))))
    return cases


@pytest.mark.parametrize("case", _random_cases(40),
                         ids=lambda c: "%02d_M%dN%d_%s_%s_pad%d_s%g" % c)
def test_row_softmax_random(case):
    """Seeded draws of M, N (log-uniform up to 150000: every kernel shape and
    both passes), dtype pair and row padding (16-byte pieces or element
    loads), against the oracle."""
    i, M, N, tin, tout, pad, sigma = case
    print("case", case, flush=True)
    x = _x(M, N, tin, sigma, seed=500 + i)
    xg = torch.zeros(M, N + pad, dtype=DT[tin], device=DEV)
    xg[:, :N] = x.to(DEV)
    ybuf = torch.zeros(M, N + pad, dtype=DT[tout], device=DEV)
    y = binding.row_softmax(xg[:, :N], out_dtype=DT[tout], out=ybuf[:, :N])
    torch.cuda.synchronize()
    _check(y, x, tout, "random %s" % (case,))
    if pad:
        assert torch.count_nonzero(ybuf[:, N:]) == 0, "wrote past the row"
