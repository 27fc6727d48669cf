"""The entry points captured in a HIP graph (torch.cuda.CUDAGraph) and replayed,
and run on two streams at once.

The C entry points only enqueue kernels on the caller's stream (no
allocation, no memset, no synchronisation), so a caller may capture them in
a graph and replay it instead of launching each time. Each case captures one
call on tensors it owns, then three times: writes new inputs into those
tensors, replays the graph, runs the same call eagerly into other outputs,
synchronises, and requires the replay to equal the eager result bit for bit
(the kernels are deterministic). The eager result itself is held to the
oracle by the parity tests; here the first eager run is also checked against
the oracle on a few rows, so a graph that replayed nothing cannot pass.
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_attention_flash_amd import binding
from io_aware_attention_flash_amd import build as hipbuild
from io_aware_attention_flash_amd.inputs import make_dout, make_qkv

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def setup_module(module):
    hipbuild.ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _scale(d):
    return float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))


def _capture(fn):
    """Warm fn up on a side stream, then capture one call of it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays(g, refill, graph_out, eager, what):
    for r in range(3):
        refill(100 + r)
        g.replay()
        got = [x.clone() for x in graph_out]
        want = eager()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.isfinite(b).all(), "%s replay %d output %d: non-finite" % (what, r, i)
            assert torch.equal(a, b), "%s replay %d output %d: max diff %.3e" % (
                what, r, i, float((a.double() - b.double()).abs().max()))
        print("%s: replay %d equals the eager call" % (what, r), flush=True)


def _rows_vs_oracle(q, k, v, causal, scale, o, lse, rows):
    """Rows of the first head against the oracle (the parity bar)."""
    qc, kc, vc = q[:1, :1].cpu(), k[:1, :1].cpu(), v[:1, :1].cpu()
    ref_o, ref_l = oracle.attn_oracle(qc, kc, vc, causal=causal, scale=scale, rows=rows)
    got_o = o[0, 0].cpu().double().numpy()[rows]
    got_l = lse[0, 0].cpu().double().numpy()[rows]
    assert np.abs(got_o - ref_o).max() <= 1e-2
    assert np.abs(got_l - ref_l).max() <= 1e-3


@pytest.mark.parametrize("B,H,N,d,dt,causal", [
    (2, 4, 1000, 128, "bf16", True),
    (1, 2, 8192, 128, "bf16", True),   # first pass into a caller's workspace
    (2, 3, 777, 64, "f16", False),
])
def test_forward_graph(B, H, N, d, dt, causal):
    dev = torch.device("cuda:0")
    scale = _scale(d)
    q, k, v = (x.to(dev) for x in make_qkv(B, H, N, d, dt, 1.0, seed=41))
    o = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    need = binding.workspace_bytes(B, H, N, d, binding.ATTN_BF16 if dt == "bf16" else
                                   binding.ATTN_F16)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None

    def call(out, l):
        binding.attn_fwd(q, k, v, causal=causal, scale=scale, out_dtype=torch.float32, out=out,
                         lse=l, workspace=ws)

    g = _capture(lambda: call(o, lse))
    _rows_vs_oracle(q, k, v, causal, scale, o, lse, np.array([0, 1, N // 2, N - 1]))

    def refill(seed):
        for dst, src in zip((q, k, v), make_qkv(B, H, N, d, dt, 1.0, seed=seed)):
            dst.copy_(src.to(dev))

    def eager():
        o2, l2 = torch.empty_like(o), torch.empty_like(lse)
        call(o2, l2)
        return o2, l2

    _replays(g, refill, (o, lse), eager, "forward %s" % ((B, H, N, d, dt, causal),))


def test_general_forward_graph():
    """Strided [B, N, H, d] views with a key length unlike the query length."""
    dev = torch.device("cuda:0")
    B, H, Nq, Nk, d = 2, 3, 300, 517, 96
    scale = _scale(d)
    q4 = torch.empty((B, Nq, H, d), dtype=torch.bfloat16, device=dev)
    k4 = torch.empty((B, Nk, H, d), dtype=torch.bfloat16, device=dev)
    v4 = torch.empty((B, Nk, H, d), dtype=torch.bfloat16, device=dev)
    q, k, v = (x.transpose(1, 2) for x in (q4, k4, v4))

    def refill(seed):
        q_, _, _ = make_qkv(B, H, Nq, d, "bf16", 1.0, seed=seed)
        _, k_, v_ = make_qkv(B, H, Nk, d, "bf16", 1.0, seed=seed + 1)
        q.copy_(q_.to(dev)), k.copy_(k_.to(dev)), v.copy_(v_.to(dev))

    refill(7)
    o = torch.empty((B, H, Nq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)

    def call(out, l):
        binding.attn_fwd(q, k, v, causal=False, scale=scale, out_dtype=torch.float32, out=out,
                         lse=l)

    g = _capture(lambda: call(o, lse))

    def eager():
        o2, l2 = torch.empty_like(o), torch.empty_like(lse)
        call(o2, l2)
        return o2, l2

    _replays(g, refill, (o, lse), eager, "general forward")


@pytest.mark.parametrize("noalloc", [False, True])
def test_backward_graph(noalloc):
    """attn_bwd with a caller's workspace, and attn_bwd_noalloc (static scratch)."""
    dev = torch.device("cuda:0")
    B, H, N, d, dt, causal = 2, 4, 1000, 128, "bf16", True
    scale = _scale(d)
    q, k, v = (x.to(dev) for x in make_qkv(B, H, N, d, dt, 1.0, seed=61))
    dout = make_dout(B, H, N, d, dt, seed=61).to(dev)
    o, lse = binding.attn_fwd(q, k, v, causal=causal, scale=scale, out_dtype=torch.float32)
    ws_bytes = binding.bwd_workspace_bytes(B, H, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    grads = [torch.empty(x.shape, dtype=torch.float32, device=dev) for x in (q, k, v)]
    stream_of = lambda: torch.cuda.current_stream().cuda_stream

    def call(gs):
        if noalloc:
            st = binding.attn_bwd_noalloc_raw(
                q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                dout.data_ptr(), *[x.data_ptr() for x in gs], B, H, N, N, d, causal, scale,
                binding.ATTN_BF16, binding.ATTN_F32, binding.ATTN_F32, stream_of())
            assert st == 0, binding.status_string(st)
        else:
            binding.attn_bwd(q, k, v, o, lse, dout, causal=causal, scale=scale,
                             grad_dtype=torch.float32, workspace=ws, grads=gs)

    g = _capture(lambda: call(grads))

    def refill(seed):
        for dst, src in zip((q, k, v), make_qkv(B, H, N, d, dt, 1.0, seed=seed)):
            dst.copy_(src.to(dev))
        dout.copy_(make_dout(B, H, N, d, dt, seed=seed).to(dev))
        binding.attn_fwd(q, k, v, causal=causal, scale=scale, out_dtype=torch.float32, out=o,
                         lse=lse)

    def eager():
        gs = [torch.empty_like(x) for x in grads]
        call(gs)
        return gs

    _replays(g, refill, grads, eager, "backward (noalloc=%s)" % noalloc)


def test_two_streams_at_once():
    """The library keeps no per-call state: a forward and backward on one
    stream and a forward on another, enqueued alternately so that they can
    overlap on the GPU, give the same bits as the same calls made one after
    another on the current stream."""
    dev = torch.device("cuda:0")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    qa, ka, va = (x.to(dev) for x in make_qkv(2, 4, 1000, 128, "bf16", 1.0, seed=71))
    da = make_dout(2, 4, 1000, 128, "bf16", seed=71).to(dev)
    qb, kb, vb = (x.to(dev) for x in make_qkv(2, 3, 777, 64, "f16", 1.0, seed=72))
    sca, scb = _scale(128), _scale(64)

    def run_a():
        o, lse = binding.attn_fwd(qa, ka, va, causal=True, scale=sca, out_dtype=torch.float32)
        g = binding.attn_bwd(qa, ka, va, o, lse, da, causal=True, scale=sca,
                             grad_dtype=torch.float32)
        return [o, lse, *g]

    def run_b():
        return list(binding.attn_fwd(qb, kb, vb, causal=False, scale=scb,
                                     out_dtype=torch.float32))

    want_a, want_b = run_a(), run_b()
    torch.cuda.synchronize()
    got = []
    for _ in range(3):
        with torch.cuda.stream(sa):
            ga = run_a()
        with torch.cuda.stream(sb):
            gb = run_b()
        got.append((ga, gb))
    torch.cuda.synchronize()
    for r, (ga, gb) in enumerate(got):
        for i, (x, y) in enumerate(zip(ga + gb, want_a + want_b)):
            assert torch.equal(x, y), "round %d output %d differs" % (r, i)
    print("two streams: 3 rounds equal the sequential calls", flush=True)
