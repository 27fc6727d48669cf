"""Benchmark of the attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--out-dtype f32|in] [--no-cpu-baseline] [--pass fwd|bwd]

A step is one attn_fwd call (the whole forward: QK^T, masking, online
softmax, P.V, normalisation, LSE) over one batch of seeded synthetic input
that is already resident in HBM. W untimed steps, then exactly K timed steps
bracketed by torch.cuda.synchronize(); the kernel duration comes from HIP
events recorded on the stream the kernel is launched on.

The defaults (200 warm-up launches, 1000 timed) measure the sustained rate.
The kernel draws the board's full power: coming out of idle, the first few
launches run at a high clock, then the power controller pulls the clock down
hard for some tens of launches before settling. Timing a few dozen launches
right after a short warm-up lands in that dip and reads about 15% slow.

Prints one JSON line. FLOPs count the two N x N x d contractions per head,
halved when causal: 4*B*H*N^2*d (/2). Algorithmic bytes read Q, K, V once
and write O and LSE once.

--pass bwd times the backward instead (one attn_bwd call per step, all of
its launches, with O and LSE from one untimed forward). Its FLOPs count the
five contractions of the backward (S recomputed, dP, dV, dK, dQ), 2.5x the
forward's; the atomic-free split recomputes S and dP in its dQ kernel, so it
executes 1.4x that count.
"""
import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from io_aware_attention_flash_amd import binding  # noqa: E402
from io_aware_attention_flash_amd import build as hipbuild  # noqa: E402
from io_aware_attention_flash_amd.inputs import HEADLINE, WORKLOADS, make_dout, workload_qkv  # noqa: E402

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}  # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd TFLOP/s + % bf16 MFMA peak (causal, N=4096, d=128)"
KERNEL_SRC = os.path.join(ROOT, "io_aware_attention_flash_amd", "csrc", "attn_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def kernel_source_digest(text=None):
    """sha256[:16] of attn_fwd.hip's code: comments, trailing blanks and
    empty lines removed, so an edit of the comments keeps recorded counters
    valid and any edit of the code voids them."""
    src = open(KERNEL_SRC).read() if text is None else text
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = "\n".join(line.rstrip() for line in src.splitlines() if line.strip())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def measured_traffic(workload, out_dtype):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs, or None when absent or taken on a different kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = rec.get("entries", {}).get("%s/%s" % (workload, out_dtype))
    if not ent or ent.get("kernel_source_digest") != kernel_source_digest():
        return None
    return ent.get("hbm_bytes_per_launch")


def flushed_timing(step, stream, launches, flush_mb):
    """Per-launch times with the caches cold: before each launch, write a
    `flush_mb` MiB buffer (more than the 4 MB L2 of every XCD and the 256 MB
    Infinity Cache), then time that launch alone with events on its stream.
    Returns the median, the interquartile range and the extremes in ms."""
    buf = torch.empty(flush_mb << 20, dtype=torch.uint8, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    for i, (a, b) in enumerate(evs):
        buf.fill_(i & 0xFF)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)

    def q(f):
        x = f * (len(ts) - 1)
        lo = int(x)
        hi = min(lo + 1, len(ts) - 1)
        return ts[lo] + (ts[hi] - ts[lo]) * (x - lo)
    del buf
    return {"launches": launches, "flush_bytes": flush_mb << 20, "median_ms": round(q(0.5), 5),
            "p25_ms": round(q(0.25), 5), "p75_ms": round(q(0.75), 5),
            "iqr_ms": round(q(0.75) - q(0.25), 5), "min_ms": round(ts[0], 5),
            "max_ms": round(ts[-1], 5)}


def cpu_baseline(w, q, k, v, budget_s=12.0):
    """Time the fp64 oracle on whole heads of the same inputs until about
    `budget_s` seconds of CPU work; report the FLOP rate of that sample."""
    import numpy as np
    import oracle
    oracle.build_oracle()
    threads = oracle.oracle_threads()
    B, H, N, d = q.shape
    heads_done, flops, elapsed = 0, 0.0, 0.0
    for bh in range(B * H):
        b, h = divmod(bh, H)
        args = [x[b:b + 1, h:h + 1] for x in (q, k, v)]
        t0 = time.perf_counter()
        oracle.attn_oracle(*args, causal=w.causal, scale=w.scale)
        elapsed += time.perf_counter() - t0
        heads_done += 1
        n_keys = np.arange(1, N + 1, dtype=np.float64) if w.causal else np.full(N, float(N))
        flops += float(4.0 * d * n_keys.sum())
        if elapsed >= budget_s:
            break
    # Scale the sample's rate to the metric's FLOP convention (the causal
    # half-count); the sample's exact triangle count is what was executed.
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d heads of %s (fp64 three-pass oracle, %.1f s, %.3g FLOP)"
                      % (heads_done, B * H, w.name, elapsed, flops),
            "seconds": round(elapsed, 3)}


def cpu_baseline_bwd(w, q, k, v, dout, budget_s=12.0):
    """Time the fp64 backward oracle (dQ of every row, dK and dV of every key)
    on whole heads of the same inputs until about `budget_s` seconds."""
    import oracle
    oracle.build_oracle()
    threads = oracle.oracle_threads()
    B, H, N, d = q.shape
    heads_done, elapsed = 0, 0.0
    for bh in range(B * H):
        b, h = divmod(bh, H)
        args = [x[b:b + 1, h:h + 1] for x in (q, k, v, dout)]
        t0 = time.perf_counter()
        oracle.attn_bwd_oracle(*args, causal=w.causal, scale=w.scale)
        elapsed += time.perf_counter() - t0
        heads_done += 1
        if elapsed >= budget_s:
            break
    flops = w.bwd_flops() * heads_done / (B * H)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d heads of %s (fp64 backward oracle, %.1f s; rate on the "
                      "backward's five-contraction FLOP count)" % (heads_done, B * H, w.name, elapsed),
            "seconds": round(elapsed, 3)}


def bench_bwd(args):
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    if w.dtype not in ("bf16", "f16"):
        print("the backward supports bf16 and fp16 inputs only", file=sys.stderr)
        sys.exit(2)
    qc, kc, vc = workload_qkv(w, seed=0)
    dc = make_dout(w.B, w.H, w.N, w.d, w.dtype, seed=0)
    q, k, v, dout = qc.to(dev), kc.to(dev), vc.to(dev), dc.to(dev)
    o, lse = binding.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out_dtype=torch.float32)
    grads = [torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3)]
    ws = torch.empty(binding.bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8,
                     device=dev)

    def step():
        binding.attn_bwd(q, k, v, o, lse, dout, causal=w.causal, scale=w.scale,
                         grad_dtype=torch.float32, workspace=ws, grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = w.bwd_flops()
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    alg_bytes = w.bwd_algorithmic_bytes("f32", "f32")
    res = {
        "metric": "attention bwd TFLOP/s (five contractions%s)" % (", causal halved" if w.causal else ""),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0, sigma^2) Q/K/V, N(0, 1) dO)",
        "config": {"workload": w.name, "pass": "bwd", "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "in_dtype": w.dtype, "o_dtype": "f32", "grad_dtype": "f32",
                   "sigma": w.sigma, "scale": w.scale},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": None,
                     "scope": "whole attn_bwd call (prep + dK/dV + dQ launches)"},
        "hbm": {"algorithmic_bytes": alg_bytes,
                "achieved_GBps": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
                "peak_GBps": PEAK_HBM_GBS},
        "wall_s_timed_region": round(wall, 4),
        "flops_per_step": flops,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_bwd(w, qc, kc, vc, dc, args.cpu_budget)
    print(json.dumps(res), flush=True)


def bench_general(args):
    """The general-layout kernel (attn_fwd_strided) on the workload's shape,
    with Q, K, V as [B, N, H, d] tensors seen through [B, H, N, d] views (the
    layout a fused projection produces) and O written the same way."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    qc, kc, vc = workload_qkv(w, seed=0)
    q, k, v = (x.to(dev).transpose(1, 2).contiguous().transpose(1, 2) for x in (qc, kc, vc))
    assert not q.is_contiguous()
    obuf = torch.empty((w.B, w.N, w.H, w.d), dtype=torch.float32, device=dev)
    o = obuf.transpose(1, 2)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def step():
        binding.attn_fwd_general(q, k, v, causal=w.causal, scale=w.scale, out_dtype=torch.float32,
                                 out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    tflops = w.flops() / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    res = {"metric": "attention fwd TFLOP/s, general-layout kernel", "value": round(tflops, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded N(0, sigma^2) Q/K/V)",
           "config": {"workload": w.name, "pass": "fwd_general", "layout": "BNHD views",
                      "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                      "in_dtype": w.dtype, "out_dtype": "f32"},
           "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                        "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": None},
           "wall_s_timed_region": round(wall, 4), "flops_per_step": w.flops()}
    print(json.dumps(res), flush=True)


def bench_softmax(args):
    """attn_row_softmax on an M x N matrix (HBM-bound: one read, one write)."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M, N = args.sm_rows, args.sm_cols
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[args.sm_dtype]
    g = torch.Generator().manual_seed(0)
    xc = torch.randn(M, N, generator=g).to(tdt)
    x = xc.to(dev)
    y = torch.empty_like(x)

    def step():
        binding.row_softmax(x, out=y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    nbytes = 2 * M * N * x.element_size()
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"metric": "row softmax HBM GB/s (one read + one write)", "value": round(gbs, 1),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": args.sm_dtype, "data": "synthetic (seeded N(0, 1))",
           "config": {"workload": "row_softmax_m%d_n%d_%s" % (M, N, args.sm_dtype),
                      "pass": "softmax", "M": M, "N": N},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
           "wall_s_timed_region": round(wall, 4), "bytes_per_step": nbytes}
    if not args.no_cpu_baseline:
        import oracle
        rows = 0
        t1 = time.perf_counter()
        while rows < M and time.perf_counter() - t1 < args.cpu_budget:
            oracle.row_softmax(xc[rows:rows + 256])
            rows += min(256, M - rows)
        el = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": 2 * rows * N * x.element_size() / el / 1e9, "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": "%d of %d rows (fp64 NumPy oracle, %.1f s)" % (rows, M, el),
                               "seconds": round(el, 3)}
    print(json.dumps(res), flush=True)


class PowerSampler:
    """Board power and gfx clocks of GPU 0 while the timed launches run:
    amd-smi, polled 12 times in a child process (about 3.5 s). Its first
    reading can predate the load, so the summary takes the medians over the
    samples from 0.5 s after the start of the timed region to its end, and
    lists every sample (seconds from the start, W, mean gfx MHz over the
    XCDs). The timed region should outlast the sampling (say --steps 20000)."""

    CMD = ("for i in $(seq 1 12); do printf '%s ' $(date +%s.%N); "
           "amd-smi metric -p -c -g 0 --json 2>/dev/null | tr -d '\\n'; echo; sleep 0.25; done")
    LAG_S = 0.5

    def __init__(self):
        self.t0 = time.time()
        self.proc = subprocess.Popen(["bash", "-c", self.CMD], stdout=subprocess.PIPE,
                                     stderr=subprocess.DEVNULL, text=True)

    def stop(self):
        t1 = time.time()
        out, _ = self.proc.communicate(timeout=60)
        samples = []
        for line in out.splitlines():
            try:
                stamp, body = line.split(" ", 1)
                g = json.loads(body)
                g = g["gpu_data"][0] if isinstance(g, dict) else g[0]
                watts = float(g["power"]["socket_power"]["value"])
                mhz = [float(c["clk"]["value"]) for name, c in g["clock"].items()
                       if name.startswith("gfx_") and isinstance(c, dict) and
                       isinstance(c.get("clk"), dict)]
                samples.append((round(float(stamp) - self.t0, 2), watts,
                                round(sum(mhz) / len(mhz), 1) if mhz else None))
            except (ValueError, KeyError, IndexError, TypeError):
                continue
        loaded = [x for x in samples if self.LAG_S <= x[0] <= t1 - self.t0]

        def med(x):
            x = [v for v in x if v is not None]
            return sorted(x)[len(x) // 2] if x else None
        return {"tool": "amd-smi metric -p -c", "timed_s": round(t1 - self.t0, 2),
                "loaded_samples": len(loaded),
                "socket_power_w_median": med([x[1] for x in loaded]),
                "gfx_clock_mhz_median": med([x[2] for x in loaded]),
                "samples_s_w_mhz": samples}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "in"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", default="fwd",
                    choices=["fwd", "bwd", "fwd_general", "softmax"],
                    help="time the forward (default), the backward, the general-layout "
                         "forward on [B, N, H, d] views, or the row softmax")
    ap.add_argument("--sm-rows", type=int, default=32768)
    ap.add_argument("--sm-cols", type=int, default=4096)
    ap.add_argument("--sm-dtype", default="bf16", choices=["f32", "bf16", "f16"])
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--power", action="store_true",
                    help="forward: sample board power and gfx clocks with amd-smi during the "
                         "timed launches (use --steps 20000 or more for a few seconds of them)")
    ap.add_argument("--flush", type=int, default=0, metavar="LAUNCHES",
                    help="forward: after the timed region, also time LAUNCHES single launches "
                         "each preceded by a write of --flush-mb MiB (cold L2 and Infinity "
                         "Cache); report their median and interquartile range")
    ap.add_argument("--flush-mb", type=int, default=512)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB --steps times (reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": args.steps}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every (batch, head) is independent; see the sharding notes in the design doc). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    hipbuild.ensure_built()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.which == "bwd":
        bench_bwd(args)
        return
    if args.which == "fwd_general":
        bench_general(args)
        return
    if args.which == "softmax":
        bench_softmax(args)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = WORKLOADS[args.workload]
    qc, kc, vc = workload_qkv(w, seed=0)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    out_dtype = torch.float32 if args.out_dtype == "f32" else w.torch_dtype
    out_name = "f32" if args.out_dtype == "f32" else w.dtype
    o = torch.empty(q.shape, dtype=out_dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def step():
        binding.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out_dtype=out_dtype, out=o,
                         lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    sampler = PowerSampler() if args.power else None
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    power = sampler.stop() if sampler else None

    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    alg_bytes = w.algorithmic_bytes(out_name)
    traffic = measured_traffic(w.name, out_name)
    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0, sigma^2) Q/K/V)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "in_dtype": w.dtype, "out_dtype": out_name,
                   "sigma": w.sigma, "scale": w.scale},
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_TFLOPS["bf16"], 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": traffic},
        "hbm": {"algorithmic_bytes": alg_bytes,
                "achieved_GBps": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
                "peak_GBps": PEAK_HBM_GBS},
        "wall_s_timed_region": round(wall, 4),
        "flops_per_step": flops,
    }
    if w.causal:
        res["flops_exact_triangle_per_step"] = w.flops_exact_causal()
    if power is not None:
        res["power"] = power
    if args.flush > 0:
        fl = flushed_timing(step, stream, args.flush, args.flush_mb)
        fl["tflops_at_median"] = round(flops / (fl["median_ms"] * 1e-3) / 1e12, 2)
        res["flushed"] = fl
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, qc, kc, vc, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
