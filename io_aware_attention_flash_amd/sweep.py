"""Offline sweep of the kernels' compile-time configurations: the gfx950
counterpart of the pages' autotuning ("4.4 Writing GPU Kernels with Triton",
sections "Sizing the attention kernel" and "Autotuning": time a list of
tile configurations per problem size and keep the best).

Triton compiles a configuration when it is first called. Here the tile
shapes are compile-time constants of hand-written kernels, so the
alternatives are built ahead of time: each knob below is a -D macro whose
default is the configuration the library ships. `build` compiles one library
per alternative (on any host: hipcc cross-compiles for gfx950); `run` times
the alternatives against the default on the GPU, interleaved in one process,
and compares their outputs with the default's.

    python -m io_aware_attention_flash_amd.sweep build [--knobs K ...]
    python -m io_aware_attention_flash_amd.sweep run [--knobs K ...] [--write PATH]

Libraries go to build/sweep/ at the repository root; results to
build/sweep/results.json, and with --write to a markdown table.
"""
import argparse
import concurrent.futures
import ctypes
import json
import os
import time

from . import build as hipbuild

SWEEP_DIR = os.path.join(hipbuild.ROOT, "build", "sweep")

# knob -> the macro, its values (the first is what the library ships: a number,
# or a label when the shipped value depends on the head dimension), the pass
# that exercises it and the workloads it is timed on.
KNOBS = {
    "fwd_tile_d128": dict(macro=("ATTN_CFG_FWD_WAVES_D128", "ATTN_CFG_FWD_BN_D128"),
                          values=["dispatch", "8x64", "8x32", "4x32"], pass_="fwd",
                          workloads=["b2h32_n4096_d128_bf16_causal",
                                     "b1h16_n16384_d128_bf16_sigma3_causal",
                                     "b4h16_n1024_d128_bf16", "b8h12_n3000_d128_bf16",
                                     "b1h8_n2048_d128_bf16_causal"],
                          what="forward tile at d=128: waves per workgroup (32 query rows "
                               "each) x keys per K/V tile (shipped: chosen per problem between "
                               "8x64 and 4x32 by a round-count cost model)"),
    "fwd_tile_d64": dict(macro=("ATTN_CFG_FWD_WAVES_D64", "ATTN_CFG_FWD_BN_D64"),
                         values=["dispatch", "4x128", "4x64", "8x128", "8x64"], pass_="fwd",
                         workloads=["b8h12_n3000_d64_f16", "b4h16_n1024_d64_bf16",
                                    "b4h16_n2048_d64_bf16", "b2h16_n8192_d64_bf16",
                                    "b2h16_n4096_d64_bf16_causal", "b1h16_n16384_d64_bf16_causal",
                                    "b8h16_n512_d64_bf16_causal"],
                         what="forward tile at d=64: waves per workgroup x keys per K/V tile "
                              "(shipped: chosen per problem between 8x128 and 4x64 by a "
                              "round-count cost model)"),
    "fwd_causal_short_first": dict(macro="ATTN_CFG_CAUSAL_SHORT_FIRST", values=[0, 1, 2],
                                   pass_="fwd",
                                   workloads=["b2h32_n4096_d128_bf16_causal",
                                              "b1h16_n16384_d128_bf16_sigma3_causal"],
                                   what="causal workgroups run their short query tile first "
                                        "(1), their long one (0), or alternate by pair (2)"),
    "fwd_head_blocked": dict(macro="ATTN_CFG_HEAD_BLOCKED", values=[0, 1], pass_="fwd",
                             workloads=["b2h32_n4096_d128_bf16_causal",
                                        "b1h16_n16384_d128_bf16_sigma3_causal",
                                        "b8h12_n3000_d64_f16", "b4h16_n1024_d64_bf16"],
                             what="heads of one XCD: every eighth one (0) or a block of B*H/8 "
                                  "adjacent ones (1)"),
    "fwd_causal_pairs": dict(macro="ATTN_CFG_CAUSAL_PAIRS", values=[1, 0], pass_="fwd",
                             workloads=["b2h32_n4096_d128_bf16_causal",
                                        "b1h16_n16384_d128_bf16_sigma3_causal"],
                             what="causal workgroups take pairs of query tiles (1) or one tile "
                                  "each, longest first (0)"),
    "fwd_o_nontemporal": dict(macro="ATTN_CFG_O_NONTEMPORAL", values=[1, 0], pass_="fwd",
                              workloads=["b2h32_n4096_d128_bf16_causal",
                                         "b8h12_n3000_d64_f16"],
                              what="stores of O with the non-temporal hint (1) or plain (0)"),
    "fwd_q_nontemporal": dict(macro="ATTN_CFG_Q_NONTEMPORAL", values=[0, 1], pass_="fwd",
                              workloads=["b2h32_n4096_d128_bf16_causal",
                                         "b1h16_n16384_d128_bf16_sigma3_causal",
                                         "b8h12_n3000_d64_f16"],
                              what="copies of the query tile with the non-temporal hint (1) or "
                                   "plain (0)"),
    "bwd_nontemporal": dict(macro="ATTN_CFG_BWD_NONTEMPORAL", values=[0, 1], pass_="bwd",
                            workloads=["b2h32_n4096_d128_bf16_causal", "b8h12_n3000_d64_f16"],
                            what="the backward's gradient stores with the non-temporal hint (1) "
                                 "or plain (0)"),
    "strided_tuned": dict(macro="ATTN_CFG_STRIDED_TUNED", values=[1, 0], pass_="general",
                          workloads=["b2h32_n4096_d128_bf16_causal", "b8h12_n3000_d64_f16",
                                     "b4h16_n1024_d64_bf16"],
                          what="strided self-attention at d = 64 or 128 (bf16/fp16) on the tuned "
                               "kernels (1) or on the general kernel (0)"),
    "gen_o_nontemporal": dict(macro="ATTN_CFG_GEN_O_NONTEMPORAL", values=[0, 1], pass_="general",
                              workloads=["b2h32_n4096_d128_bf16_causal", "b8h12_n3000_d64_f16"],
                              base_defs=["-DATTN_CFG_STRIDED_TUNED=0"],
                              what="the general kernel's stores of O with the non-temporal hint "
                                   "(1) or plain (0)"),
    "fwd_lookahead": dict(macro="ATTN_CFG_LOOKAHEAD", values=[3, 2, 4], pass_="fwd",
                          workloads=["b2h32_n4096_d128_bf16_causal",
                                     "b1h16_n16384_d128_bf16_sigma3_causal"],
                          what="LDS operand reads issued this many MFMA steps ahead"),
    "fwd_rescale_log2": dict(macro="ATTN_CFG_RESCALE_LOG2", values=[8, 0, 4], pass_="fwd",
                             workloads=["b2h32_n4096_d128_bf16_causal",
                                        "b1h16_n16384_d128_bf16_sigma3_causal"],
                             what="lazy rescale: rescale only when the row maximum grows by "
                                  "more than 2^value (0: whenever it grows)"),
    "fwd_prepass_min_n": dict(macro="ATTN_CFG_PREPASS_MIN_N", values=[8192, 4096, 1 << 30],
                              pass_="fwd_ws",
                              workloads=["b2h32_n4096_d128_bf16_causal",
                                         "b1h32_n8192_d128_bf16_causal",
                                         "b1h16_n16384_d128_bf16_sigma3_causal"],
                              what="bf16 V converted to fp16 by a first pass from this N on "
                                   "(2^30: never)"),
    "bwd_o_nontemporal": dict(macro="ATTN_CFG_BWD_O_NONTEMPORAL", values=[0, 1], pass_="bwd",
                              workloads=["b2h32_n4096_d128_bf16_causal", "b8h12_n3000_d64_f16",
                                         "b4h16_n1024_d64_bf16"],
                              what="the dQ kernel's loads of O (read once, for D) with the "
                                   "non-temporal hint (1) or plain (0)"),
    "bwd_dq_tile_k": dict(macro="ATTN_CFG_BWD_DQ_TILE_K", values=[64, 32, 128], pass_="bwd",
                          workloads=["b2h32_n4096_d128_bf16_causal",
                                     "b8h12_n3000_d64_f16"],
                          what="keys per step of the backward's dQ kernel"),
    "bwd_dkdv_waves": dict(macro="ATTN_CFG_BWD_DKDV_WAVES", values=[4, 8],
                           pass_="bwd",
                           workloads=["b2h32_n4096_d128_bf16_causal",
                                      "b1h16_n16384_d128_bf16_sigma3_causal",
                                      "b4h16_n1024_d128_bf16", "b8h12_n3000_d128_bf16"],
                           what="waves per dK/dV workgroup at d=128 (32 keys each)"),
    "sm_nontemporal": dict(macro="ATTN_CFG_SM_NONTEMPORAL", values=[1, 0], pass_="softmax",
                           workloads=["sm_m32768_n4096_bf16", "sm_m8192_n16384_bf16",
                                      "sm_m32768_n4096_f32"],
                           what="the row softmax's one-pass loads and stores with the "
                                "non-temporal hint (1) or plain (0)"),
    "sm_f32_vpl": dict(macro="ATTN_CFG_SM_F32_VPL_MAX", values=[16, 32, 64], pass_="softmax",
                       workloads=["sm_m32768_n4096_f32", "sm_m65536_n2048_f32",
                                  "sm_m8192_n16384_f32", "sm_m16384_n8192_f32"],
                       what="fp32 values per lane a one- or four-wave softmax row holds "
                            "(fewer: more waves per row)"),
    "sm_packed": dict(macro="ATTN_CFG_SM_PACKED", values=[0, 1], pass_="softmax",
                      workloads=["sm_m32768_n4096_bf16", "sm_m8192_n16384_bf16",
                                 "sm_m4096_n65536_f16", "sm_m16384_n32768_bf16",
                                 "sm_m262144_n512_bf16"],
                      what="16-bit softmax rows held packed as loaded, each exponential "
                           "taken twice (1), or held as fp32 exponentials (0)"),
    "sm_h_vpl": dict(macro="ATTN_CFG_SM_H_VPL_MAX", values=[32, 64, 16], pass_="softmax",
                     workloads=["sm_m32768_n4096_bf16", "sm_m65536_n2048_bf16",
                                "sm_m8192_n16384_bf16", "sm_m262144_n512_bf16",
                                "sm_m16384_n8192_f16"],
                     what="16-bit values per lane a one- or four-wave softmax row holds "
                          "(fewer: more waves per row)"),
    "bwd_lookahead": dict(macro="ATTN_CFG_BWD_LOOKAHEAD", values=[2, 1], pass_="bwd",
                          workloads=["b2h32_n4096_d128_bf16_causal", "b8h12_n3000_d64_f16"],
                          what="MFMA steps by which the backward's LDS operand reads run ahead "
                               "(3 spills)"),
    "gen_lookahead": dict(macro="ATTN_CFG_GEN_LOOKAHEAD", values=[2, 1, 3], pass_="general",
                          workloads=["b2h32_n4096_d128_bf16_causal", "b4h16_n1024_d64_bf16"],
                          base_defs=["-DATTN_CFG_STRIDED_TUNED=0"],
                          what="MFMA steps by which the general kernel's LDS operand reads run "
                               "ahead"),
    "gen_tile_k": dict(macro="ATTN_CFG_GEN_TILE_K", values=["32@d128/64@d64", 32, 64, 128],
                       pass_="general",
                       workloads=["b2h32_n4096_d128_bf16_causal", "b8h12_n3000_d64_f16"],
                       base_defs=["-DATTN_CFG_STRIDED_TUNED=0"],
                       what="keys per step of the general-layout forward"),
}


def variant_name(knob, value):
    """The shipped library for a knob's first value, unless the knob sets
    base_defs (flags every variant of it is built with, e.g. to time the
    general kernel on shapes the tuned kernels would otherwise take): then a
    library of its own."""
    if value == KNOBS[knob]["values"][0]:
        return "%s_base" % knob if KNOBS[knob].get("base_defs") else "default"
    return "%s_%s" % (knob, value)


def variant_defs(knob, value):
    """-D flags of one value: a number for a one-macro knob, or "AxB" for a
    knob over a pair of macros; plus the knob's base_defs."""
    macro = KNOBS[knob]["macro"]
    base = list(KNOBS[knob].get("base_defs", []))
    if isinstance(value, str) and "x" not in value:
        return base  # the library's own per-problem choice
    if isinstance(macro, tuple):
        return base + ["-D%s=%s" % (m, x) for m, x in zip(macro, str(value).split("x"))]
    return base + ["-D%s=%d" % (macro, value)]


def _alternatives(knob):
    """The values of a knob that need a build of their own: all but the
    shipped one, and the first too when the knob sets base_defs."""
    vals = KNOBS[knob]["values"]
    return vals if KNOBS[knob].get("base_defs") else vals[1:]


def lib_path(name):
    return os.path.join(SWEEP_DIR, "lib_%s.so" % name)


def _build_one(name, defs):
    out = lib_path(name)
    t0 = time.time()
    hipbuild.build(extra=defs, out=out, jobs=2)
    return "built %-28s %s (%.0f s)" % (name, " ".join(defs) or "(shipped)", time.time() - t0)


def build_all(jobs=4, knobs=None):
    os.makedirs(SWEEP_DIR, exist_ok=True)
    todo = [("default", [])]
    for knob, k in KNOBS.items():
        if knobs and knob not in knobs:
            continue
        for v in _alternatives(knob):
            todo.append((variant_name(knob, v), variant_defs(knob, v)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for msg in ex.map(lambda t: _build_one(*t), todo):
            print(msg, flush=True)


class SoftmaxWorkload:
    """An M x N row-softmax problem, named sm_m<M>_n<N>_<dtype>."""

    def __init__(self, name):
        m, n, dt = name.split("_")[1:]
        self.name, self.M, self.N, self.dtype = name, int(m[1:]), int(n[1:]), dt
        self.d = None


def _workload(name):
    from .inputs import WORKLOADS, Workload
    if name.startswith("sm_"):
        return SoftmaxWorkload(name)
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name == "b1h32_n8192_d128_bf16_causal":
        return Workload(name, 1, 32, 8192, 128, "bf16", True)
    if name == "b4h16_n1024_d128_bf16":
        return Workload(name, 4, 16, 1024, 128, "bf16", False)
    if name == "b2h16_n4096_d64_bf16_causal":
        return Workload(name, 2, 16, 4096, 64, "bf16", True)
    if name == "b8h12_n3000_d128_bf16":
        return Workload(name, 8, 12, 3000, 128, "bf16", False)
    if name == "b1h8_n2048_d128_bf16_causal":
        return Workload(name, 1, 8, 2048, 128, "bf16", True)
    if name == "b4h16_n2048_d64_bf16":
        return Workload(name, 4, 16, 2048, 64, "bf16", False)
    if name == "b2h16_n8192_d64_bf16":
        return Workload(name, 2, 16, 8192, 64, "bf16", False)
    if name == "b1h16_n16384_d64_bf16_causal":
        return Workload(name, 1, 16, 16384, 64, "bf16", True)
    if name == "b8h16_n512_d64_bf16_causal":
        return Workload(name, 8, 16, 512, 64, "bf16", True)
    raise KeyError(name)


def _runner(lib, w, pass_, tensors):
    """A zero-argument function that enqueues one call of `pass_` through
    the library `lib` on the prepared tensors."""
    import torch
    from . import binding
    q, k, v, o, lse, dout, grads, ws, qs = tensors
    dt = {"bf16": binding.ATTN_BF16, "f16": binding.ATTN_F16, "f32": binding.ATTN_F32}[w.dtype]
    stream = torch.cuda.current_stream().cuda_stream
    if pass_ == "softmax":  # q is x, o is y
        return lambda: lib.attn_row_softmax(q.data_ptr(), w.N, o.data_ptr(), w.N, w.M, w.N, dt,
                                            dt, stream)
    if pass_ == "fwd":
        return lambda: lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), w.B, w.H, w.N, w.d, int(w.causal), w.scale, dt,
                                    binding.ATTN_F32, stream)
    if pass_ == "fwd_ws":
        need = lib.attn_fwd_workspace_bytes(w.B, w.H, w.N, w.d, dt)
        ptr = ws.data_ptr() if need else None
        return lambda: lib.attn_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), w.B, w.H, w.N, w.d, int(w.causal), w.scale,
                                       dt, binding.ATTN_F32, ptr, ws.numel(), stream)
    if pass_ == "bwd":
        nws = lib.attn_bwd_workspace_bytes(w.B, w.H, w.N, w.d)
        return lambda: lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), dout.data_ptr(), grads[0].data_ptr(),
                                    grads[1].data_ptr(), grads[2].data_ptr(), w.B, w.H, w.N, w.d,
                                    int(w.causal), w.scale, dt, binding.ATTN_F32,
                                    binding.ATTN_F32, ws.data_ptr(), nws, stream)
    if pass_ == "general":
        sq = (ctypes.c_int64 * 3)(*qs[0].stride()[:3])
        return lambda: lib.attn_fwd_strided(qs[0].data_ptr(), sq, qs[1].data_ptr(), sq,
                                            qs[2].data_ptr(), sq, o.data_ptr(), None,
                                            lse.data_ptr(), w.B, w.H, w.N, w.N, w.d,
                                            int(w.causal), w.scale, dt, binding.ATTN_F32, stream)
    raise ValueError(pass_)


def _softmax_input(w):
    """x ~ N(0, 1), seeded, in the workload's dtype (on the CPU)."""
    import torch
    g = torch.Generator().manual_seed(1)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    return torch.randn(w.M, w.N, generator=g).to(tdt)


def _time_and_compare(knob, kn, wl, names, calls, out, rounds, target_ms):
    """Time every variant's call interleaved (median of `rounds` alternating
    rounds of ~target_ms each), then compare each one's outputs with the
    shipped library's. Returns one result row per variant."""
    import torch

    def timed(n, count):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(count):
            calls[n]()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / count

    ms1 = timed(names[0], 3)
    per = max(3, int(target_ms / max(ms1, 1e-3)))
    for n in names:  # warm every variant, then time them in alternating order
        timed(n, per)
    times = {n: [] for n in names}
    for r in range(rounds):
        for n in (names if r % 2 == 0 else names[::-1]):
            times[n].append(timed(n, per))
    rows, ref = [], None
    base = sorted(times[names[0]])[rounds // 2]
    for n in names:
        for x in out:
            x.zero_()
        assert calls[n]() == 0
        torch.cuda.synchronize()
        got = [x.clone() for x in out]
        if ref is None:
            ref = got
        diff = max(float((a.float() - b.float()).abs().max()) for a, b in zip(got, ref))
        med = sorted(times[n])[len(times[n]) // 2]
        rows.append(dict(knob=knob, macro=kn["macro"], value=kn["values"][names.index(n)],
                         shipped=n == names[0], workload=wl, pass_=kn["pass_"],
                         us=med * 1e3, rel=base / med - 1.0, max_abs_diff_vs_shipped=diff))
        print("%-18s %-10s %-40s %9.1f us  %+6.2f%%  diff %.1e" % (
            knob, rows[-1]["value"], wl, med * 1e3, 100 * rows[-1]["rel"], diff), flush=True)
    return rows


def run_all(rounds=8, target_ms=60.0, knobs=None):
    import torch
    from . import binding
    from .inputs import make_dout, workload_qkv
    results = []
    for knob, kn in KNOBS.items():
        if knobs and knob not in knobs:
            continue
        names = [variant_name(knob, v) for v in kn["values"]]
        libs = {n: binding.load_library(lib_path(n)) for n in names}
        for wl in kn["workloads"]:
            w = _workload(wl)
            dev = torch.device("cuda:0")
            if kn["pass_"] == "softmax":
                x = _softmax_input(w).to(dev)
                y = torch.empty_like(x)
                tensors = (x, None, None, y, None, None, None, None, None)
                calls = {n: _runner(libs[n], w, "softmax", tensors) for n in names}
                results += _time_and_compare(knob, kn, wl, names, calls, [y], rounds, target_ms)
                continue
            q, k, v = (x.to(dev) for x in workload_qkv(w, seed=0))
            dout = make_dout(w.B, w.H, w.N, w.d, w.dtype, seed=0).to(dev)
            o = torch.empty(q.shape, dtype=torch.float32, device=dev)
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
            grads = [torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3)]
            nws = max(w.B * w.H * w.N * w.d * 2, w.B * w.H * w.N * 8) + 256
            ws = torch.empty(nws, dtype=torch.uint8, device=dev)
            qs = [x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v)]
            if kn["pass_"] == "bwd":  # the backward's O and LSE, from the shipped forward
                assert libs[names[0]].attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                               o.data_ptr(), lse.data_ptr(), w.B, w.H, w.N, w.d,
                                               int(w.causal), w.scale,
                                               {"bf16": 2, "f16": 1}[w.dtype], 0,
                                               torch.cuda.current_stream().cuda_stream) == 0
            tensors = (q, k, v, o, lse, dout, grads, ws, qs)
            calls = {n: _runner(libs[n], w, kn["pass_"], tensors) for n in names}
            out = grads if kn["pass_"] == "bwd" else [o, lse]
            results += _time_and_compare(knob, kn, wl, names, calls, out, rounds, target_ms)
    with open(os.path.join(SWEEP_DIR, "results.json"), "w") as f:
        json.dump(results, f, indent=1)
    return results


def markdown(results):
    lines = ["| knob (macro) | value | pass | workload | µs | vs shipped | max abs diff vs shipped |",
             "|---|---|---|---|---|---|---|"]
    for r in results:
        macro = r["macro"] if isinstance(r["macro"], str) else " x ".join(r["macro"])
        lines.append("| %s (`%s`) | %s%s | %s | %s | %.1f | %+.2f%% | %.1e |" % (
            r["knob"], macro, r["value"], " (shipped)" if r["shipped"] else "", r["pass_"],
            r["workload"], r["us"], 100 * r["rel"], r["max_abs_diff_vs_shipped"]))
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("what", choices=["build", "run"])
    ap.add_argument("--write", help="markdown file for the results table (run)")
    ap.add_argument("--jobs", type=int, default=4, help="parallel compilations (build)")
    ap.add_argument("--knobs", nargs="*", choices=list(KNOBS), help="only these knobs")
    args = ap.parse_args(argv)
    if args.what == "build":
        build_all(args.jobs, args.knobs)
        return
    res = run_all(knobs=args.knobs)
    table = markdown(res)
    print(table)
    if args.write:
        with open(args.write, "w") as f:
            f.write(table + "\n")


if __name__ == "__main__":
    main()
