"""Host logic of the tile-configuration sweep (io_aware_attention_flash_amd/sweep.py):
the -D flags and library names of every variant, without building or timing
anything. Each knob names macros the kernel sources define with #ifndef, so a
variant's flag really overrides a shipped default."""
import os
import re

import pytest

from io_aware_attention_flash_amd import build as hipbuild
from io_aware_attention_flash_amd import sweep

SOURCES = "".join(open(p).read() for p in hipbuild.SRCS)


def _macros(knob):
    m = sweep.KNOBS[knob]["macro"]
    return m if isinstance(m, tuple) else (m,)


@pytest.mark.parametrize("knob", list(sweep.KNOBS))
def test_knob_macros_are_overridable(knob):
    for m in _macros(knob):
        assert "#ifndef %s" % m in SOURCES, m


@pytest.mark.parametrize("knob", list(sweep.KNOBS))
def test_variant_names_and_flags(knob):
    kn = sweep.KNOBS[knob]
    vals = kn["values"]
    names = [sweep.variant_name(knob, v) for v in vals]
    assert len(set(names)) == len(names), "every value needs a library of its own"
    base = kn.get("base_defs", [])
    if base:
        assert names[0] == "%s_base" % knob
        assert sweep._alternatives(knob) == vals
    else:
        assert names[0] == "default"
        assert sweep._alternatives(knob) == vals[1:]
    for v in vals:
        defs = sweep.variant_defs(knob, v)
        assert defs[:len(base)] == list(base)
        rest = defs[len(base):]
        if isinstance(v, str) and "x" not in v:
            assert rest == []  # the library's own choice: no override
        else:
            assert len(rest) == len(_macros(knob))
            for flag, m in zip(rest, _macros(knob)):
                assert flag.startswith("-D%s=" % m)
        for flag in defs:
            assert re.fullmatch(r"-D[A-Z0-9_]+=-?\d+", flag), flag


def test_pair_knob_values_split_into_both_macros():
    assert sweep.variant_defs("fwd_tile_d128", "4x32") == [
        "-DATTN_CFG_FWD_WAVES_D128=4", "-DATTN_CFG_FWD_BN_D128=32"]


def test_general_kernel_knobs_time_the_general_kernel():
    # the strided self-attention shapes they time now run on the tuned kernels
    # unless the variant turns that routing off
    for knob in ("gen_lookahead", "gen_tile_k", "gen_o_nontemporal"):
        for v in sweep.KNOBS[knob]["values"]:
            assert "-DATTN_CFG_STRIDED_TUNED=0" in sweep.variant_defs(knob, v)


def test_workloads_resolve():
    for knob, kn in sweep.KNOBS.items():
        for wl in kn["workloads"]:
            w = sweep._workload(wl)
            if kn["pass_"] == "softmax":
                assert w.name == wl and w.M >= 1 and w.N >= 1 and w.dtype in ("bf16", "f16", "f32")
                assert "sm_m%d_n%d_%s" % (w.M, w.N, w.dtype) == wl
            else:
                assert w.name == wl and w.d in (64, 128)


def test_markdown_table():
    rows = [dict(knob="fwd_lookahead", macro="ATTN_CFG_LOOKAHEAD", value=3, shipped=True,
                 workload="w", pass_="fwd", us=100.0, rel=0.0, max_abs_diff_vs_shipped=0.0),
            dict(knob="fwd_lookahead", macro="ATTN_CFG_LOOKAHEAD", value=2, shipped=False,
                 workload="w", pass_="fwd", us=110.0, rel=100.0 / 110.0 - 1,
                 max_abs_diff_vs_shipped=0.0)]
    md = sweep.markdown(rows).splitlines()
    assert md[0].startswith("| knob (macro) |") and len(md) == 4
    assert "3 (shipped)" in md[2] and "-9.09%" in md[3]


def test_library_paths_stay_in_the_build_tree():
    p = sweep.lib_path("default")
    assert os.path.dirname(p) == sweep.SWEEP_DIR
    assert sweep.SWEEP_DIR.startswith(hipbuild.ROOT)
