"""The C ABI on a host without a GPU: the library loads, exports every
function include/attn.h declares, agrees with the header's constants, and
rejects bad arguments before making any HIP call."""
import ctypes
import os
import re

import pytest

from io_aware_attention_flash_amd import binding
from io_aware_attention_flash_amd import build as hipbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    if hipbuild.is_stale():
        hipbuild.build()
    return binding.load_library()


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def _header_enum(name):
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"\b(%s_[A-Z0-9_]+)\s*=\s*(\d+)" % name, text)}


def test_exports_every_declared_function(lib):
    declared = _header_functions()
    assert set(declared) == set(binding.EXPORTS)
    for fn in declared:
        assert hasattr(lib, fn), "library does not export %s" % fn


def test_exported_symbols_are_c_linkage():
    out = os.popen("nm -D --defined-only %s" % binding.LIB_PATH).read()
    syms = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for fn in _header_functions():
        assert fn in syms


def test_header_constants_match_binding():
    st = _header_enum("ATTN_ERR")
    st["ATTN_OK"] = 0
    assert {v: k for k, v in st.items()} == binding.STATUS
    dt = {k: v for k, v in _header_enum("ATTN").items() if k in ("ATTN_F32", "ATTN_F16", "ATTN_BF16")}
    assert dt == {"ATTN_F32": binding.ATTN_F32, "ATTN_F16": binding.ATTN_F16,
                  "ATTN_BF16": binding.ATTN_BF16}
    ver = int(re.search(r"#define ATTN_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert binding.load_library().attn_abi_version() == ver


def test_status_strings(lib):
    for code in range(7):
        s = binding.status_string(code)
        assert isinstance(s, str) and s
    assert binding.status_string(0) == "ok"
    assert binding.status_string(99) == "unknown status"
    assert lib.attn_last_hip_error() == 0


# Fake, never-dereferenced addresses: validation fails before any use.
P = 0x1000


@pytest.mark.parametrize("args,code", [
    # null pointers
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(o=0), 1), (dict(lse=0), 1),
    # shapes
    (dict(B=0), 2), (dict(H=0), 2), (dict(N=0), 2), (dict(N=-5), 2),
    (dict(N=(1 << 24) + 1), 2), (dict(B=1 << 12, H=(1 << 12) + 1), 2),
    # head dims and dtype pairs
    (dict(d=32), 3), (dict(d=96), 3), (dict(d=0), 3), (dict(d=256), 3),
    (dict(i=0, o_t=1), 3), (dict(i=0, o_t=2), 3), (dict(i=1, o_t=2), 3),
    (dict(i=2, o_t=1), 3), (dict(i=3, o_t=3), 3), (dict(i=2, o_t=7), 3),
    # scale
    (dict(scale=float("nan")), 4), (dict(scale=float("inf")), 4),
    (dict(scale=float("-inf")), 4), (dict(scale=-0.125), 4),
])
def test_error_paths_need_no_gpu(lib, args, code):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=64, causal=0, scale=0.125,
             i=2, o_t=2)
    a.update(args)
    st = binding.attn_fwd_raw(a["q"] or None, a["k"] or None, a["v"] or None, a["o"] or None,
                              a["lse"] or None, a["B"], a["H"], a["N"], a["d"], a["causal"],
                              a["scale"], a["i"], a["o_t"])
    assert st == code, (args, st)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library(str(tmp_path / "nope.so"))


def test_package_import_loads_nothing():
    import io_aware_attention_flash_amd as pkg
    assert callable(pkg.attn_fwd)
    assert ctypes is not None


@pytest.mark.parametrize("B,H,N,d,dt,want", [
    (1, 1, 8192, 128, 2, 8192 * 128 * 2),
    (2, 3, 8192, 64, 2, 2 * 3 * 8192 * 64 * 2),
    (1, 16, 16384, 128, 2, 16 * 16384 * 128 * 2),
    (1, 1, 8191, 128, 2, 0),          # shorter sequences convert inside the kernel
    (1, 1, 8192, 128, 1, 0),          # fp16 V needs no conversion
    (1, 1, 8192, 128, 0, 0),
    (1, 1, 8192, 96, 2, 0),           # invalid arguments give 0
    (0, 1, 8192, 128, 2, 0),
    (1, 1, (1 << 24) + 1, 128, 2, 0),
])
def test_workspace_bytes(lib, B, H, N, d, dt, want):
    assert binding.workspace_bytes(B, H, N, d, dt) == want


@pytest.mark.parametrize("args,code", [
    (dict(q=0), 1), (dict(lse=0), 1), (dict(N=0), 2), (dict(d=96), 3),
    (dict(i=2, o_t=1), 3), (dict(scale=float("nan")), 4),
])
def test_workspace_entry_validates_first(lib, args, code):
    """attn_fwd_ws validates exactly like attn_fwd, before any HIP call,
    with or without a workspace."""
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=8192, d=128, causal=0, scale=0.125,
             i=2, o_t=0)
    a.update(args)
    for ws, nbytes in ((None, 0), (P, 1 << 30)):
        st = binding.attn_fwd_ws_raw(a["q"] or None, a["k"] or None, a["v"] or None,
                                     a["o"] or None, a["lse"] or None, a["B"], a["H"], a["N"],
                                     a["d"], a["causal"], a["scale"], a["i"], a["o_t"], ws, nbytes)
        assert st == code, (args, ws, st)


@pytest.mark.parametrize("B,H,N,d,want", [
    (2, 32, 4096, 128, 2 * 32 * 4096 * 8),
    (1, 1, 1, 64, 256),                 # rounded up to 256 bytes
    (1, 3, 77, 64, 256 * ((3 * 77 * 8 + 255) // 256)),
    (1, 1, 128, 96, 1024),              # any multiple of 8 up to 128
    (1, 1, 128, 100, 0), (1, 1, 128, 136, 0), (0, 1, 128, 64, 0), (1, 1, (1 << 24) + 1, 64, 0),
])
def test_bwd_workspace_bytes(lib, B, H, N, d, want):
    assert binding.bwd_workspace_bytes(B, H, N, d) == want


@pytest.mark.parametrize("args,code", [
    # null pointers
    (dict(q=0), 1), (dict(o=0), 1), (dict(lse=0), 1), (dict(do=0), 1), (dict(dq=0), 1),
    (dict(dk=0), 1), (dict(dv=0), 1),
    # shapes
    (dict(B=0), 2), (dict(N=0), 2), (dict(N=(1 << 24) + 1), 2),
    # head dims and dtypes: d not a multiple of 8 in [8, 128]; fp32 inputs with
    # a 16-bit O or gradients; O or gradient types outside {in, F32}
    (dict(d=100), 3), (dict(d=136), 3), (dict(d=0), 3), (dict(i=0, o_t=2, g_t=0), 3),
    (dict(i=0, o_t=0, g_t=1), 3), (dict(i=2, o_t=1), 3), (dict(i=1, g_t=2), 3), (dict(i=5), 3),
    # scale
    (dict(scale=float("nan")), 4), (dict(scale=-1.0), 4),
    # workspace: missing, too small, misaligned
    (dict(ws=0), 6), (dict(ws_bytes=100), 6), (dict(ws=P + 8), 6),
])
def test_bwd_error_paths_need_no_gpu(lib, args, code):
    """attn_bwd rejects every bad argument before any HIP call (each case
    here is invalid, so nothing is launched)."""
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=1, N=128, d=64,
             causal=0, scale=0.125, i=2, o_t=0, g_t=0, ws=P, ws_bytes=1 << 20)
    a.update(args)
    st = binding.attn_bwd_raw(a["q"] or None, a["k"] or None, a["v"] or None, a["o"] or None,
                              a["lse"] or None, a["do"] or None, a["dq"] or None, a["dk"] or None,
                              a["dv"] or None, a["B"], a["H"], a["N"], a["d"], a["causal"],
                              a["scale"], a["i"], a["o_t"], a["g_t"], a["ws"] or None, a["ws_bytes"])
    assert st == code, (args, st)


@pytest.mark.parametrize("args,code", [
    (dict(q=0), 1), (dict(v=0), 1), (dict(lse=0), 1),
    (dict(Nq=0), 2), (dict(Nk=0), 2), (dict(causal=1, Nk=64), 2),
    (dict(d=0), 3), (dict(d=4), 3), (dict(d=100), 3), (dict(d=136), 3),
    (dict(i=0, o_t=2), 3), (dict(i=2, o_t=1), 3),
    (dict(q=P + 8), 3),                                   # misaligned base
    (dict(q_st=(-4096, 4096, 64)), 3),                    # negative stride
    (dict(k_st=(1 << 20, 1 << 14, 32)), 3),               # row stride < d
    (dict(v_st=(1 << 20, 1 << 14, 68)), 3),               # row not 16-byte aligned (bf16)
    (dict(o_st=(4096, 0, 64)), 3),                        # output heads alias (stride 0)
    (dict(o_st=(4096, 32, 64)), 3),                       # output heads overlap (stride < d)
    (dict(o_st=(4096, 64, 64)), 3),                       # head and row strides equal
    (dict(scale=float("nan")), 4),
])
def test_strided_error_paths_need_no_gpu(lib, args, code):
    """attn_fwd_strided rejects every bad argument before any HIP call (each
    case here is invalid, so nothing is launched)."""
    a = dict(q=P, k=P, v=P, o=P, lse=P, q_st=None, k_st=None, v_st=None, o_st=None, B=1, H=2,
             Nq=32, Nk=48, d=64, causal=0, scale=0.125, i=2, o_t=0)
    a.update(args)
    st = binding.attn_fwd_strided_raw(a["q"] or None, a["q_st"], a["k"] or None, a["k_st"],
                                      a["v"] or None, a["v_st"], a["o"] or None, a["o_st"],
                                      a["lse"] or None, a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                                      a["causal"], a["scale"], a["i"], a["o_t"])
    assert st == code, (args, st)


@pytest.mark.parametrize("args,code", [
    (dict(x=0), 1), (dict(y=0), 1),
    (dict(M=0), 2), (dict(N=0), 2), (dict(xs=10), 2), (dict(ys=10), 2),
    (dict(N=(1 << 30) + 1, xs=(1 << 31), ys=(1 << 31)), 2),
    (dict(i=0, o=2), 3), (dict(i=2, o=1), 3), (dict(i=7, o=7), 3),
    (dict(x=P + 1), 3),                          # not aligned to its element size
])
def test_row_softmax_error_paths_need_no_gpu(lib, args, code):
    a = dict(x=P, xs=64, y=P, ys=64, M=4, N=64, i=2, o=2)
    a.update(args)
    st = binding.row_softmax_raw(a["x"] or None, a["xs"], a["y"] or None, a["ys"], a["M"], a["N"],
                                 a["i"], a["o"])
    assert st == code, (args, st)


@pytest.mark.parametrize("args,code", [
    (dict(Nk=0), 2), (dict(Nq=0), 2), (dict(causal=1), 2),   # causal needs Nq == Nk
    (dict(d=100), 3), (dict(ws=0), 6),
])
def test_bwd_qk_error_paths_need_no_gpu(lib, args, code):
    a = dict(B=1, H=1, Nq=64, Nk=80, d=64, causal=0, ws=P)
    a.update(args)
    st = binding.attn_bwd_qk_raw(P, P, P, P, P, P, P, P, P, a["B"], a["H"], a["Nq"], a["Nk"],
                                 a["d"], a["causal"], 0.125, 2, 0, 0, a["ws"] or None, 1 << 20)
    assert st == code, (args, st)


@pytest.mark.parametrize("args,code", [
    (dict(q=0), 1), (dict(dv=0), 1),
    (dict(Nq=0), 2), (dict(causal=1), 2),                    # causal needs Nq == Nk
    (dict(d=100), 3), (dict(i=0, o_t=2, g_t=0), 3),
    (dict(scale=-1.0), 4),
    # B*H*Nq rows of 8 bytes beyond the 16 MiB static scratch (2^21 rows)
    (dict(B=2, H=16, Nq=(1 << 16) + 1, Nk=128), 7), (dict(B=1, H=1, Nq=(1 << 21) + 1, Nk=64), 7),
])
def test_bwd_noalloc_error_paths_need_no_gpu(lib, args, code):
    """attn_bwd_noalloc checks its arguments, and the size of the problem
    against its static scratch, before any HIP call."""
    a = dict(q=P, dv=P, B=1, H=1, Nq=64, Nk=80, d=64, causal=0, scale=0.125, i=2, o_t=0, g_t=0)
    a.update(args)
    st = binding.attn_bwd_noalloc_raw(a["q"] or None, P, P, P, P, P, P, P, a["dv"] or None, a["B"],
                                      a["H"], a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"],
                                      a["i"], a["o_t"], a["g_t"])
    assert st == code, (args, st)
    assert "static scratch" in binding.status_string(7)


@pytest.mark.parametrize("args,code", [
    (dict(q=0), 1), (dict(dk=0), 1),
    (dict(Nq=0), 2), (dict(causal=1), 2),
    (dict(d=12), 3), (dict(i=0, o_t=2), 3),
    (dict(q=P + 8), 3),                                   # misaligned base
    (dict(q_st=(-4096, 4096, 64)), 3),                    # negative stride
    (dict(k_st=(1 << 20, 1 << 14, 32)), 3),               # row stride < d
    (dict(v_st=(1 << 20, 1 << 14, 68)), 3),               # row not 16-byte aligned (bf16)
    (dict(dq_st=(1 << 20, 1 << 14, 66)), 3),              # gradient row not aligned (fp32)
    (dict(o_st=(1 << 47, 1 << 14, 64)), 3),               # offsets beyond 2^47 elements
    (dict(do_st=(1 << 30, 1 << 24, 1 << 23)), 3),         # 128 rows span >= 2^31 bytes
    (dict(dq_st=(1 << 20, 0, 64)), 3),                    # gradient heads alias (stride 0)
    (dict(dq_st=(0, 1 << 14, 64)), 3),                    # gradient batches alias (B = 2)
    (dict(scale=float("nan")), 4),
    (dict(ws=0), 6),
])
def test_bwd_strided_error_paths_need_no_gpu(lib, args, code):
    """attn_bwd_strided rejects every bad argument before any HIP call (each
    case here is invalid, so nothing is launched)."""
    a = dict(q=P, dk=P, q_st=None, k_st=None, v_st=None, o_st=None, do_st=None, dq_st=None,
             B=2, H=2, Nq=64, Nk=80, d=64, causal=0, scale=0.125, i=2, o_t=0, g_t=0, ws=P)
    a.update(args)
    st = binding.attn_bwd_strided_raw(a["q"] or None, a["q_st"], P, a["k_st"], P, a["v_st"], P,
                                      a["o_st"], P, P, a["do_st"], P, a["dq_st"], a["dk"] or None,
                                      None, P, None, a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                                      a["causal"], a["scale"], a["i"], a["o_t"], a["g_t"],
                                      a["ws"] or None, 1 << 20)
    assert st == code, (args, st)
