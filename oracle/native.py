"""ctypes front end of the fp64 C oracle -- TEST INFRASTRUCTURE ONLY.

Builds ``attn_oracle.c`` with the host C compiler (no fast-math) into
``liboracle_attn.so`` next to this file and calls ``attn_oracle_rows``.
Inputs may be any real tensors or arrays; they are upcast to fp64 exactly
(bf16, fp16 and fp32 values are all representable in fp64).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_attn.so")
_lib = None


def library_path():
    return _LIB


def compile_oracle(src, out):
    """gcc -O2 -fopenmp, IEEE-exact (no fast-math, no FMA contraction)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_oracle(force=False):
    """Build liboracle_attn.so next to its source (skipped if up to date)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    return compile_oracle(_SRC, _LIB)


def open_oracle_library(path):
    lib = ctypes.CDLL(path)
    i64, dp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double)
    lib.attn_oracle_rows.restype = ctypes.c_int
    lib.attn_oracle_rows.argtypes = [dp, dp, dp, i64, i64, i64, i64, ctypes.c_int,
                                     ctypes.c_double, ctypes.POINTER(i64), i64,
                                     dp, dp, ctypes.c_int]
    lib.attn_oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build_oracle()
        _lib = open_oracle_library(_LIB)
    return _lib


def oracle_threads():
    """OpenMP threads the oracle uses by default."""
    return int(_load().attn_oracle_max_threads())


def _as_f64(x):
    if hasattr(x, "detach"):  # torch tensor: exact upcast on the CPU
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def attn_oracle(q, k, v, causal=False, scale=None, rows=None, nthreads=0, lib=None):
    """fp64 attention of [B,H,N,d] inputs.

    scale: the softmax scale; None means 1/sqrt(d). Pass the exact value the
           GPU path receives (e.g. the fp32 number) to compare like for like.
    rows:  optional flat row ids (b*H + h)*N + i; then O is [len(rows), d]
           and LSE is [len(rows)]. Without rows O is [B,H,N,d], LSE [B,H,N].
    lib:   another build of attn_oracle.c (used by the tests that check the
           pins catch planted mistakes); default: this package's build.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B,H,N,d] shape")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lib = lib or _load()
    dp = ctypes.POINTER(ctypes.c_double)
    if rows is None:
        nrows = B * H * N
        rows_ptr = None
        o = np.empty((B, H, N, d), dtype=np.float64)
        lse = np.empty((B, H, N), dtype=np.float64)
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
        rows_ptr = rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        o = np.empty((nrows, d), dtype=np.float64)
        lse = np.empty((nrows,), dtype=np.float64)
    st = lib.attn_oracle_rows(q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp),
                              B, H, N, d, int(bool(causal)), float(scale), rows_ptr, nrows,
                              o.ctypes.data_as(dp), lse.ctypes.data_as(dp), int(nthreads))
    if st != 0:
        raise RuntimeError("attn_oracle_rows failed with status %d" % st)
    return o, lse
