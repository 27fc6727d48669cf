"""ctypes front end of the fp64 C oracles -- TEST INFRASTRUCTURE ONLY.

Builds ``attn_oracle.c`` (forward) and ``attn_bwd_oracle.c`` (backward) with
the host C compiler (no fast-math) into ``liboracle_attn.so`` and
``liboracle_attn_bwd.so`` next to this file and calls ``attn_oracle_rows`` /
``attn_bwd_oracle_rows``. Inputs may be any real tensors or arrays; they are
upcast to fp64 exactly (bf16, fp16 and fp32 values are all representable in
fp64).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_attn.so")
_BWD_SRC = os.path.join(_HERE, "attn_bwd_oracle.c")
_BWD_LIB = os.path.join(_HERE, "liboracle_attn_bwd.so")
_lib = None
_bwd_lib = None


def library_path():
    return _LIB


def bwd_library_path():
    return _BWD_LIB


def compile_oracle(src, out):
    """gcc -O2 -fopenmp, IEEE-exact (no fast-math, no FMA contraction)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _build_one(src, lib, force):
    if not force and os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(src):
        return lib
    return compile_oracle(src, lib)


def build_oracle(force=False):
    """Build both oracle libraries next to their sources (each skipped if up
    to date). Returns the forward library's path."""
    _build_one(_BWD_SRC, _BWD_LIB, force)
    return _build_one(_SRC, _LIB, force)


def open_oracle_library(path):
    lib = ctypes.CDLL(path)
    i64, dp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double)
    lib.attn_oracle_rows.restype = ctypes.c_int
    lib.attn_oracle_rows.argtypes = [dp, dp, dp, i64, i64, i64, i64, ctypes.c_int,
                                     ctypes.c_double, ctypes.POINTER(i64), i64,
                                     dp, dp, ctypes.c_int]
    lib.attn_oracle_rows_qk.restype = ctypes.c_int
    lib.attn_oracle_rows_qk.argtypes = [dp, dp, dp, i64, i64, i64, i64, i64, ctypes.c_int,
                                        ctypes.c_double, ctypes.POINTER(i64), i64,
                                        dp, dp, ctypes.c_int]
    lib.attn_oracle_max_threads.restype = ctypes.c_int
    return lib


def open_bwd_oracle_library(path):
    lib = ctypes.CDLL(path)
    i64, dp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(i64)
    lib.attn_bwd_oracle_rows_qk.restype = ctypes.c_int
    lib.attn_bwd_oracle_rows_qk.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, i64, ctypes.c_int,
                                            ctypes.c_double, ip, i64, dp, ip, i64, dp, dp,
                                            ctypes.c_int]
    lib.attn_bwd_oracle_rows.restype = ctypes.c_int
    lib.attn_bwd_oracle_rows.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, ctypes.c_int,
                                         ctypes.c_double, ip, i64, dp, ip, i64, dp, dp,
                                         ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        build_oracle()
        _lib = open_oracle_library(_LIB)
    return _lib


def _load_bwd():
    global _bwd_lib
    if _bwd_lib is None:
        build_oracle()
        _bwd_lib = open_bwd_oracle_library(_BWD_LIB)
    return _bwd_lib


def oracle_threads():
    """OpenMP threads the oracle uses by default."""
    return int(_load().attn_oracle_max_threads())


def _as_f64(x):
    if hasattr(x, "detach"):  # torch tensor: exact upcast on the CPU
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def attn_oracle(q, k, v, causal=False, scale=None, rows=None, nthreads=0, lib=None):
    """fp64 attention of [B,H,Nq,d] queries over [B,H,Nk,d] keys and values
    (Nq and Nk may differ when not causal).

    scale: the softmax scale; None means 1/sqrt(d). Pass the exact value the
           GPU path receives (e.g. the fp32 number) to compare like for like.
    rows:  optional flat row ids (b*H + h)*N + i; then O is [len(rows), d]
           and LSE is [len(rows)]. Without rows O is [B,H,N,d], LSE [B,H,N].
    lib:   another build of attn_oracle.c (used by the tests that check the
           pins catch planted mistakes); default: this package's build.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape or k.shape[:2] + k.shape[3:] != \
            q.shape[:2] + q.shape[3:]:
        raise ValueError("q [B,H,Nq,d] and k, v [B,H,Nk,d] must agree in B, H and d")
    B, H, N, d = q.shape
    Nk = k.shape[2]
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
    if Nk == N:
        st = lib.attn_oracle_rows(q.ctypes.data_as(dp), k.ctypes.data_as(dp),
                                  v.ctypes.data_as(dp), B, H, N, d, int(bool(causal)),
                                  float(scale), rows_ptr, nrows, o.ctypes.data_as(dp),
                                  lse.ctypes.data_as(dp), int(nthreads))
    else:
        st = lib.attn_oracle_rows_qk(q.ctypes.data_as(dp), k.ctypes.data_as(dp),
                                     v.ctypes.data_as(dp), B, H, N, Nk, d, int(bool(causal)),
                                     float(scale), rows_ptr, nrows, o.ctypes.data_as(dp),
                                     lse.ctypes.data_as(dp), int(nthreads))
    if st != 0:
        raise RuntimeError("attn_oracle_rows failed with status %d" % st)
    return o, lse


def _rows_arg(rows, total):
    if rows is None:
        return None, total, None
    arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    return arr, arr.size, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def attn_bwd_oracle(q, k, v, dout, causal=False, scale=None, qrows=None, krows=None,
                    nthreads=0, lib=None):
    """fp64 gradients (dQ, dK, dV) of attention of [B,H,Nq,d] queries over
    [B,H,Nk,d] keys and values for the upstream gradient dout [B,H,Nq,d]
    (Nq and Nk may differ when not causal).

    scale: the forward's softmax scale; None means 1/sqrt(d).
    qrows: optional flat query row ids (b*H + h)*N + i; dQ is then
           [len(qrows), d] (an empty list skips dQ). Default: all rows,
           dQ [B,H,N,d].
    krows: the same for the key rows of dK and dV.
    lib:   another build of attn_bwd_oracle.c (mutant tests).
    """
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    if q.ndim != 4 or k.ndim != 4 or dout.shape != q.shape or v.shape != k.shape or \
            (k.shape[0], k.shape[1], k.shape[3]) != (q.shape[0], q.shape[1], q.shape[3]):
        raise ValueError("q, dout [B,H,Nq,d] and k, v [B,H,Nk,d] must agree in B, H and d")
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lib = lib or _load_bwd()
    qa, nq, qp = _rows_arg(qrows, B * H * N)
    ka, nk, kp = _rows_arg(krows, B * H * Nk)
    dq = np.empty((nq, d), dtype=np.float64)
    dk = np.empty((nk, d), dtype=np.float64)
    dv = np.empty((nk, d), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    if Nk == N:
        st = lib.attn_bwd_oracle_rows(q.ctypes.data_as(dp), k.ctypes.data_as(dp),
                                      v.ctypes.data_as(dp), dout.ctypes.data_as(dp), B, H, N, d,
                                      int(bool(causal)), float(scale), qp, nq,
                                      dq.ctypes.data_as(dp), kp, nk, dk.ctypes.data_as(dp),
                                      dv.ctypes.data_as(dp), int(nthreads))
    else:
        st = lib.attn_bwd_oracle_rows_qk(q.ctypes.data_as(dp), k.ctypes.data_as(dp),
                                         v.ctypes.data_as(dp), dout.ctypes.data_as(dp), B, H, N,
                                         Nk, d, int(bool(causal)), float(scale), qp, nq,
                                         dq.ctypes.data_as(dp), kp, nk, dk.ctypes.data_as(dp),
                                         dv.ctypes.data_as(dp), int(nthreads))
    if st != 0:
        raise RuntimeError("attn_bwd_oracle_rows failed with status %d" % st)
    if qrows is None:
        dq = dq.reshape(B, H, N, d)
    if krows is None:
        dk, dv = dk.reshape(B, H, Nk, d), dv.reshape(B, H, Nk, d)
    return dq, dk, dv
