"""Thin ctypes binding of libattn_fwd.so (the C ABI in include/attn.h).

Argument marshalling only: every step of the attention forward and backward
runs in the library's HIP kernels. torch supplies the device buffers and the stream.
There is no fallback: if the library cannot be loaded the call raises.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# ATTN_LIB_PATH selects another build of the same library (e.g. a tile-configuration
# variant from sweep.py) for the process.
LIB_PATH = os.environ.get("ATTN_LIB_PATH") or os.path.join(_PKG, "libattn_fwd.so")

# attn_dtype / attn_status values of include/attn.h
ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
          4: "ATTN_ERR_SCALE", 5: "ATTN_ERR_HIP", 6: "ATTN_ERR_WORKSPACE", 7: "ATTN_ERR_CAPACITY"}
EXPORTS = ("attn_fwd", "attn_fwd_ws", "attn_fwd_workspace_bytes", "attn_fwd_strided", "attn_bwd",
           "attn_bwd_qk", "attn_bwd_noalloc", "attn_bwd_strided",
           "attn_bwd_workspace_bytes", "attn_row_softmax", "attn_status_string", "attn_abi_version",
           "attn_last_hip_error")

_TORCH_TO_ATTN = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}
_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, msg))
        self.status = status


def load_library(path=LIB_PATH):
    """Open the library and declare its signatures. Raises if it is missing."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("HIP attention library not built: %s is missing "
                           "(run python -m io_aware_attention_flash_amd.build)" % path)
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                             ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.attn_fwd_ws.restype = ctypes.c_int
    lib.attn_fwd_ws.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                ctypes.c_float, ctypes.c_int, ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.attn_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    i64p = ctypes.POINTER(i64)
    lib.attn_fwd_strided.restype = ctypes.c_int
    lib.attn_fwd_strided.argtypes = [vp, i64p, vp, i64p, vp, i64p, vp, i64p, vp, i64, i64, i64, i64,
                                     i64, ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                     vp]
    lib.attn_row_softmax.restype = ctypes.c_int
    lib.attn_row_softmax.argtypes = [vp, i64, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                             ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                             ctypes.c_size_t, vp]
    lib.attn_bwd_qk.restype = ctypes.c_int
    lib.attn_bwd_qk.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.attn_bwd_noalloc.restype = ctypes.c_int
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                     ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, vp]
    lib.attn_bwd_strided.restype = ctypes.c_int
    lib.attn_bwd_strided.argtypes = [vp, i64p, vp, i64p, vp, i64p, vp, i64p, vp, vp, i64p, vp, i64p,
                                     vp, i64p, vp, i64p, i64, i64, i64, i64, i64, ctypes.c_int,
                                     ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                     ctypes.c_size_t, vp]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_abi_version.restype = ctypes.c_int
    lib.attn_abi_version.argtypes = []
    lib.attn_last_hip_error.restype = ctypes.c_int
    lib.attn_last_hip_error.argtypes = []
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(status):
    return load_library().attn_status_string(int(status)).decode()


def attn_fwd_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, N, d, causal, scale,
                 in_dtype, out_dtype, stream=None):
    """Direct call of the C entry point with integer pointers; returns the status."""
    return load_library().attn_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, int(B), int(H), int(N),
                                   int(d), int(bool(causal)), float(scale), int(in_dtype),
                                   int(out_dtype), stream)


def attn_fwd_ws_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, N, d, causal, scale,
                    in_dtype, out_dtype, ws_ptr, ws_bytes, stream=None):
    """Direct call of attn_fwd_ws (caller-owned workspace); returns the status."""
    return load_library().attn_fwd_ws(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, int(B), int(H), int(N),
                                      int(d), int(bool(causal)), float(scale), int(in_dtype),
                                      int(out_dtype), ws_ptr, int(ws_bytes), stream)


def _strides(st):
    return None if st is None else (ctypes.c_int64 * 3)(*[int(x) for x in st])


def attn_fwd_strided_raw(q_ptr, q_st, k_ptr, k_st, v_ptr, v_st, o_ptr, o_st, lse_ptr, B, H, Nq,
                         Nk, d, causal, scale, in_dtype, out_dtype, stream=None):
    """Direct call of attn_fwd_strided; *_st are (b, h, row) element strides
    or None (contiguous). Returns the status."""
    return load_library().attn_fwd_strided(q_ptr, _strides(q_st), k_ptr, _strides(k_st), v_ptr,
                                           _strides(v_st), o_ptr, _strides(o_st), lse_ptr,
                                           int(B), int(H), int(Nq), int(Nk), int(d),
                                           int(bool(causal)), float(scale), int(in_dtype),
                                           int(out_dtype), stream)


def needs_general(q, k, v):
    """Whether a call needs the general-layout kernel (attn_fwd_strided):
    different query and key lengths, a head dim other than 64 or 128, or
    tensors that are not contiguous [B, H, N, d]."""
    return (k.shape[2] != q.shape[2] or q.shape[3] not in (64, 128) or
            not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()))


def attn_fwd_general(q, k, v, causal=False, scale=None, out_dtype=None, out=None, lse=None):
    """Attention forward through attn_fwd_strided: q [B, H, Nq, d], k and v
    [B, H, Nk, d], any strides with a unit column stride and 16-byte aligned
    rows, d a multiple of 8 up to 128. `out` may be a strided [B, H, Nq, d]
    view; lse is [B, H, Nq] contiguous."""
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or \
            (q.shape[0], q.shape[1], q.shape[3]) != (k.shape[0], k.shape[1], k.shape[3]):
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _TORCH_TO_ATTN:
        raise ValueError("q, k, v must share one dtype among float32/float16/bfloat16")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one GPU")
    if any(x.stride(3) != 1 for x in (q, k, v)):
        raise ValueError("the last dimension must be contiguous")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / d ** 0.5
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != out_dtype or out.stride(3) != 1 or out.device != q.device:
        raise ValueError("out must be a [B, H, Nq, d] tensor of out_dtype with a unit last stride")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous [B, H, Nq] float32 tensor")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_fwd_strided_raw(q.data_ptr(), q.stride()[:3], k.data_ptr(), k.stride()[:3],
                              v.data_ptr(), v.stride()[:3], out.data_ptr(), out.stride()[:3],
                              lse.data_ptr(), B, H, Nq, Nk, d, causal, scale,
                              _TORCH_TO_ATTN[q.dtype], _TORCH_TO_ATTN[out_dtype], stream)
    if st != 0:
        msg = status_string(st)
        if st == 5:
            msg += " (hipError_t %d)" % load_library().attn_last_hip_error()
        raise AttnError(st, msg)
    return out, lse


def workspace_bytes(B, H, N, d, in_dtype):
    """Bytes of device workspace attn_fwd_ws can use for this problem (0: none)."""
    return int(load_library().attn_fwd_workspace_bytes(int(B), int(H), int(N), int(d),
                                                       int(in_dtype)))


def attn_fwd(q, k, v, causal=False, scale=None, out_dtype=None, out=None, lse=None,
             workspace=None):
    """Attention forward of [B, H, N, d] tensors on the current HIP stream.

    Calls that need the general-layout kernel (different key length, a head
    dim other than 64 or 128, strided tensors) go to attn_fwd_general.

    scale defaults to 1/sqrt(d); out_dtype defaults to the input dtype
    (torch.float32 is also accepted for bf16/fp16 inputs). Returns (o, lse)
    with lse [B, H, N] fp32 natural-log logsumexp. Preallocated `out`/`lse`
    may be passed to avoid allocation. When the problem can use a device
    workspace (long bf16 sequences), a uint8 tensor of at least
    workspace_bytes(...) bytes may be passed as `workspace`; otherwise one is
    taken from torch's allocator for the call.
    """
    if q.dim() == 4 and k.dim() == 4 and needs_general(q, k, v) and \
            (out is None or out.stride(3) == 1):
        return attn_fwd_general(q, k, v, causal=causal, scale=scale, out_dtype=out_dtype, out=out,
                                lse=lse)
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must all be [B, H, N, d] of one shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _TORCH_TO_ATTN:
        raise ValueError("q, k, v must share one dtype among float32/float16/bfloat16")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, N, d]")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / d ** 0.5
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous [B, H, N, d] tensor of out_dtype on q's device")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous [B, H, N] float32 tensor on q's device")
    if out_dtype not in _TORCH_TO_ATTN:
        raise ValueError("unsupported out_dtype %s" % out_dtype)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    need = workspace_bytes(B, H, N, d, _TORCH_TO_ATTN[q.dtype])
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if not (workspace.is_cuda and workspace.device == q.device and workspace.is_contiguous()
                and workspace.numel() * workspace.element_size() >= need):
            raise ValueError("workspace must be a contiguous tensor of at least %d bytes on q's "
                             "device" % need)
        st = attn_fwd_ws_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, H, N, d, causal, scale, _TORCH_TO_ATTN[q.dtype],
                             _TORCH_TO_ATTN[out_dtype], workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), stream)
    else:
        st = attn_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          B, H, N, d, causal, scale, _TORCH_TO_ATTN[q.dtype],
                          _TORCH_TO_ATTN[out_dtype], stream)
    if st != 0:
        msg = status_string(st)
        if st == 5:
            msg += " (hipError_t %d)" % load_library().attn_last_hip_error()
        raise AttnError(st, msg)
    return out, lse


def attn_bwd_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, B, H, N, d,
                 causal, scale, in_dtype, o_dtype, grad_dtype, ws_ptr, ws_bytes, stream=None):
    """Direct call of attn_bwd with integer pointers; returns the status."""
    return load_library().attn_bwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr,
                                   dv_ptr, int(B), int(H), int(N), int(d), int(bool(causal)),
                                   float(scale), int(in_dtype), int(o_dtype), int(grad_dtype),
                                   ws_ptr, int(ws_bytes), stream)


def attn_bwd_qk_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, B, H, Nq,
                    Nk, d, causal, scale, in_dtype, o_dtype, grad_dtype, ws_ptr, ws_bytes,
                    stream=None):
    """Direct call of attn_bwd_qk (Nq query rows, Nk keys); returns the status."""
    return load_library().attn_bwd_qk(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr,
                                      dv_ptr, int(B), int(H), int(Nq), int(Nk), int(d),
                                      int(bool(causal)), float(scale), int(in_dtype), int(o_dtype),
                                      int(grad_dtype), ws_ptr, int(ws_bytes), stream)


def attn_bwd_noalloc_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, B, H,
                         Nq, Nk, d, causal, scale, in_dtype, o_dtype, grad_dtype, stream=None):
    """Direct call of attn_bwd_noalloc (no workspace, no allocation); returns
    the status."""
    return load_library().attn_bwd_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr,
                                           dk_ptr, dv_ptr, int(B), int(H), int(Nq), int(Nk),
                                           int(d), int(bool(causal)), float(scale), int(in_dtype),
                                           int(o_dtype), int(grad_dtype), stream)


def bwd_workspace_bytes(B, H, N, d):
    """Bytes of device workspace attn_bwd needs (0 for an invalid problem)."""
    return int(load_library().attn_bwd_workspace_bytes(int(B), int(H), int(N), int(d)))


def attn_bwd_strided_raw(q_ptr, q_st, k_ptr, k_st, v_ptr, v_st, o_ptr, o_st, lse_ptr, do_ptr,
                         do_st, dq_ptr, dq_st, dk_ptr, dk_st, dv_ptr, dv_st, B, H, Nq, Nk, d,
                         causal, scale, in_dtype, o_dtype, grad_dtype, ws_ptr, ws_bytes,
                         stream=None):
    """Direct call of attn_bwd_strided; *_st are (b, h, row) element strides
    or None (contiguous). Returns the status."""
    return load_library().attn_bwd_strided(
        q_ptr, _strides(q_st), k_ptr, _strides(k_st), v_ptr, _strides(v_st), o_ptr, _strides(o_st),
        lse_ptr, do_ptr, _strides(do_st), dq_ptr, _strides(dq_st), dk_ptr, _strides(dk_st), dv_ptr,
        _strides(dv_st), int(B), int(H), int(Nq), int(Nk), int(d), int(bool(causal)),
        float(scale), int(in_dtype), int(o_dtype), int(grad_dtype), ws_ptr, int(ws_bytes), stream)


def attn_bwd(q, k, v, o, lse, dout, causal=False, scale=None, grad_dtype=None, workspace=None,
             grads=None):
    """Attention backward on the current HIP stream: (dq, dk, dv) for the
    upstream gradient dout, given the forward's inputs, its output o (input
    dtype or float32) and its lse. q, o and dout are [B, H, Nq, d]; k and v
    [B, H, Nk, d] (Nk may differ from Nq when not causal). Any strides with a
    unit last dimension and 16-byte aligned rows are taken as they are
    (attn_bwd_strided); d is a multiple of 8 up to 128. float32 inputs need
    a float32 o and give float32 gradients. grad_dtype defaults to the input
    dtype (torch.float32 is also accepted). The workspace (a uint8 tensor of
    at least bwd_workspace_bytes(B, H, Nq, d) bytes) is taken from torch's
    allocator when not given. Preallocated (dq, dk, dv) may be passed as
    `grads`, with any strides of the same kind.
    """
    if q.dim() != 4 or k.dim() != 4 or o.shape != q.shape or dout.shape != q.shape or \
            v.shape != k.shape or (k.shape[0], k.shape[1], k.shape[3]) != \
            (q.shape[0], q.shape[1], q.shape[3]):
        raise ValueError("q, o, dout must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    if not (q.dtype == k.dtype == v.dtype == dout.dtype) or q.dtype not in _TORCH_TO_ATTN:
        raise ValueError("q, k, v, dout must share one dtype among float32/float16/bfloat16")
    tensors = (q, k, v, o, lse, dout)
    if not (q.is_cuda and all(x.device == q.device for x in tensors)):
        raise ValueError("all tensors must be on one GPU")
    if any(x.stride(3) != 1 for x in (q, k, v, o, dout)):
        raise ValueError("the last dimension must be contiguous")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if d % 8 or not 8 <= d <= 128:
        raise ValueError("the head dim must be a multiple of 8 from 8 to 128")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous [B, H, Nq] float32 tensor")
    if o.dtype not in (q.dtype, torch.float32):
        raise ValueError("o must be in the input dtype or float32")
    if scale is None:
        scale = 1.0 / d ** 0.5
    grad_dtype = grad_dtype or q.dtype
    if grad_dtype not in (q.dtype, torch.float32):
        raise ValueError("grad_dtype must be the input dtype or float32")
    if grads is None:
        grads = [torch.empty(x.shape, dtype=grad_dtype, device=q.device) for x in (q, k, v)]
    dq, dk, dv = grads
    if any(g.shape != x.shape or g.dtype != grad_dtype or g.stride(3) != 1 or
           g.device != q.device for g, x in zip(grads, (q, k, v))):
        raise ValueError("grads must be tensors shaped like q, k, v, of grad_dtype, with a unit "
                         "last stride, on q's device")
    need = bwd_workspace_bytes(B, H, Nq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_bwd_strided_raw(
        q.data_ptr(), q.stride()[:3], k.data_ptr(), k.stride()[:3], v.data_ptr(), v.stride()[:3],
        o.data_ptr(), o.stride()[:3], lse.data_ptr(), dout.data_ptr(), dout.stride()[:3],
        dq.data_ptr(), dq.stride()[:3], dk.data_ptr(), dk.stride()[:3], dv.data_ptr(),
        dv.stride()[:3], B, H, Nq, Nk, d, causal, scale, _TORCH_TO_ATTN[q.dtype],
        _TORCH_TO_ATTN[o.dtype], _TORCH_TO_ATTN[grad_dtype], workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), stream)
    if st != 0:
        msg = status_string(st)
        if st == 5:
            msg += " (hipError_t %d)" % load_library().attn_last_hip_error()
        raise AttnError(st, msg)
    return dq, dk, dv


def row_softmax_raw(x_ptr, xs, y_ptr, ys, M, N, in_dtype, out_dtype, stream=None):
    """Direct call of attn_row_softmax; returns the status."""
    return load_library().attn_row_softmax(x_ptr, int(xs), y_ptr, int(ys), int(M), int(N),
                                           int(in_dtype), int(out_dtype), stream)


def row_softmax(x, out_dtype=None, out=None):
    """Softmax over the last dimension of a 2-D GPU tensor x (rows may be
    strided; the last dimension must be contiguous), into a new tensor or
    into `out`."""
    if x.dim() != 2 or not x.is_cuda or x.dtype not in _TORCH_TO_ATTN or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32/float16/bfloat16 GPU tensor with unit column "
                         "stride")
    M, N = x.shape
    out_dtype = out_dtype or x.dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    if out.shape != x.shape or out.dtype != out_dtype or out.stride(1) != 1 or \
            out.device != x.device:
        raise ValueError("out must be an M x N tensor of out_dtype with unit column stride")
    st = row_softmax_raw(x.data_ptr(), x.stride(0), out.data_ptr(), out.stride(0), M, N,
                         _TORCH_TO_ATTN[x.dtype], _TORCH_TO_ATTN[out_dtype],
                         torch.cuda.current_stream(x.device).cuda_stream)
    if st != 0:
        msg = status_string(st)
        if st == 5:
            msg += " (hipError_t %d)" % load_library().attn_last_hip_error()
        raise AttnError(st, msg)
    return out
