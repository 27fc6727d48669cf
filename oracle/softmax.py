"""Row softmax in fp64 -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use it. It shares no code with the HIP library.

What it computes: the numerically stable softmax of every row of an M x N
matrix, the operation of "4.4 Writing GPU Kernels with Triton", section
"Kernel 2: Fused Softmax" (subtract the row maximum, exponentiate, divide by
the row sum), written as its three passes per row:

  m_i  = max_j x_ij
  e_ij = exp(x_ij - m_i),   l_i = sum_j e_ij
  y_ij = e_ij / l_i
"""
import numpy as np


def row_softmax(x, axis_len=None):
    """fp64 softmax over the last dimension of a 2-D array (any real dtype
    or a torch tensor; values are upcast exactly)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("row_softmax takes an M x N matrix")
    M, N = x.shape
    y = np.empty_like(x)
    for i in range(M):
        row = x[i]
        m = row.max()                # pass 1: the row maximum
        e = np.exp(row - m)          # pass 2: exponentials relative to it,
        l = e.sum()                  #         and their sum
        y[i] = e / l                 # pass 3: normalise
    return y
