"""Two small fp64 NumPy variants of attention -- TEST INFRASTRUCTURE ONLY.

They exist to pin the C oracle by brute force on tiny inputs: three
independent orderings of the same arithmetic must agree to ~1e-12.

attn_two_pass_np
    Pass 1 finds the row maximum of the scaled scores; pass 2 accumulates
    the exponentials and the un-normalised output together and divides once
    at the end ("4.4 Writing GPU Kernels with Triton", section "Kernel 2:
    Fused Softmax" for the max-subtraction; "Kernel 4", "The Online Softmax
    Recurrence", for the single division at the end).

attn_online_np
    One streaming pass over key blocks of a chosen size, keeping per query
    row the running maximum m, the running sum l and the un-normalised
    output O. When a block with maximum m_blk arrives, the new maximum is
    m' = max(m, m_blk); the old state is rescaled by alpha = exp(m - m'),
    then l += sum_j exp(s_j - m') and O += sum_j exp(s_j - m') v_j. After the
    last block O / l is the output and m + ln l the log-sum-exp ("4.4
    Writing GPU Kernels with Triton", section "The Online Softmax
    Recurrence"; the same state update in "Triton Kernel Practice", section
    "Kernel 3: The FlashAttention Core"). Natural exp is used; the pages'
    base-2 form is the same arithmetic with log2(e) folded into the scale.

Both take q, k, v as [N, d] (one head) fp64 arrays. Pure Python loops over
rows and blocks: for N up to a few dozen only.
"""
import math

import numpy as np


def _scores(q_row, k, scale, n_keys):
    return np.array([scale * float(np.dot(q_row, k[j])) for j in range(n_keys)])


def attn_two_pass_np(q, k, v, causal=False, scale=None):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((N, v.shape[1]))
    lse = np.zeros(N)
    for i in range(N):
        n_keys = i + 1 if causal else k.shape[0]
        s = _scores(q[i], k, scale, n_keys)
        m = s.max()
        l = 0.0
        acc = np.zeros(v.shape[1])
        for j in range(n_keys):
            e = math.exp(s[j] - m)
            l += e
            acc += e * v[j]
        o[i] = acc / l
        lse[i] = m + math.log(l)
    return o, lse


def attn_online_np(q, k, v, causal=False, scale=None, block=1, trace=None):
    """Online-softmax attention over key blocks of `block` keys.

    If `trace` is a list, one dict per (row, block) step is appended with the
    state after that block: {'row', 'block', 'alpha', 'm', 'l', 'O'}.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if block < 1:
        raise ValueError("block must be >= 1")
    o = np.zeros((N, v.shape[1]))
    lse = np.zeros(N)
    for i in range(N):
        n_keys = i + 1 if causal else k.shape[0]
        m = -math.inf
        l = 0.0
        acc = np.zeros(v.shape[1])
        for b0 in range(0, n_keys, block):
            js = range(b0, min(b0 + block, n_keys))
            s = _scores(q[i], k[b0:], scale, len(js))
            m_new = max(m, float(s.max()))
            alpha = math.exp(m - m_new)  # exp(-inf) = 0 on the first block
            p = np.exp(s - m_new)
            l = alpha * l + float(p.sum())
            acc = alpha * acc + p @ v[b0:b0 + len(js)]
            m = m_new
            if trace is not None:
                trace.append({"row": i, "block": b0 // block, "alpha": alpha,
                              "m": m, "l": l, "O": acc.copy()})
        o[i] = acc / l
        lse[i] = m + math.log(l)
    return o, lse
