"""Pins of the fp64 oracle: facts fixed by the pages or by mathematics.

Each check takes ``attn(q, k, v, causal, scale, rows=None) -> (O, LSE)``
(fp64 numpy, [B,H,N,d]) and raises AssertionError when the fact fails. The
same checks run against the real oracle (``test_oracle.py``) and against
copies of it with a planted mistake (``test_oracle_mutants.py``), which must
each fail at least one of them.

None of them retypes the oracle's formula: they use worked examples from the
pages, closed forms, invariants, library routines and brute-force variants
with a different order of operations.
"""
import json
import math
import os

import numpy as np
import torch

from oracle import attn_online_np, attn_two_pass_np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b))))
    assert err <= tol, "%s: max abs error %.3e > %.1e" % (what, err, tol)


def check_exercise5(attn):
    """Exercise 5 of the Triton chapter: scores (2, 4), values (1, 3)."""
    g = json.load(open(os.path.join(GOLDEN, "exercise5_online_softmax.json")))
    q = np.ones((1, 1, 2, 1))
    k = np.array(g["scores"]).reshape(1, 1, 2, 1)
    v = np.array(g["values"]).reshape(1, 1, 2, 1)
    # Row 1 is the query that sees both keys; row 0 only matters as filler.
    o, lse = attn(q, k, v, False, 1.0)
    _close(o[0, 0, 1, 0], g["O_normalised"], 1e-14, "exercise 5 O")
    _close(lse[0, 0, 1], g["lse"], 1e-14, "exercise 5 LSE")
    # Weights: O is linear in V, so unit value vectors expose them.
    o1, _ = attn(q, k, np.array([1.0, 0.0]).reshape(1, 1, 2, 1), False, 1.0)
    _close(o1[0, 0, 1, 0], g["weights"][0], 1e-15, "exercise 5 weight 1")


def check_weights_sum_to_one(attn):
    """Rows of the softmax sum to 1: a constant V column comes back unchanged."""
    for causal in (False, True):
        q, k = _rand((2, 3, 97, 16), 1), _rand((2, 3, 97, 16), 2)
        v = np.ones((2, 3, 97, 16)) * 0.75
        o, _ = attn(q, k, v, causal, 0.25)
        _close(o, 0.75, 1e-12, "constant V, causal=%s" % causal)


def check_weights_identity_v(attn):
    """With V = I (N = d) row i of O is row i of the softmax: non-negative,
    summing to 1, zero above the diagonal when causal, and with ratios
    P_ij / P_i0 = exp(scale * q_i . (k_j - k_0))."""
    n = 12
    q, k = _rand((1, 1, n, n), 3), _rand((1, 1, n, n), 4)
    v = np.eye(n).reshape(1, 1, n, n)
    scale = 0.3
    for causal in (False, True):
        o, _ = attn(q, k, v, causal, scale)
        p = o[0, 0]
        assert np.all(p >= 0.0)
        _close(p.sum(axis=1), 1.0, 1e-13, "identity-V row sums")
        if causal:
            assert np.all(np.triu(p, 1) == 0.0), "causal weights above the diagonal"
        for i in range(n):
            hi = i + 1 if causal else n
            dk = k[0, 0, :hi] - k[0, 0, 0]
            want = np.exp(scale * (dk @ q[0, 0, i]))
            _close(p[i, :hi] / p[i, 0], want, 1e-11 * want.max(), "weight ratios")


def check_constant_scores(attn):
    """q = 0, scale = 0 or equal keys: O is the mean of the visible V rows
    and LSE = score + ln(#visible keys)."""
    B, H, N, d = 1, 2, 40, 8
    v = _rand((B, H, N, d), 5)
    k = _rand((B, H, N, d), 6)
    q = _rand((B, H, N, d), 7)
    counts = np.arange(1, N + 1, dtype=np.float64)
    for causal in (False, True):
        means = np.cumsum(v, axis=2) / counts[None, None, :, None] if causal \
            else np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        n_vis = counts if causal else np.full(N, float(N))
        o, lse = attn(np.zeros_like(q), k, v, causal, 0.5)
        _close(o, means, 1e-13, "q = 0")
        _close(lse, np.broadcast_to(np.log(n_vis), lse.shape), 1e-13, "q = 0 LSE")
        o, lse = attn(q, k, v, causal, 0.0)
        _close(o, means, 1e-13, "scale = 0")
        kk = np.broadcast_to(k[:, :, :1, :], k.shape).copy()
        o, lse = attn(q, kk, v, causal, 0.5)
        _close(o, means, 1e-13, "equal keys")
        s = 0.5 * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0, :])
        _close(lse, s + np.log(n_vis), 1e-12, "equal keys LSE")


def check_single_key(attn):
    """N = 1: O = V[0], LSE = scale q0 . k0, causal or not."""
    q, k, v = _rand((3, 2, 1, 5), 8), _rand((3, 2, 1, 5), 9), _rand((3, 2, 1, 5), 10)
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.7)
        _close(o, v, 0.0, "N = 1 output")
        _close(lse[..., 0], 0.7 * np.sum(q[..., 0, :] * k[..., 0, :], axis=-1), 1e-14, "N = 1 LSE")


def check_causal_first_and_last_row(attn):
    """Causal row 0 sees key 0 only; causal last row equals the non-causal one."""
    q, k, v = _rand((2, 2, 33, 8), 11), _rand((2, 2, 33, 8), 12), _rand((2, 2, 33, 8), 13)
    o, lse = attn(q, k, v, True, 0.4)
    _close(o[:, :, 0], v[:, :, 0], 0.0, "causal first row")
    _close(lse[:, :, 0], 0.4 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), 1e-14, "causal row 0 LSE")
    o2, lse2 = attn(q, k, v, False, 0.4)
    _close(o[:, :, -1], o2[:, :, -1], 1e-15, "causal last row")
    _close(lse[:, :, -1], lse2[:, :, -1], 1e-15, "causal last row LSE")
    assert np.max(np.abs(o[:, :, 1:-1] - o2[:, :, 1:-1])) > 1e-3, "mask had no effect"


def check_prefix_consistency(attn):
    """Causal row i = non-causal attention of q_i over K[0..i], V[0..i]."""
    q, k, v = _rand((1, 1, 20, 6), 14), _rand((1, 1, 20, 6), 15), _rand((1, 1, 20, 6), 16)
    o, lse = attn(q, k, v, True, 0.6)
    for i in (1, 7, 19):
        oi, li = attn(q[:, :, :i + 1], k[:, :, :i + 1], v[:, :, :i + 1], False, 0.6)
        _close(o[0, 0, i], oi[0, 0, i], 1e-14, "prefix row %d" % i)
        _close(lse[0, 0, i], li[0, 0, i], 1e-14, "prefix LSE row %d" % i)


def check_variants_agree(attn, seeds=range(50)):
    """Two-pass and online (block 1, 2, 3, 7, N) variants agree within 1e-12."""
    for seed in seeds:
        rng = np.random.default_rng(1000 + seed)
        n = int(rng.integers(1, 18))
        d = int(rng.integers(1, 9))
        q, k, v = (rng.standard_normal((n, d)) * 2.0 for _ in range(3))
        scale = float(rng.uniform(0.1, 1.5))
        causal = bool(seed % 2)
        o, lse = attn(q[None, None], k[None, None], v[None, None], causal, scale)
        o2, l2 = attn_two_pass_np(q, k, v, causal, scale)
        _close(o[0, 0], o2, 1e-12, "two-pass variant, seed %d" % seed)
        _close(lse[0, 0], l2, 1e-12, "two-pass LSE, seed %d" % seed)
        for blk in (1, 2, 3, 7, n):
            o3, l3 = attn_online_np(q, k, v, causal, scale, block=blk)
            _close(o[0, 0], o3, 1e-12, "online variant block %d, seed %d" % (blk, seed))
            _close(lse[0, 0], l3, 1e-12, "online LSE block %d, seed %d" % (blk, seed))


def check_torch_library(attn):
    """torch's fp64 CPU softmax / logsumexp and its scaled_dot_product_attention."""
    B, H, N, d = 2, 3, 50, 24
    q, k, v = _rand((B, H, N, d), 17), _rand((B, H, N, d), 18), _rand((B, H, N, d), 19)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    for causal in (False, True):
        s = (tq @ tk.transpose(-2, -1)) * 0.2
        if causal:
            s = s.masked_fill(~torch.tril(torch.ones(N, N, dtype=torch.bool)), float("-inf"))
        ref_o = (torch.softmax(s, dim=-1) @ tv).numpy()
        ref_l = torch.logsumexp(s, dim=-1).numpy()
        sdpa = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                                scale=0.2).numpy()
        o, lse = attn(q, k, v, causal, 0.2)
        _close(o, ref_o, 1e-12, "torch softmax @ V, causal=%s" % causal)
        _close(lse, ref_l, 1e-12, "torch logsumexp, causal=%s" % causal)
        _close(o, sdpa, 1e-12, "torch sdpa, causal=%s" % causal)


def check_shift_invariance(attn):
    """K <- K + 1 w^T adds scale q_i . w to row i's scores: O unchanged,
    LSE_i grows by exactly that amount."""
    q, k, v = _rand((1, 2, 30, 8), 20), _rand((1, 2, 30, 8), 21), _rand((1, 2, 30, 8), 22)
    w = _rand((8,), 23)
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.5)
        o2, lse2 = attn(q, k + w, v, causal, 0.5)
        _close(o2, o, 1e-12, "shift O")
        _close(lse2 - lse, 0.5 * (q @ w), 1e-12, "shift LSE")


def check_key_permutation(attn):
    """Non-causal attention does not depend on the order of the keys."""
    q, k, v = _rand((1, 1, 25, 8), 24), _rand((1, 1, 25, 8), 25), _rand((1, 1, 25, 8), 26)
    perm = np.random.default_rng(27).permutation(25)
    o, lse = attn(q, k, v, False, 0.5)
    o2, lse2 = attn(q, k[:, :, perm], v[:, :, perm], False, 0.5)
    _close(o2, o, 1e-13, "key permutation O")
    _close(lse2, lse, 1e-13, "key permutation LSE")


def check_linearity_and_hull(attn):
    """O is linear in V and each output lies between the min and max of the
    visible values of its column."""
    q, k = _rand((1, 2, 31, 8), 28, 2.0), _rand((1, 2, 31, 8), 29, 2.0)
    v1, v2 = _rand((1, 2, 31, 8), 30), _rand((1, 2, 31, 8), 31)
    for causal in (False, True):
        o1, _ = attn(q, k, v1, causal, 0.5)
        o2, _ = attn(q, k, v2, causal, 0.5)
        o12, _ = attn(q, k, v1 + 2.0 * v2, causal, 0.5)
        _close(o12, o1 + 2.0 * o2, 1e-12, "linearity in V")
        for i in range(31):
            hi = i + 1 if causal else 31
            lo_v = v1[:, :, :hi].min(axis=2)
            hi_v = v1[:, :, :hi].max(axis=2)
            assert np.all(o1[:, :, i] >= lo_v - 1e-13) and np.all(o1[:, :, i] <= hi_v + 1e-13)


def check_head_dim_zero_padding(attn):
    """Zero-padding the head dimension at a fixed scale is exact ("Sizing the
    attention kernel"): same O in the real columns, zeros in the padding,
    same LSE."""
    q, k, v = _rand((1, 2, 40, 64), 32), _rand((1, 2, 40, 64), 33), _rand((1, 2, 40, 64), 34)
    pad = lambda x: np.concatenate([x, np.zeros_like(x)], axis=-1)  # noqa: E731
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.125)
        o2, lse2 = attn(pad(q), pad(k), pad(v), causal, 0.125)
        _close(o2[..., :64], o, 1e-13, "padded O")
        _close(o2[..., 64:], 0.0, 0.0, "padded columns")
        _close(lse2, lse, 1e-13, "padded LSE")


def check_large_logits(attn):
    """Scores near +-1000 (exp overflows without the max subtraction): one
    key dominating by ~1000 gives exactly its value row; LSE = its score."""
    N, d = 9, 4
    q = np.zeros((1, 1, N, d))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, d))
    k[0, 0, :, 0] = np.arange(N) * 1000.0 - 4000.0
    v = _rand((1, 1, N, d), 35)
    o, lse = attn(q, k, v, False, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    _close(o[0, 0], np.broadcast_to(v[0, 0, -1], (N, d)), 0.0, "dominant key")
    _close(lse[0, 0], 4000.0, 0.0, "dominant key LSE")
    o, lse = attn(q, k, v, True, 1.0)  # row i is dominated by key i
    _close(o[0, 0], v[0, 0], 0.0, "causal dominant key")
    _close(lse[0, 0], k[0, 0, :, 0], 0.0, "causal dominant key LSE")


def check_row_subset(attn):
    """Asking for a subset of rows returns exactly those rows of the full result."""
    q, k, v = _rand((2, 3, 21, 8), 36), _rand((2, 3, 21, 8), 37), _rand((2, 3, 21, 8), 38)
    rows = [0, 5, 20, 21, 62, 125, 7]
    for causal in (False, True):
        o, lse = attn(q, k, v, causal, 0.5)
        os_, ls_ = attn(q, k, v, causal, 0.5, rows=rows)
        _close(os_, o.reshape(-1, 8)[rows], 0.0, "row subset O")
        _close(ls_, lse.reshape(-1)[rows], 0.0, "row subset LSE")


def check_cross_attention(attn):
    """Query and key lengths that differ ("Programming an attention kernel in
    Triton", section "Kernel 4: bringing it together, a self-attention
    kernel", validates its kernel on Q (5, 32) against K, V (15, 32) and on a single query
    against 10 keys): agreement with torch's fp64 scaled_dot_product_attention
    and with the brute-force two-pass and online variants, at the page's
    shapes and a few more."""
    shapes = [(1, 1, 5, 15, 32), (1, 1, 1, 10, 64), (2, 3, 7, 40, 16), (1, 2, 33, 3, 8)]
    for t, (B, H, nq, nk, d) in enumerate(shapes):
        q = _rand((B, H, nq, d), 200 + t)
        k, v = _rand((B, H, nk, d), 210 + t), _rand((B, H, nk, d), 220 + t)
        scale = 1.0 / np.sqrt(d)
        o, lse = attn(q, k, v, False, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()
        ref_l = torch.logsumexp((tq @ tk.transpose(-2, -1)) * scale, dim=-1).numpy()
        _close(o, ref, 1e-12, "cross-attention vs sdpa %s" % (shapes[t],))
        _close(lse, ref_l, 1e-12, "cross-attention LSE %s" % (shapes[t],))
        o2, l2 = attn_two_pass_np(q[0, 0], k[0, 0], v[0, 0], False, scale)
        _close(o[0, 0], o2, 1e-12, "cross-attention two-pass")
        o3, l3 = attn_online_np(q[0, 0], k[0, 0], v[0, 0], False, scale, block=4)
        _close(o[0, 0], o3, 1e-12, "cross-attention online")
        _close(lse[0, 0], l3, 1e-12, "cross-attention online LSE")


def check_cross_rows_independent(attn):
    """Each query row attends on its own: the rows of a cross-attention
    batch equal single-query calls, and row subsets equal the full result."""
    q, k, v = _rand((1, 2, 9, 8), 230), _rand((1, 2, 21, 8), 231), _rand((1, 2, 21, 8), 232)
    o, lse = attn(q, k, v, False, 0.4)
    for i in (0, 4, 8):
        oi, li = attn(q[:, :, i:i + 1], k, v, False, 0.4)
        _close(oi[:, :, 0], o[:, :, i], 1e-15, "single query row %d" % i)
        _close(li[:, :, 0], lse[:, :, i], 1e-15, "single query LSE %d" % i)
    rows = [17, 0, 9, 3]
    os_, ls_ = attn(q, k, v, False, 0.4, rows=rows)
    _close(os_, o.reshape(-1, 8)[rows], 0.0, "cross-attention row subset")


ALL_CHECKS = [
    check_exercise5, check_weights_sum_to_one, check_weights_identity_v,
    check_constant_scores, check_single_key, check_causal_first_and_last_row,
    check_prefix_consistency, check_variants_agree, check_torch_library,
    check_shift_invariance, check_key_permutation, check_linearity_and_hull,
    check_head_dim_zero_padding, check_large_logits, check_row_subset,
    check_cross_attention, check_cross_rows_independent,
]
