"""Pins of the fp64 backward oracle: facts fixed by the pages or by mathematics.

Each check takes ``grads(q, k, v, dout, causal, scale, qrows=None, krows=None)
-> (dQ, dK, dV)`` (fp64 numpy, [B,H,N,d] without row lists) and raises
AssertionError when the fact fails. The same checks run against the real
backward oracle (``test_oracle_bwd.py``) and against copies of it with a
planted mistake (``test_oracle_bwd_mutants.py``), which must each fail at
least one of them.

None of them retypes the oracle's formulas. They use:
- the pages' Exercise 5 example, differentiated in closed form;
- central finite differences of the (separately pinned) forward oracle;
- torch's fp64 autograd;
- closed forms for special inputs;
- invariants of the softmax Jacobian.
"""
import json
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b))))
    assert err <= tol, "%s: max abs error %.3e > %.1e" % (what, err, tol)


def check_exercise5_gradient(grads):
    """Exercise 5 of the Triton chapter ("4.4 Writing GPU Kernels with
    Triton", section "Exercises"), differentiated by hand. One query (q = 1,
    scale 1) sees keys with scores k = (2, 4) and values v = (1, 3); with
    weights p = softmax(k) and output O = p . v, an upstream gradient of 1 on
    O gives dV_j = p_j, dK_j = q p_j (v_j - O) and
    dQ = sum_j p_j (v_j - O) k_j = p_1 p_2 (v_2 - v_1)(k_2 - k_1)."""
    g = json.load(open(os.path.join(GOLDEN, "exercise5_online_softmax.json")))
    p1, p2 = g["weights"]
    o = g["O_normalised"]
    (k1, k2), (v1, v2) = g["scores"], g["values"]
    q = np.ones((1, 1, 2, 1))
    k = np.array([k1, k2]).reshape(1, 1, 2, 1)
    v = np.array([v1, v2]).reshape(1, 1, 2, 1)
    dout = np.array([0.0, 1.0]).reshape(1, 1, 2, 1)  # row 1 carries the gradient
    dq, dk, dv = grads(q, k, v, dout, False, 1.0)
    _close(dq[0, 0, :, 0], [0.0, p1 * p2 * (v2 - v1) * (k2 - k1)], 1e-14, "exercise 5 dQ")
    _close(dk[0, 0, :, 0], [p1 * (v1 - o), p2 * (v2 - o)], 1e-14, "exercise 5 dK")
    _close(dv[0, 0, :, 0], [p1, p2], 1e-15, "exercise 5 dV")


def _loss(q, k, v, dout, causal, scale):
    o, _ = oracle.attn_oracle(q, k, v, causal=causal, scale=scale)
    return float(np.sum(o * dout))


def check_finite_differences(grads):
    """Every element of dQ, dK, dV equals the central difference of the
    pinned forward oracle's sum(O * dout), on tiny heads (brute force)."""
    h = 1e-5
    for seed, (N, d, causal) in enumerate([(5, 3, False), (6, 2, True), (4, 3, True)]):
        q, k, v = (_rand((1, 1, N, d), 40 + 4 * seed + t) for t in range(3))
        dout = _rand((1, 1, N, d), 43 + 4 * seed)
        scale = 0.7
        got = grads(q, k, v, dout, causal, scale)
        for which, g in enumerate(got):
            fd = np.zeros((N, d))
            for i in range(N):
                for c in range(d):
                    args = [q.copy(), k.copy(), v.copy()]
                    args[which][0, 0, i, c] += h
                    fp = _loss(*args, dout, causal, scale)
                    args[which][0, 0, i, c] -= 2 * h
                    fm = _loss(*args, dout, causal, scale)
                    fd[i, c] = (fp - fm) / (2 * h)
            _close(g[0, 0], fd, 1e-8, "finite differences of %s, case %d" % ("QKV"[which], seed))


def check_torch_autograd(grads):
    """torch's fp64 CPU autograd of softmax(scale Q K^T + mask) V."""
    B, H, N, d = 2, 3, 37, 16
    q, k, v, dout = (_rand((B, H, N, d), 50 + t) for t in range(4))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = (tq @ tk.transpose(-2, -1)) * 0.3
        if causal:
            s = s.masked_fill(~torch.tril(torch.ones(N, N, dtype=torch.bool)), float("-inf"))
        (torch.softmax(s, dim=-1) @ tv).backward(torch.tensor(dout))
        dq, dk, dv = grads(q, k, v, dout, causal, 0.3)
        _close(dq, tq.grad.numpy(), 1e-12, "torch dQ, causal=%s" % causal)
        _close(dk, tk.grad.numpy(), 1e-12, "torch dK, causal=%s" % causal)
        _close(dv, tv.grad.numpy(), 1e-12, "torch dV, causal=%s" % causal)


def _visible_counts(N, causal):
    return np.arange(1, N + 1, dtype=np.float64) if causal else np.full(N, float(N))


def _uniform_dv(dout, causal):
    """dV_j = sum over rows i that see key j of dO_i / n_i, for uniform
    weights 1/n_i over the n_i visible keys."""
    N = dout.shape[2]
    w = dout / _visible_counts(N, causal)[None, None, :, None]
    if not causal:
        return np.broadcast_to(w.sum(axis=2, keepdims=True), dout.shape)
    return np.flip(np.cumsum(np.flip(w, axis=2), axis=2), axis=2)  # sum over i >= j


def check_scale_zero(grads):
    """scale = 0: the weights are uniform and do not depend on Q or K, so
    dQ = dK = 0 exactly, and dV_j = sum_{i sees j} dO_i / n_i."""
    q, k, v, dout = (_rand((1, 2, 23, 6), 60 + t) for t in range(4))
    for causal in (False, True):
        dq, dk, dv = grads(q, k, v, dout, causal, 0.0)
        _close(dq, 0.0, 0.0, "scale 0 dQ")
        _close(dk, 0.0, 0.0, "scale 0 dK")
        _close(dv, _uniform_dv(dout, causal), 1e-13, "scale 0 dV")


def check_query_zero(grads):
    """q = 0: uniform weights again; dK = 0 exactly (it is a sum of multiples
    of q), dV as for scale 0, and dQ_i = (scale / n_i) sum_j (dO_i . (v_j -
    mean_i v)) k_j, the derivative of the mean at a flat softmax."""
    N, d, scale = 19, 5, 0.8
    k, v, dout = (_rand((1, 1, N, d), 64 + t) for t in range(3))
    q = np.zeros((1, 1, N, d))
    for causal in (False, True):
        dq, dk, dv = grads(q, k, v, dout, causal, scale)
        _close(dk, 0.0, 0.0, "q = 0 dK")
        _close(dv, _uniform_dv(dout, causal), 1e-13, "q = 0 dV")
        want = np.zeros((N, d))
        for i in range(N):
            n = i + 1 if causal else N
            vm = v[0, 0, :n].mean(axis=0)
            want[i] = scale / n * ((v[0, 0, :n] - vm) @ dout[0, 0, i]) @ k[0, 0, :n]
        _close(dq[0, 0], want, 1e-13, "q = 0 dQ")


def check_jacobian_invariants(grads):
    """Each row of dS sums to zero (the softmax Jacobian annihilates
    constants), so the dK rows of a head sum to zero; each row of P sums to
    one, so the dV rows of a head sum to the dO rows of the head."""
    q, k, v, dout = (_rand((2, 2, 41, 8), 70 + t, 1.5) for t in range(4))
    for causal in (False, True):
        _, dk, dv = grads(q, k, v, dout, causal, 0.5)
        _close(dk.sum(axis=2), 0.0, 1e-12, "dK column sums")
        _close(dv.sum(axis=2), dout.sum(axis=2), 1e-12, "dV column sums")


def check_single_key(grads):
    """N = 1: the weight is 1 whatever Q and K are, so dQ = dK = 0 and
    dV = dO."""
    q, k, v, dout = (_rand((3, 2, 1, 5), 80 + t) for t in range(4))
    for causal in (False, True):
        dq, dk, dv = grads(q, k, v, dout, causal, 0.9)
        _close(dq, 0.0, 0.0, "N = 1 dQ")
        _close(dk, 0.0, 0.0, "N = 1 dK")
        _close(dv, dout, 0.0, "N = 1 dV")


def check_causal_edges(grads):
    """Causal row 0 sees one key, so its dQ is 0 exactly. The last causal row
    sees every key, so its dQ equals the non-causal one. The last key is seen
    by the last row alone, so its dV is P_{N-1,N-1} dO_{N-1}, with that
    weight read off the forward oracle (V = unit vector trick)."""
    N, d = 29, 7
    q, k, v, dout = (_rand((1, 2, N, d), 90 + t) for t in range(4))
    dq, dk, dv = grads(q, k, v, dout, True, 0.6)
    dq2, _, _ = grads(q, k, v, dout, False, 0.6)
    _close(dq[:, :, 0], 0.0, 0.0, "causal row 0 dQ")
    _close(dq[:, :, -1], dq2[:, :, -1], 1e-13, "causal last row dQ")
    e = np.zeros((1, 2, N, d))
    e[:, :, -1, 0] = 1.0  # V = e_{N-1} in column 0 picks out the weight of key N-1
    o, _ = oracle.attn_oracle(q, k, e, causal=True, scale=0.6)
    p_last = o[:, :, -1, 0]
    _close(dv[:, :, -1], p_last[:, :, None] * dout[:, :, -1], 1e-14, "causal last key dV")
    assert np.max(np.abs(dq[:, :, 1:-1] - dq2[:, :, 1:-1])) > 1e-3, "mask had no effect"


def check_shift_invariance(grads):
    """K <- K + 1 w^T adds a per-row constant to the scores and V <- V + 1 u^T
    a constant to O and to dP's rows: neither changes any gradient."""
    q, k, v, dout = (_rand((1, 2, 27, 6), 100 + t) for t in range(4))
    w, u = _rand((6,), 104), _rand((6,), 105)
    for causal in (False, True):
        base = grads(q, k, v, dout, causal, 0.5)
        for what, args in (("K shift", (q, k + w, v)), ("V shift", (q, k, v + u))):
            got = grads(*args, dout, causal, 0.5)
            for name, a, b in zip("QKV", got, base):
                _close(a, b, 1e-12, "%s: d%s" % (what, name))


def check_linearity_in_dout(grads):
    """The gradients are linear in the upstream gradient."""
    q, k, v, d1, d2 = (_rand((1, 1, 24, 6), 110 + t) for t in range(5))
    for causal in (False, True):
        g1 = grads(q, k, v, d1, causal, 0.5)
        g2 = grads(q, k, v, d2, causal, 0.5)
        g12 = grads(q, k, v, d1 - 3.0 * d2, causal, 0.5)
        for name, a, b, c in zip("QKV", g12, g1, g2):
            _close(a, b - 3.0 * c, 1e-12, "linearity d%s" % name)


def check_key_permutation(grads):
    """Non-causal attention ignores key order: permuting K and V rows permutes
    dK and dV the same way and leaves dQ unchanged."""
    q, k, v, dout = (_rand((1, 1, 21, 6), 120 + t) for t in range(4))
    perm = np.random.default_rng(124).permutation(21)
    dq, dk, dv = grads(q, k, v, dout, False, 0.5)
    dq2, dk2, dv2 = grads(q, k[:, :, perm], v[:, :, perm], dout, False, 0.5)
    _close(dq2, dq, 1e-13, "permutation dQ")
    _close(dk2, dk[:, :, perm], 1e-13, "permutation dK")
    _close(dv2, dv[:, :, perm], 1e-13, "permutation dV")


def check_head_dim_zero_padding(grads):
    """Zero-padding d (Q, K, V and dO) at a fixed scale changes nothing in the
    real columns and gives zero gradients in the padding."""
    q, k, v, dout = (_rand((1, 2, 30, 8), 130 + t) for t in range(4))
    pad = lambda x: np.concatenate([x, np.zeros_like(x)], axis=-1)  # noqa: E731
    for causal in (False, True):
        base = grads(q, k, v, dout, causal, 0.25)
        got = grads(pad(q), pad(k), pad(v), pad(dout), causal, 0.25)
        for name, a, b in zip("QKV", got, base):
            _close(a[..., :8], b, 1e-13, "padded d%s" % name)
            _close(a[..., 8:], 0.0, 0.0, "padded columns of d%s" % name)


def check_large_logits(grads):
    """Scores around +-1000 stay finite; one key dominating every row by
    ~1000 gives dV = dO on that key, 0 elsewhere, and dQ = dK = 0 (to within
    exp(-1000))."""
    N, d = 9, 4
    q = np.zeros((1, 1, N, d))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, d))
    k[0, 0, :, 0] = np.arange(N) * 1000.0 - 4000.0
    v, dout = _rand((1, 1, N, d), 140), _rand((1, 1, N, d), 141)
    dq, dk, dv = grads(q, k, v, dout, False, 1.0)
    assert all(np.all(np.isfinite(x)) for x in (dq, dk, dv))
    want = np.zeros((N, d))
    want[-1] = dout[0, 0].sum(axis=0)
    _close(dv[0, 0], want, 1e-12, "dominant key dV")
    _close(dq, 0.0, 1e-12, "dominant key dQ")
    _close(dk, 0.0, 1e-12, "dominant key dK")


def check_row_subsets(grads):
    """Asking for subsets of rows returns exactly those rows of the full
    result, for query rows (dQ) and key rows (dK, dV) independently."""
    q, k, v, dout = (_rand((2, 3, 19, 5), 150 + t) for t in range(4))
    qrows = [0, 5, 18, 19, 60, 113, 7]
    krows = [113, 0, 40, 18, 19]
    for causal in (False, True):
        dq, dk, dv = grads(q, k, v, dout, causal, 0.5)
        sq, sk, sv = grads(q, k, v, dout, causal, 0.5, qrows=qrows, krows=krows)
        _close(sq, dq.reshape(-1, 5)[qrows], 0.0, "dQ row subset")
        _close(sk, dk.reshape(-1, 5)[krows], 0.0, "dK row subset")
        _close(sv, dv.reshape(-1, 5)[krows], 0.0, "dV row subset")


def check_cross_attention(grads):
    """Query and key lengths that differ (the shapes "Programming an attention
    kernel in Triton", section "Kernel 4: bringing it together, a
    self-attention kernel", validates its forward on, and more): torch's fp64 autograd, every element
    against central finite differences of the forward oracle on a tiny
    case, and the Jacobian invariants."""
    for t, (B, H, nq, nk, d) in enumerate([(1, 1, 5, 15, 32), (1, 1, 1, 10, 64), (2, 3, 7, 19, 8)]):
        q, dout = _rand((B, H, nq, d), 400 + t), _rand((B, H, nq, d), 410 + t)
        k, v = _rand((B, H, nk, d), 420 + t), _rand((B, H, nk, d), 430 + t)
        scale = 1.0 / np.sqrt(d)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = (tq @ tk.transpose(-2, -1)) * scale
        (torch.softmax(s, dim=-1) @ tv).backward(torch.tensor(dout))
        dq, dk, dv = grads(q, k, v, dout, False, scale)
        _close(dq, tq.grad.numpy(), 1e-12, "cross dQ %d" % t)
        _close(dk, tk.grad.numpy(), 1e-12, "cross dK %d" % t)
        _close(dv, tv.grad.numpy(), 1e-12, "cross dV %d" % t)
        _close(dk.sum(axis=2), 0.0, 1e-12, "cross dK column sums")
        _close(dv.sum(axis=2), dout.sum(axis=2), 1e-12, "cross dV column sums")
    q, dout = _rand((1, 1, 3, 2), 440), _rand((1, 1, 3, 2), 441)
    k, v = _rand((1, 1, 5, 2), 442), _rand((1, 1, 5, 2), 443)
    h = 1e-5
    got = grads(q, k, v, dout, False, 0.8)
    for which, g in enumerate(got):
        base = [q, k, v][which]
        fd = np.zeros(base.shape[2:])
        for i in range(base.shape[2]):
            for c in range(base.shape[3]):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][0, 0, i, c] += h
                fp = _loss(*args, dout, False, 0.8)
                args[which][0, 0, i, c] -= 2 * h
                fm = _loss(*args, dout, False, 0.8)
                fd[i, c] = (fp - fm) / (2 * h)
        _close(g[0, 0], fd, 1e-8, "cross finite differences of %s" % "QKV"[which])


ALL_CHECKS = [
    check_exercise5_gradient, check_finite_differences, check_torch_autograd,
    check_scale_zero, check_query_zero, check_jacobian_invariants, check_single_key,
    check_causal_edges, check_shift_invariance, check_linearity_in_dout,
    check_key_permutation, check_head_dim_zero_padding, check_large_logits, check_row_subsets,
    check_cross_attention,
]
