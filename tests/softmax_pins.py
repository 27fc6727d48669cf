"""Pins of the fp64 row-softmax oracle: facts fixed by the pages or by
mathematics. Each check takes ``softmax(x) -> y`` (fp64 numpy, M x N) and
raises AssertionError when the fact fails; the same checks run against the
real oracle and against copies with a planted mistake."""
import numpy as np
import torch


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b))))
    assert err <= tol, "%s: max abs error %.3e > %.1e" % (what, err, tol)


def check_torch(softmax):
    """torch's fp64 CPU softmax, on the page's test shape (1823 x 781) and on
    the 2000-column case of the bug story in "Programming an attention kernel
    in Triton", section "Kernel 3: fused softmax, and the bug that mattered"."""
    for t, shape in enumerate([(1823, 781), (4, 5), (3, 2000), (7, 1)]):
        x = _rand(shape, 300 + t, 2.0)
        ref = torch.softmax(torch.from_numpy(x), dim=1).numpy()
        _close(softmax(x), ref, 1e-15, "torch softmax %s" % (shape,))


def check_rows_sum_to_one_and_ratios(softmax):
    """Rows sum to 1, entries are positive, and y_ij / y_ik = exp(x_ij - x_ik)."""
    x = _rand((9, 37), 310, 3.0)
    y = softmax(x)
    assert np.all(y > 0)
    _close(y.sum(axis=1), 1.0, 1e-14, "row sums")
    _close((y / y[:, :1]) / np.exp(x - x[:, :1]), 1.0, 1e-13, "ratios (relative)")


def check_closed_forms(softmax):
    """A constant row gives 1/N everywhere; a row with one entry larger than
    the rest by 1000 gives exactly the one-hot vector (exp(-1000) underflows);
    one column gives 1."""
    x = np.full((3, 10), 2.5)
    _close(softmax(x), 0.1, 1e-16, "constant rows")
    x = np.zeros((2, 6))
    x[0, 4] = 1000.0
    x[1, 0] = -1000.0
    y = softmax(x)
    want0 = np.zeros(6)
    want0[4] = 1.0
    _close(y[0], want0, 0.0, "dominant entry")
    _close(y[1, 1:], 0.2, 1e-16, "one very small entry")
    _close(softmax(_rand((4, 1), 311)), 1.0, 0.0, "single column")


def check_shift_invariance(softmax):
    """Adding a constant to a row changes nothing, also at +-1e4 where exp
    overflows without the max subtraction."""
    x = _rand((5, 50), 312)
    y = softmax(x)
    for c in (7.0, -3.25, 1e4, -1e4):
        _close(softmax(x + c), y, 1e-12, "shift by %g" % c)


def check_rows_independent(softmax):
    """Each row is normalised on its own: permuting rows permutes the result,
    and a row's result does not depend on the other rows."""
    x = _rand((8, 13), 313)
    perm = np.random.default_rng(314).permutation(8)
    _close(softmax(x[perm]), softmax(x)[perm], 0.0, "row permutation")
    _close(softmax(x[3:4]), softmax(x)[3:4], 0.0, "single row")


ALL_CHECKS = [check_torch, check_rows_sum_to_one_and_ratios, check_closed_forms,
              check_shift_invariance, check_rows_independent]
