"""Independent checks used to pin the oracle (and, on the GPU, the HIP path).

None of these calls the oracle.  They restate the selection rule in other
ways: an O(n^2) rank count, numpy's stable argsort, closed forms for special
rows, and invariants that any correct output satisfies.
"""

from __future__ import annotations

import numpy as np


def bruteforce_row(row, n: int, K: int) -> list[int]:
    """Rank count straight from the rule: position c is chosen iff fewer than
    K positions beat it (d beats c: larger value, or equal value and d < c).
    Chosen positions ascending, then -1 up to K.  Pure Python; tiny rows."""
    n = max(0, min(int(n), len(row)))
    vals = [float(row[i]) for i in range(n)]

    def beats(d, c):
        return vals[d] > vals[c] or (vals[d] == vals[c] and d < c)

    chosen = [c for c in range(n) if sum(1 for d in range(n) if beats(d, c)) < K]
    return chosen + [-1] * (K - len(chosen))


def argsort_row(row: np.ndarray, n: int, K: int) -> np.ndarray:
    """Library route: numpy's stable argsort of -x lists positions by
    decreasing value with equal values kept in index order, which is exactly
    the rule's order when the prefix holds no NaN.  (-x maps -0.0 and +0.0 to
    values that compare equal, so signed zeros stay tied.)"""
    n = max(0, min(int(n), row.shape[0]))
    m = min(K, n)
    x = row[:n].astype(np.float64)
    order = np.argsort(-x, kind="stable")
    out = np.full(K, -1, dtype=np.int32)
    out[:m] = np.sort(order[:m])
    return out


def check_invariants(row: np.ndarray, n: int, K: int, out: np.ndarray) -> None:
    """Properties every correct output row has (assert on failure)."""
    n = max(0, min(int(n), row.shape[0]))
    m = min(K, n)
    out = np.asarray(out)
    assert out.shape == (K,)
    sel = out[:m]
    assert np.all(out[m:] == -1), "padding must be -1 after the first min(K, n) entries"
    assert np.all(sel >= 0) and np.all(sel < n), "indices must lie in [0, n)"
    assert np.all(np.diff(sel) > 0), "indices must be strictly ascending"
    if m == 0 or m == n:
        if m == n:
            assert np.array_equal(sel, np.arange(n))
        return
    x = row[:n].astype(np.float64)
    mask = np.zeros(n, dtype=bool)
    mask[sel] = True
    lo = x[mask].min()
    hi = x[~mask].max()
    assert lo >= hi, "every chosen value must be >= every unchosen value"
    if lo == hi:
        # Among positions holding the threshold value, the chosen ones all
        # come before the unchosen ones.
        eq = np.nonzero(x == lo)[0]
        chosen_eq = eq[mask[eq]]
        unchosen_eq = eq[~mask[eq]]
        if chosen_eq.size and unchosen_eq.size:
            assert chosen_eq.max() < unchosen_eq.min(), "ties must go to the lower index"
