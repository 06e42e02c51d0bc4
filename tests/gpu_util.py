"""Helpers for the GPU parity tests (comparison only; no method arithmetic)."""
import numpy as np

RTOL = 1e-3
ATOL = 1e-4


def assert_close(got, want, rtol=RTOL, atol=ATOL, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want)
    bad = err > atol + rtol * np.abs(want)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(want))), got.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside rtol={rtol} atol={atol}; worst at {i}: "
            f"got {got[i]!r} want {want[i]!r}"
        )


def topk_is_valid(scores, sel, k, rel=1e-4):
    """A k-subset of the top-k by `scores` up to a relative near-tie margin: every
    chosen item scores at least the k-th largest (minus margin) and every other item
    at most the k-th largest (plus margin).  Returns (valid, exact_margin_ok) where the
    second flag says the k-th and (k+1)-th scores are separated by more than `rel`."""
    scores = np.asarray(scores, dtype=np.float64)
    sel = np.asarray(sel, dtype=np.int64)
    if len(sel) != k or len(set(sel.tolist())) != k:
        return False, False
    if k == 0:
        return True, True
    order = np.sort(scores)[::-1]
    kth = order[k - 1]
    nxt = order[k] if k < len(order) else -np.inf
    mask = np.zeros(len(scores), dtype=bool)
    mask[sel] = True
    ok = np.all(scores[mask] >= kth * (1 - rel)) and np.all(scores[~mask] <= kth * (1 + rel))
    separated = (kth - nxt) > rel * kth
    return bool(ok), bool(separated)
