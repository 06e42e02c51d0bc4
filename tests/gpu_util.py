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
    # scores of exactly zero (every head's weight below the cutoff) tie exactly on
    # both sides and go to the lower index: that choice is unique too
    separated = (kth - nxt) > rel * kth or kth == 0.0
    return bool(ok), bool(separated)


def separated_query(cfg, layer, batch, n_kv, G, d, k_res, scale, k_sel, rel=1e-4, max_redraws=400):
    """A query fp16 [batch][n_kv*G][d] whose oracle token scores separate the k-th and
    the (k+1)-th token of every (batch, kv head) by at least `rel` (relative), so that
    the top-k index set is unique in any precision the kernels use.

    k_res(bi, g) -> resident keys fp64 [T][d] of KV head g of batch row bi.  Every
    (batch, kv head) group starts with its heads of inputs.query(cfg, layer, 0, ...);
    while its scores have a near-tie at the boundary it takes its heads from the draw
    of the next step.  Returns (q, steps): steps[(bi, g)] = the step used."""
    from bit_decode_selective_amd import inputs
    from oracle import attention as o_attn

    n_q = n_kv * G
    draws = {0: inputs.query(cfg, layer, 0, batch, n_q, d)}
    q = draws[0].copy()
    steps = {}
    for bi in range(batch):
        for g in range(n_kv):
            kr = k_res(bi, g)
            for step in range(max_redraws):
                if step not in draws:
                    draws[step] = inputs.query(cfg, layer, step, batch, n_q, d)
                qg = draws[step][bi, g * G:(g + 1) * G]
                if k_sel == 0 or token_gap(o_attn.token_scores(qg, kr, scale), k_sel) >= rel:
                    q[bi, g * G:(g + 1) * G] = qg
                    steps[(bi, g)] = step
                    break
            else:
                raise RuntimeError(f"no separated query for group {(bi, g)} in {max_redraws} draws")
    return q, steps


def token_gap(scores, k):
    """Relative gap (s_k - s_{k+1}) / s_k of the k-th and (k+1)-th largest scores."""
    order = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    if k == 0 or k >= len(order):
        return np.inf
    return (order[k - 1] - order[k]) / order[k - 1]
