"""Pins for the oracle's channel selection and refined GEMV (CPU only).

Selection follows the rag-lover.com StrataFlux summary, explainer dialogue (weight
refinements chosen by input-activation magnitude); the miss fallback follows its
limitations section.  Pins: hand-derived worked example, brute-force subset search
for top-k, and the invariants all-selected => (b+r)-bit GEMV, none => b-bit GEMV,
additivity over disjoint refined sets.
"""
import itertools

import numpy as np
import pytest

from oracle import gemv, nested, selection


def test_k_select():
    assert selection.k_select(5, 4096) == 205
    assert selection.k_select(3, 4096) == 123
    assert selection.k_select(3, 14336) == 431
    assert selection.k_select(3, 12288) == 369
    assert selection.k_select(2, 32768) == 656
    assert selection.k_select(2, 8192) == 164
    assert selection.k_select(2, 131072) == 2622
    assert selection.k_select(0, 4096) == 0
    assert selection.k_select(100, 4096) == 4096


def _brute_top_k(scores, k):
    """The unique k-subset in which every member beats every non-member under the
    order (higher score first, then lower index)."""
    n = len(scores)
    found = []
    for sub in itertools.combinations(range(n), k):
        s = set(sub)
        if all(
            (scores[i] > scores[j]) or (scores[i] == scores[j] and i < j)
            for i in s
            for j in range(n)
            if j not in s
        ):
            found.append(list(sub))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(6))
def test_top_k_brute_force(seed):
    g = np.random.default_rng(seed)
    n = 9
    scores = g.integers(0, 4, size=n).astype(float)  # many ties
    for k in range(0, n + 1):
        assert selection.top_k(scores, k) == _brute_top_k(list(scores), k)


def test_channel_scores_batch_max():
    x = np.array([[1.0, -3.0, 0.5], [-2.0, 1.0, 0.25]], dtype=np.float16)
    assert selection.channel_scores(x).tolist() == [2.0, 3.0, 0.5]
    assert selection.select_channels(x, 2) == [0, 1]


def test_worked_example_gemv(golden):
    ex = golden["nested_2bit"]
    gx = golden["gemv_row"]
    w = np.array([ex["x"]], dtype=np.float32)
    q = nested.quantize(w, ex["b"], ex["r"], ex["group"])
    x = np.array([gx["x"]], dtype=np.float16)
    assert gemv.refined_gemv(q, x, [])[0, 0] == gx["y_none"]
    assert gemv.refined_gemv(q, x, range(4))[0, 0] == gx["y_all"]
    s1 = selection.select_channels(x, 1)
    assert s1 == gx["k1_selected"]
    assert gemv.refined_gemv(q, x, s1)[0, 0] == gx["y_k1"]
    s2 = selection.select_channels(x, 2)
    assert s2 == gx["k2_selected"]
    assert gemv.refined_gemv(q, x, s2)[0, 0] == gx["y_k2"]


def _quantized(seed, n, k, b=2, r=2):
    g = np.random.default_rng(seed)
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    x = g.standard_normal((2, k)).astype(np.float16)
    return nested.quantize(w, b, r, 128), x


def test_gemv_all_and_none():
    q, x = _quantized(3, 16, 256)
    xf = x.astype(np.float64)
    y_all = gemv.refined_gemv(q, x, range(256))
    y_none = gemv.refined_gemv(q, x, [])
    # (b+r)-bit and b-bit GEMVs written element by element
    full = nested.dequant_full(q)
    res = nested.dequant_resident(q)
    for bi in range(2):
        for n in range(16):
            assert y_all[bi, n] == pytest.approx(sum(xf[bi, k] * full[n, k] for k in range(256)), rel=1e-12, abs=1e-12)
            assert y_none[bi, n] == pytest.approx(sum(xf[bi, k] * res[n, k] for k in range(256)), rel=1e-12, abs=1e-12)


def test_gemv_additive_over_disjoint_sets():
    q, x = _quantized(4, 24, 384)
    e1 = [0, 5, 130, 200]
    e2 = [1, 6, 300, 383]
    y12 = gemv.refined_gemv(q, x, e1 + e2)
    y1 = gemv.refined_gemv(q, x, e1)
    y2 = gemv.refined_gemv(q, x, e2)
    y0 = gemv.refined_gemv(q, x, [])
    np.testing.assert_allclose(y12, y1 + y2 - y0, rtol=0, atol=1e-12)
    # each refined channel moves y by x_k * s * c_lo exactly
    _, lo = nested.split(q)
    s = np.repeat(q["scale"].astype(np.float64), 128, axis=1)
    d = gemv.refined_gemv(q, x, [130]) - y0
    np.testing.assert_allclose(d, x.astype(np.float64)[:, [130]] * (s[:, 130] * lo[:, 130])[None, :], atol=1e-13)


def test_lag_delta_worked_example(golden):
    """Channel 1 selected but late: the worked row's output is y_none at the GEMV
    and y_k1 once the late contribution (x_1 * s * c_lo = 2 * 0.0625 * 3) is added."""
    ex = golden["nested_2bit"]
    gx = golden["gemv_row"]
    q = nested.quantize(np.array([ex["x"]], dtype=np.float32), ex["b"], ex["r"], ex["group"])
    x = np.array([gx["x"]], dtype=np.float16)
    d = gemv.lag_delta(q, x, [1])
    assert d[0, 0] == 0.375
    assert gemv.refined_gemv(q, x, [])[0, 0] + d[0, 0] == gx["y_k1"]
    assert gemv.lag_delta(q, x, [])[0, 0] == 0.0


def test_lag_delta_completes_the_refined_output():
    """GEMV on the hits E plus the late contribution of L equals the GEMV refined on
    E and L together (disjoint sets), element by element against a written-out sum."""
    q, x = _quantized(5, 20, 384)
    hits, late = [3, 40, 200], [7, 129, 383]
    d = gemv.lag_delta(q, x, late)
    np.testing.assert_allclose(gemv.refined_gemv(q, x, hits) + d, gemv.refined_gemv(q, x, hits + late), rtol=0,
                               atol=1e-12)
    _, lo = nested.split(q)
    s = q["scale"].astype(np.float64)
    xf = x.astype(np.float64)
    for bi in range(2):
        for n in range(20):
            want = sum(xf[bi, k] * s[n, k // 128] * lo[n, k] for k in late)
            assert d[bi, n] == pytest.approx(want, rel=1e-12, abs=1e-15)
