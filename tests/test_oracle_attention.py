"""Pins for the oracle's refined GQA decode attention (CPU only).

Follows the rag-lover.com StrataFlux summary, explainer dialogue (KV refinements
chosen by the attention weight computed from the low-bit keys) and limitations
section (a miss stays at resident precision).  Pins: hand-worked two-token cases
(exp evaluated with math.exp), reduction of the all-/none-refined cases to
PyTorch's scaled_dot_product_attention on the (b+r)-bit / b-bit dequantised
cache, closed forms (T = 1, q = 0), hand-worked summed-softmax scores, and the
query-head -> KV-head mapping.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, selection, nested


def _cache(K, V, b=2, r=2):
    return attention.quantize_kv(K, b, r), attention.quantize_kv(V, b, r)


def _two_token_case():
    # d = 4 keeps the hand arithmetic short.  Rows quantise exactly:
    # [0.9375, 0, 0, 0] -> s = 0.0625, z = 0, code 15 -> resident 0.75, full 0.9375.
    K = np.zeros((1, 1, 2, 4), dtype=np.float32)
    K[0, 0, 0, 0] = 0.9375
    K[0, 0, 1, 1] = 0.9375
    V = np.zeros((1, 1, 2, 4), dtype=np.float32)
    V[0, 0, 0] = [-0.5, -0.3, 0.1, 0.4375]  # resident [-.5,-.5,0,.25], full [-.5,-.3125,.125,.4375]
    V[0, 0, 1, 1] = 0.9375  # resident [0,.75,0,0], full [0,.9375,0,0]
    return K, V


V0_RES = [-0.5, -0.5, 0.0, 0.25]
V0_FULL = [-0.5, -0.3125, 0.125, 0.4375]
V1_RES = [0.0, 0.75, 0.0, 0.0]
V1_FULL = [0.0, 0.9375, 0.0, 0.0]


def test_two_tokens_positive_query():
    K, V = _two_token_case()
    qk, qv = _cache(K, V)
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]], dtype=np.float16)
    # resident logits 0.75, 0 -> token 0 selected; its refined logit is 0.9375
    out, sel = attention.refined_attention(q, qk, qv, (1, 1, 2, 4), 1.0, 1)
    assert sel[(0, 0)] == [0]
    w0 = math.exp(0.9375) / (math.exp(0.9375) + 1.0)
    exp = [w0 * a + (1 - w0) * b for a, b in zip(V0_FULL, V1_RES)]
    np.testing.assert_allclose(out[0, 0], exp, rtol=1e-14, atol=1e-15)
    # nothing selected: resident everywhere
    out0, _ = attention.refined_attention(q, qk, qv, (1, 1, 2, 4), 1.0, 0)
    w0 = math.exp(0.75) / (math.exp(0.75) + 1.0)
    exp0 = [w0 * a + (1 - w0) * b for a, b in zip(V0_RES, V1_RES)]
    np.testing.assert_allclose(out0[0, 0], exp0, rtol=1e-14, atol=1e-15)
    # selected but missing from the cache: resident precision
    outm, _ = attention.refined_attention(q, qk, qv, (1, 1, 2, 4), 1.0, 1, hits={(0, 0): set()})
    np.testing.assert_allclose(outm[0, 0], exp0, rtol=1e-14, atol=1e-15)


def test_two_tokens_negative_query_and_scale():
    K, V = _two_token_case()
    qk, qv = _cache(K, V)
    q = np.array([[[-1.0, 0.0, 0.0, 0.0]]], dtype=np.float16)
    # resident logits -0.75*0.5, 0 -> token 1 selected; its refined logit stays 0
    out, sel = attention.refined_attention(q, qk, qv, (1, 1, 2, 4), 0.5, 1)
    assert sel[(0, 0)] == [1]
    w0 = math.exp(-0.375) / (math.exp(-0.375) + 1.0)
    exp = [w0 * a + (1 - w0) * b for a, b in zip(V0_RES, V1_FULL)]
    np.testing.assert_allclose(out[0, 0], exp, rtol=1e-14, atol=1e-15)


def test_summed_softmax_scores_by_hand():
    k_res = np.eye(3, 4)
    q = np.array([[4.0, 0.0, 0.0, 0.0], [0.0, 2.0, 1.5, 0.0]], dtype=np.float16)
    sc = attention.token_scores(q, k_res, 1.0)
    ea = [math.exp(4.0), 1.0, 1.0]  # logits 4, 0, 0
    ea = [v / sum(ea) for v in ea]
    eb = [1.0, math.exp(2.0), math.exp(1.5)]  # logits 0, 2, 1.5
    eb = [v / sum(eb) for v in eb]
    np.testing.assert_allclose(sc, [a + b for a, b in zip(ea, eb)], rtol=1e-14)
    # a token with moderate weight from both heads outranks one with a single peak
    k2 = np.eye(3, 4)
    q2 = np.array([[1.0, 1.2, 0, 0], [1.0, 0, 1.2, 0]], dtype=np.float16)
    s2 = attention.token_scores(q2, k2, 1.0)
    assert s2[0] > s2[1] and s2[0] > s2[2]


def test_negligible_weights_score_zero_and_tie_to_lower_tokens():
    """A head's weight counts in the score only while the token's logit is within 64
    of the head's maximum: logits 0, -10, -63.5, -70, -80 (one head) score their
    softmax weights for the first three and exactly 0 for the last two, which then
    tie and go to the lower token."""
    k_res = np.zeros((5, 4))
    k_res[:, 0] = [0.0, -10.0, -63.5, -70.0, -80.0]
    q = np.array([[1.0, 0.0, 0.0, 0.0]], dtype=np.float16)
    sc = attention.token_scores(q, k_res, 1.0)
    e = [math.exp(v) for v in (0.0, -10.0, -63.5, -70.0, -80.0)]
    z = sum(e)
    np.testing.assert_allclose(sc[:3], [v / z for v in e[:3]], rtol=1e-14)
    assert sc[3] == 0.0 and sc[4] == 0.0
    assert selection.top_k(sc, 4) == [0, 1, 2, 3]
    # with two heads a token keeps the weight of the head that still sees it
    q2 = np.array([[1.0, 0.0, 0.0, 0.0], [-1.0, 0.0, 0.0, 0.0]], dtype=np.float16)
    s2 = attention.token_scores(q2, k_res, 1.0)
    e2 = [math.exp(-v - 80.0) for v in (0.0, -10.0, -63.5, -70.0, -80.0)]  # head 2: logits 0..80, max 80
    np.testing.assert_allclose(s2[4], 1.0 / sum(e2) + 0.0, rtol=1e-14)
    assert s2[0] == e[0] / z  # head 2 sees token 0 at 80 below its max: nothing added


def _sdpa(q_f16, Kd, Vd, scale):
    """PyTorch's attention on dense fp64 K/V with the KV heads repeated."""
    b, nq, d = q_f16.shape
    nkv = Kd.shape[1]
    G = nq // nkv
    q = torch.from_numpy(q_f16.astype(np.float64)).unsqueeze(2)  # [b][nq][1][d]
    k = torch.from_numpy(Kd).repeat_interleave(G, dim=1)
    v = torch.from_numpy(Vd).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    return o[:, :, 0].numpy()


@pytest.mark.parametrize("G", [1, 4])
def test_all_and_none_reduce_to_sdpa(G):
    g = np.random.default_rng(7)
    batch, nkv, T, d = 2, 2, 37, 128
    K = g.standard_normal((batch, nkv, T, d)).astype(np.float32)
    V = g.standard_normal((batch, nkv, T, d)).astype(np.float32)
    q = g.standard_normal((batch, nkv * G, d)).astype(np.float16)
    qk, qv = _cache(K, V)
    scale = 1.0 / math.sqrt(d)
    out_all, sel = attention.refined_attention(q, qk, qv, (batch, nkv, T, d), scale, T)
    assert all(v == list(range(T)) for v in sel.values())
    shp = (batch, nkv, T, d)
    ref_all = _sdpa(q, nested.dequant_full(qk).reshape(shp), nested.dequant_full(qv).reshape(shp), scale)
    np.testing.assert_allclose(out_all, ref_all, rtol=1e-12, atol=1e-12)
    out_none, _ = attention.refined_attention(q, qk, qv, shp, scale, 0)
    ref_none = _sdpa(q, nested.dequant_resident(qk).reshape(shp), nested.dequant_resident(qv).reshape(shp), scale)
    np.testing.assert_allclose(out_none, ref_none, rtol=1e-12, atol=1e-12)
    # refined sits between: differs from both for a partial selection
    out_part, _ = attention.refined_attention(q, qk, qv, shp, scale, 5)
    assert not np.allclose(out_part, out_all) and not np.allclose(out_part, out_none)


def test_closed_forms():
    g = np.random.default_rng(8)
    d = 128
    K = g.standard_normal((1, 2, 1, d)).astype(np.float32)
    V = g.standard_normal((1, 2, 1, d)).astype(np.float32)
    qk, qv = _cache(K, V)
    q = g.standard_normal((1, 8, d)).astype(np.float16)
    # T = 1: every head returns its KV head's single value vector (refined: selected)
    out, _ = attention.refined_attention(q, qk, qv, (1, 2, 1, d), 0.1, 1)
    full = nested.dequant_full(qv).reshape(1, 2, 1, d)
    for h in range(8):
        np.testing.assert_allclose(out[0, h], full[0, h // 4, 0], rtol=1e-14)
    # q = 0: uniform weights, ties -> first k tokens selected, output = mean
    T = 9
    K = g.standard_normal((1, 1, T, d)).astype(np.float32)
    V = g.standard_normal((1, 1, T, d)).astype(np.float32)
    qk, qv = _cache(K, V)
    q0 = np.zeros((1, 2, d), dtype=np.float16)
    out, sel = attention.refined_attention(q0, qk, qv, (1, 1, T, d), 0.1, 3)
    assert sel[(0, 0)] == [0, 1, 2]
    veff = nested.dequant_resident(qv).reshape(T, d).copy()
    veff[:3] = nested.dequant_full(qv).reshape(T, d)[:3]
    np.testing.assert_allclose(out[0, 0], veff.mean(axis=0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out[0, 1], veff.mean(axis=0), rtol=1e-12, atol=1e-14)


def test_output_in_value_hull():
    g = np.random.default_rng(9)
    d, T = 128, 50
    K = g.standard_normal((1, 1, T, d)).astype(np.float32)
    V = g.standard_normal((1, 1, T, d)).astype(np.float32)
    qk, qv = _cache(K, V)
    q = (g.standard_normal((1, 4, d)) * 3).astype(np.float16)
    out, sel = attention.refined_attention(q, qk, qv, (1, 1, T, d), 1 / math.sqrt(d), 4)
    veff = nested.dequant_resident(qv).reshape(T, d).copy()
    s = sel[(0, 0)]
    veff[s] = nested.dequant_full(qv).reshape(T, d)[s]
    assert np.all(out[0] <= veff.max(axis=0) + 1e-12)
    assert np.all(out[0] >= veff.min(axis=0) - 1e-12)


def test_permuting_tokens():
    g = np.random.default_rng(11)
    d, T = 128, 40
    K = g.standard_normal((1, 1, T, d)).astype(np.float32)
    V = g.standard_normal((1, 1, T, d)).astype(np.float32)
    q = g.standard_normal((1, 4, d)).astype(np.float16)
    perm = g.permutation(T)
    o1, s1 = attention.refined_attention(q, *_cache(K, V), (1, 1, T, d), 0.09, 6)
    o2, s2 = attention.refined_attention(q, *_cache(K[:, :, perm], V[:, :, perm]), (1, 1, T, d), 0.09, 6)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    inv = np.argsort(perm)
    assert sorted(perm[s2[(0, 0)]].tolist()) == s1[(0, 0)]
    assert sorted(inv[s1[(0, 0)]].tolist()) == s2[(0, 0)]
