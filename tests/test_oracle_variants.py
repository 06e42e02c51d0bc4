"""Pins for the oracle's comparison variants (CPU only): the worked row, cases that
reduce to plain fp16 arithmetic or to the refined path, closed forms."""
import math

import numpy as np
import pytest

from oracle import attention, nested, selection, variants


def test_fp16_fetch_worked_row(golden):
    """The worked row with x = (1, 2, -1, 0.5), channel 1 fetched as fp16:
    fp16(-0.3) = -(1 + 205/1024) / 4 = -0.300048828125, so the resident output -1.375
    moves by 2 * (-0.300048828125 - (-0.5)) = 0.39990234375."""
    ex = golden["nested_2bit"]
    gx = golden["gemv_row"]
    W = np.array([ex["x"]], dtype=np.float32)
    q = nested.quantize(W, ex["b"], ex["r"], ex["group"])
    x = np.array([gx["x"]], dtype=np.float16)
    assert float(np.float16(np.float32(-0.3))) == -0.300048828125
    assert variants.fp16_fetch_gemv(W, q, x, [])[0, 0] == gx["y_none"]
    assert variants.fp16_fetch_gemv(W, q, x, [1])[0, 0] == -0.97509765625


def test_fp16_fetch_all_channels_is_the_fp16_gemv():
    g = np.random.default_rng(1)
    W = (g.standard_normal((24, 256)) * 0.02).astype(np.float32)
    x = g.standard_normal((2, 256)).astype(np.float16)
    q = nested.quantize(W, 2, 2, 128)
    y = variants.fp16_fetch_gemv(W, q, x, range(256))
    w16 = W.astype(np.float16).astype(np.float64)
    for bi in range(2):
        for n in range(24):
            want = math.fsum(float(x[bi, k]) * w16[n, k] for k in range(256))
            assert y[bi, n] == pytest.approx(want, rel=1e-12, abs=1e-13)


def _kv(seed, batch, n_kv, T, d=128):
    g = np.random.default_rng(seed)
    K = g.standard_normal((batch, n_kv, T, d)).astype(np.float32)
    V = g.standard_normal((batch, n_kv, T, d)).astype(np.float32)
    q = g.standard_normal((batch, 4 * n_kv, d)).astype(np.float16)
    return K, V, q, attention.quantize_kv(K, 2, 2), attention.quantize_kv(V, 2, 2)


def test_sparse_attention_with_every_token_is_the_refined_path():
    K, V, q, qk, qv = _kv(2, 1, 2, 40)
    shape, sc = (1, 2, 40, 128), 1 / math.sqrt(128)
    a, _ = variants.sparse_attention(q, qk, qv, shape, sc, 40)
    b, _ = attention.refined_attention(q, qk, qv, shape, sc, 40)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_sparse_attention_closed_forms():
    """k = 1: the output is the one selected token's (b+r)-bit value (a miss: its
    resident value); two tokens: weights e^l / (e^l0 + e^l1) written out."""
    K, V, q, qk, qv = _kv(3, 1, 1, 30)
    shape, sc = (1, 1, 30, 128), 1 / math.sqrt(128)
    out, sel = variants.sparse_attention(q, qk, qv, shape, sc, 1)
    t = sel[(0, 0)][0]
    v_full = nested.dequant_full(qv).reshape(30, 128)
    v_res = nested.dequant_resident(qv).reshape(30, 128)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], v_full[t], rtol=0, atol=1e-15)
    out_m, _ = variants.sparse_attention(q, qk, qv, shape, sc, 1, hits={(0, 0): set()})
    np.testing.assert_allclose(out_m[0, 0], v_res[t], rtol=0, atol=1e-15)
    out2, sel2 = variants.sparse_attention(q, qk, qv, shape, sc, 2)
    t0, t1 = sel2[(0, 0)]
    k_full = nested.dequant_full(qk).reshape(30, 128)
    for h in range(4):
        l0 = sc * float(q[0, h].astype(np.float64) @ k_full[t0])
        l1 = sc * float(q[0, h].astype(np.float64) @ k_full[t1])
        w0 = 1.0 / (1.0 + math.exp(l1 - l0))
        np.testing.assert_allclose(out2[0, h], w0 * v_full[t0] + (1 - w0) * v_full[t1], rtol=1e-12, atol=1e-13)


def test_fp16_token_attention_reductions():
    """Every token selected and present: plain attention on fp16(K), fp16(V) (written
    out with a per-token loop); none selected: the refined path with none selected."""
    K, V, q, qk, qv = _kv(4, 1, 2, 24)
    shape, sc = (1, 2, 24, 128), 1 / math.sqrt(128)
    out, _ = variants.fp16_token_attention(q, qk, qv, K, V, shape, sc, 24)
    k16 = K.astype(np.float16).astype(np.float64)
    v16 = V.astype(np.float16).astype(np.float64)
    for h in range(8):
        g = h // 4
        ls = [sc * math.fsum(float(q[0, h, i]) * k16[0, g, t, i] for i in range(128)) for t in range(24)]
        m = max(ls)
        ws = [math.exp(l - m) for l in ls]
        z = math.fsum(ws)
        want = sum(w / z * v16[0, g, t] for t, w in enumerate(ws))
        np.testing.assert_allclose(out[0, h], want, rtol=1e-11, atol=1e-12)
    none, _ = variants.fp16_token_attention(q, qk, qv, K, V, shape, sc, 0)
    ref, _ = attention.refined_attention(q, qk, qv, shape, sc, 0)
    np.testing.assert_allclose(none, ref, rtol=1e-12, atol=1e-13)


def test_variants_select_like_the_refined_path():
    K, V, q, qk, qv = _kv(5, 2, 2, 50)
    shape, sc = (2, 2, 50, 128), 1 / math.sqrt(128)
    _, s_ref = attention.refined_attention(q, qk, qv, shape, sc, 7)
    _, s_sp = variants.sparse_attention(q, qk, qv, shape, sc, 7)
    _, s_16 = variants.fp16_token_attention(q, qk, qv, K, V, shape, sc, 7)
    assert s_ref == s_sp == s_16
