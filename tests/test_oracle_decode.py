"""Pins of the decode-step glue oracle (CPU): closed forms, independent restatements
(complex rotation for the rotary embedding) and special values."""
import math

import numpy as np

from oracle import decode


def test_rmsnorm_closed_forms():
    # mean of squares of (3, 4) is 12.5; rms = sqrt(12.5)
    y = decode.rmsnorm([3.0, 4.0], [1.0, 1.0], 0.0)
    assert np.allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    # the weight scales per position; eps enters under the root
    y = decode.rmsnorm([[2.0, 2.0, 2.0, 2.0]], [1.0, 2.0, 3.0, 4.0], 5.0)
    assert np.allclose(y, [[2 / 3, 4 / 3, 2.0, 8 / 3]], rtol=0, atol=1e-15)
    # scale invariance without eps
    x = np.random.default_rng(0).standard_normal((3, 64))
    assert np.allclose(decode.rmsnorm(x, np.ones(64), 0.0), decode.rmsnorm(7.5 * x, np.ones(64), 0.0))


def test_rope_is_a_complex_rotation():
    rng = np.random.default_rng(1)
    d, theta = 128, 10000.0
    x = rng.standard_normal((2, 3, d))
    for pos in (0, 1, 17, 4095):
        y = decode.rope(x, pos, theta)
        # pair (i, i + d/2) as the complex number x_i + j x_{i+d/2}, times e^{j pos w_i}
        zc = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos * theta ** (-np.arange(0, d, 2) / d))
        assert np.allclose(y[..., : d // 2], zc.real, atol=1e-12)
        assert np.allclose(y[..., d // 2:], zc.imag, atol=1e-12)
        assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
    assert np.array_equal(decode.rope(x, 0, theta), x)


def test_rope_first_pair_angle_is_pos():
    x = np.zeros(128)
    x[0] = 1.0
    y = decode.rope(x, 1, 1e6)
    assert math.isclose(y[0], math.cos(1.0), abs_tol=1e-15) and math.isclose(y[64], math.sin(1.0), abs_tol=1e-15)


def test_swiglu_special_values():
    assert decode.silu(0.0) == 0.0
    # silu(ln 3) = ln 3 * 3/4
    assert math.isclose(float(decode.silu(math.log(3.0))), math.log(3.0) * 0.75, rel_tol=1e-15)
    assert math.isclose(float(decode.silu(-math.log(3.0))), -math.log(3.0) * 0.25, rel_tol=1e-15)
    assert math.isclose(float(decode.swiglu(math.log(3.0), 2.0)), math.log(3.0) * 1.5, rel_tol=1e-15)
    assert float(decode.silu(-800.0)) == 0.0 and float(decode.silu(800.0)) == 800.0


def test_argmax_takes_the_lowest_index_among_equals():
    assert decode.argmax([[1.0, 5.0, 5.0, 2.0], [7.0, 7.0, -1.0, 7.0]]).tolist() == [1, 0]


def test_embed_gathers_fp16_rows():
    t = np.arange(12, dtype=np.float16).reshape(4, 3) / np.float16(8)
    assert np.array_equal(decode.embed(t, [2, 0]), t[[2, 0]].astype(np.float64))


def test_qk_heads_norm_then_rotate():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 4 * 128))
    k = rng.standard_normal((1, 2 * 128))
    wq, wk = rng.uniform(0.5, 1.5, 128), rng.uniform(0.5, 1.5, 128)
    qh, kh = decode.qk_heads(q, k, 4, 2, 128, wq, wk, 1e-6, 9, 1e6)
    assert np.allclose(qh[0, 3], decode.rope(decode.rmsnorm(q[0, 384:], wq, 1e-6), 9, 1e6))
    assert np.allclose(kh[0, 1], decode.rope(decode.rmsnorm(k[0, 128:], wk, 1e-6), 9, 1e6))
    qh2, _ = decode.qk_heads(q, k, 4, 2, 128, None, None, 1e-6, 0, 1e6)
    assert np.array_equal(qh2[0].reshape(-1), q[0])
