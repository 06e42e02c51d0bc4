"""Pins for the oracle's nested quantisation and packing (CPU only).

Each test checks the oracle against something outside itself: hand-derived worked
examples (tests/golden/worked_examples.json), an independent fp16 rounding
(Python's struct 'e' format, round-half-even), a textbook min-max round-to-nearest
quantiser written with scalar Python, and the bounds the nested representation
must satisfy (refinement bits subdivide the cell between resident levels, per the
rag-lover.com StrataFlux summary's explainer dialogue).
"""
import math
import struct

import numpy as np
import pytest

from oracle import nested


def _py_fp16(v: float) -> float:
    """Independent fp16 rounding: CPython packs binary16 with round-half-even."""
    return struct.unpack("<e", struct.pack("<e", v))[0]


def test_fp16_rounding_matches_struct():
    g = np.random.default_rng(1)
    vals = list(g.standard_normal(2000) * 10.0 ** g.integers(-6, 4, 2000))
    # exact half-way points between fp16 neighbours, and points just beside them
    for base in (1.0, 1.5, 2.0 ** -14, 1000.0):
        ulp = math.ulp(base) * 2 ** (52 - 10) if base >= 2 ** -14 else 2 ** -24
        vals += [base + ulp / 2, base + ulp / 2 + 1e-12 * base, base + 1.5 * ulp]
    got = nested.fp16_rne(np.array(vals))
    for v, h in zip(vals, got):
        assert float(h) == _py_fp16(v)


def test_worked_example_2bit(golden):
    ex = golden["nested_2bit"]
    x = np.array([ex["x"]], dtype=np.float32)
    q = nested.quantize(x, ex["b"], ex["r"], ex["group"])
    assert float(q["zero"][0, 0]) == ex["zero"]
    assert float(q["scale"][0, 0]) == ex["scale"]
    assert q["codes"][0].tolist() == ex["codes"]
    hi, lo = nested.split(q)
    assert hi[0].tolist() == ex["resident_codes"]
    assert lo[0].tolist() == ex["refine_codes"]
    assert nested.dequant_full(q)[0].tolist() == ex["full_value"]
    assert nested.dequant_resident(q)[0].tolist() == ex["resident_value"]
    res, ref = nested.pack_rows(q)
    assert res[0].tolist() == ex["resident_bytes"]
    assert ref[0].tolist() == ex["refine_bytes"]


def test_worked_example_3bit_straddle(golden):
    ex = golden["nested_3bit_straddle"]
    x = np.array([ex["x_over_0.0625"]], dtype=np.float32) * np.float32(0.0625)
    q = nested.quantize(x, ex["b"], ex["r"], ex["group"])
    assert q["codes"][0].tolist() == ex["codes"]
    hi, lo = nested.split(q)
    assert hi[0].tolist() == ex["resident_codes"]
    assert lo[0].tolist() == ex["refine_codes"]
    res, ref = nested.pack_rows(q)
    assert res[0].tolist() == ex["resident_bytes"]
    assert ref[0].tolist() == ex["refine_bytes"]


def _textbook_rtn(row, bits, group):
    """Min-max asymmetric round-to-nearest, scalar Python, fp16 step/offset."""
    Q = 2 ** bits - 1
    out = []
    for g0 in range(0, len(row), group):
        grp = [float(v) for v in row[g0 : g0 + group]]
        lo, hi = min(grp), max(grp)
        z = _py_fp16(lo)
        s = _py_fp16((hi - lo) / Q)
        for v in grp:
            if s == 0.0:
                out.append(0)
            else:
                out.append(min(max(round((v - z) / s), 0), Q))
    return out


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_r0_is_textbook_rtn(bits):
    g = np.random.default_rng(bits)
    x = (g.standard_normal((3, 256)) * 0.02).astype(np.float32)
    x[1, 128:] = 0.25  # a constant group
    q = nested.quantize(x, bits, 0, 128)
    for i in range(3):
        assert q["codes"][i].tolist() == _textbook_rtn(x[i], bits, 128)
    # r = 0: resident value == full value
    assert np.array_equal(nested.dequant_resident(q), nested.dequant_full(q))


@pytest.mark.parametrize("b,r", [(2, 2), (3, 1), (2, 1), (1, 3), (4, 4), (2, 0)])
def test_nesting_bounds(b, r):
    g = np.random.default_rng(10 * b + r)
    x = (g.standard_normal((8, 512)) * 0.02).astype(np.float32)
    x[0, :128] *= 50
    q = nested.quantize(x, b, r, 128)
    full = nested.dequant_full(q)
    res = nested.dequant_resident(q)
    s = np.repeat(q["scale"].astype(np.float64), 128, axis=1)
    z = np.repeat(q["zero"].astype(np.float64), 128, axis=1)
    Q = 2 ** (b + r) - 1
    # refinement subdivides the resident cell: res <= full <= res + (2^r - 1) s
    assert np.all(res <= full)
    assert np.all(full <= res + (2 ** r - 1) * s)
    # inside the representable range the full code is within half a step
    inside = (x >= z) & (x <= z + Q * s)
    assert np.all(np.abs(x - full)[inside] <= s[inside] / 2 + 1e-15)
    assert inside.mean() > 0.95
    # the resident value is the full value with the refinement bits cleared
    hi, lo = nested.split(q)
    assert np.array_equal(hi * 2 ** r + lo, q["codes"])
    assert np.all(q["codes"] <= Q) and np.all(q["codes"] >= 0)


def test_degenerate_group():
    x = np.zeros((1, 256), dtype=np.float32)
    x[0, 128:] = 3.0
    q = nested.quantize(x, 2, 2, 128)
    assert np.all(q["codes"] == 0)
    assert nested.dequant_full(q)[0, 0] == 0.0 and nested.dequant_full(q)[0, 200] == 3.0
    assert np.array_equal(nested.dequant_resident(q), nested.dequant_full(q))


def _manual_stream(codes, width):
    """Bit stream by explicit integer shifts (independent of numpy's packbits)."""
    acc = 0
    for i, c in enumerate(codes):
        acc |= int(c) << (i * width)
    nbytes = len(codes) * width // 8
    return [(acc >> (8 * j)) & 0xFF for j in range(nbytes)]


@pytest.mark.parametrize("width", [1, 2, 3, 4, 5, 8])
def test_pack_bits_is_lsb_first_stream(width):
    g = np.random.default_rng(width)
    codes = g.integers(0, 2 ** width, size=(4, 64))
    packed = nested.pack_bits(codes, width)
    for i in range(4):
        assert packed[i].tolist() == _manual_stream(codes[i], width)
    assert np.array_equal(nested.unpack_bits(packed, width, 64), codes)


def test_weight_refinement_is_channel_major():
    g = np.random.default_rng(5)
    x = (g.standard_normal((32, 256)) * 0.02).astype(np.float32)
    q = nested.quantize(x, 2, 2, 128)
    p = nested.pack_weight(q)
    assert p["resident"].shape == (32, 64)
    assert p["refine"].shape == (256, 8)
    _, lo = nested.split(q)
    for k in (0, 7, 255):
        assert p["refine"][k].tolist() == _manual_stream(lo[:, k], 2)
