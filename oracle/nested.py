"""Nested (resident + refinement) quantisation, packing and dequantisation, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Follows the nested-refinement representation of the rag-lover.com StrataFlux
summary, explainer dialogue (解説): the resident value is a low-bit code, and the
refinement is a few extra bits that split the interval between neighbouring
resident levels.  The pages give no formula; the reading used here is the plain
one -- one (b+r)-bit asymmetric uniform code per value whose top b bits are
resident and whose low r bits are the refinement -- with group 128, fp16 step and
offset, and LSB-first packing.
"""
from __future__ import annotations

import numpy as np


def fp16_rne(v):
    """Round fp64 values once, to nearest-even, to fp16 (numpy converts directly)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16)


def quantize(x, b: int, r: int, group: int = 128):
    """Per-group asymmetric uniform quantisation of ``x`` [rows][cols] to B=b+r bits.

    For each run of ``group`` consecutive values of a row:
      m, M  = min, max of the group (exact, fp32 inputs);
      z     = fp16(m), s = fp16((M - m) / Q), Q = 2^B - 1, quotient taken in fp64;
      c     = clip(rint((x - z) / s), 0, Q) in fp64 (ties to even);
      a group with s == 0 (constant group, or a range that rounds to 0) gets c = 0.

    Returns a dict with int64 ``codes`` [rows][cols], fp16 ``zero`` and ``scale``
    [rows][cols/group], and the format.
    """
    if not (1 <= b and 0 <= r and b + r <= 8):
        raise ValueError("need 1 <= b, 0 <= r, b + r <= 8")
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % group:
        raise ValueError("cols must be a multiple of group")
    Q = 2 ** (b + r) - 1
    xg = x.astype(np.float64).reshape(rows, cols // group, group)
    m = xg.min(axis=2)
    M = xg.max(axis=2)
    z16 = fp16_rne(m)
    s16 = fp16_rne((M - m) / Q)
    z = z16.astype(np.float64)[..., None]
    s = s16.astype(np.float64)[..., None]
    codes = np.zeros(xg.shape, dtype=np.int64)
    live = np.broadcast_to((s16 != 0)[..., None], xg.shape)
    t = np.divide(xg - z, s, out=np.zeros_like(xg), where=live)
    codes[live] = np.clip(np.rint(t[live]), 0, Q).astype(np.int64)
    return {
        "codes": codes.reshape(rows, cols),
        "zero": z16,
        "scale": s16,
        "b": b,
        "r": r,
        "group": group,
    }


def split(q):
    """Resident (top b bits) and refinement (low r bits) codes of ``quantize``'s output."""
    r = q["r"]
    c = q["codes"]
    return c >> r, c & ((1 << r) - 1)


def _expand(v, group):
    """[rows][cols/group] per-group value -> [rows][cols] fp64."""
    return np.repeat(np.asarray(v, dtype=np.float64), group, axis=1)


def dequant_full(q):
    """(b+r)-bit value z + s*c, fp64 [rows][cols]."""
    g = q["group"]
    return _expand(q["zero"], g) + _expand(q["scale"], g) * q["codes"]


def dequant_resident(q):
    """Resident value z + (s * 2^r) * (c >> r): the lower edge of the cell, fp64."""
    g = q["group"]
    hi, _ = split(q)
    return _expand(q["zero"], g) + (_expand(q["scale"], g) * float(2 ** q["r"])) * hi


def to_f32(v):
    """fp32 exposure of an fp64 dequantised value (one round-to-nearest-even)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def pack_bits(codes, width: int):
    """LSB-first little-endian bit stream of ``codes`` along the last axis.

    Element i occupies bits [i*width, (i+1)*width) of the stream; stream bit j is
    bit (j % 8) of byte j // 8.  Returns uint8 [..., n*width/8].
    """
    codes = np.asarray(codes, dtype=np.int64)
    n = codes.shape[-1]
    if (n * width) % 8:
        raise ValueError("bit stream must fill whole bytes")
    if width == 0:
        return np.zeros(codes.shape[:-1] + (0,), dtype=np.uint8)
    bits = (codes[..., :, None] >> np.arange(width)) & 1
    bits = bits.reshape(codes.shape[:-1] + (n * width,)).astype(np.uint8)
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack_bits(packed, width: int, n: int):
    """Inverse of ``pack_bits``: uint8 [..., n*width/8] -> int64 [..., n]."""
    packed = np.asarray(packed, dtype=np.uint8)
    bits = np.unpackbits(packed, axis=-1, bitorder="little")[..., : n * width]
    bits = bits.reshape(packed.shape[:-1] + (n, width)).astype(np.int64)
    return (bits << np.arange(width)).sum(axis=-1)


def pack_weight(q):
    """Packed buffers of a weight matrix quantised with ``quantize``.

    resident   uint8 [N][K*b/8]   row-major, LSB-first stream of c>>r along K;
    refine     uint8 [K][N*r/8]   channel-major: unit k is the stream of the
                                  refinement codes of input channel k over all N
                                  output rows (one fetch unit per input channel);
    scale/zero fp16  [N][K/group].
    """
    hi, lo = split(q)
    return {
        "resident": pack_bits(hi, q["b"]),
        "refine": pack_bits(lo.T, q["r"]),
        "scale": q["scale"],
        "zero": q["zero"],
    }


def pack_rows(q):
    """Row-major packing (used for KV, one row per token-head): resident and
    refinement streams of each row."""
    hi, lo = split(q)
    return pack_bits(hi, q["b"]), pack_bits(lo, q["r"])
