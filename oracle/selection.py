"""Refinement selection: which input channels / tokens get their refinement bits.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

rag-lover.com StrataFlux summary, explainer dialogue (解説): weight refinements
are chosen by the magnitude of the input activation, KV refinements by the
attention weight computed from the low-bit keys.  The pages state no count or tie
rule; readings: ``k_sel = ceil(p * n / 100)`` (at least p percent) and ties go to
the lower index.
"""
from __future__ import annotations

import numpy as np


def k_select(percent: int, n: int) -> int:
    """ceil(percent * n / 100) in integer arithmetic."""
    return (percent * n + 99) // 100


def top_k(scores, k: int):
    """Indices of the k largest ``scores``, ties to the lower index, returned sorted
    ascending.  Plain ordering by (-score, index)."""
    scores = [float(v) for v in np.asarray(scores).ravel()]
    order = sorted(range(len(scores)), key=lambda i: (-scores[i], i))
    return sorted(order[:k])


def channel_scores(x_f16):
    """Per input channel: max over the batch rows of |x| (exact on fp16 values).

    Reading for batch > 1: one shared channel set per GEMV call, because one
    fetched refinement unit (an input channel's bits for every output row) serves
    all rows of the batch; the maximum is exact in any precision.
    """
    x = np.asarray(x_f16, dtype=np.float16).astype(np.float64)
    if x.ndim == 1:
        x = x[None, :]
    return np.abs(x).max(axis=0)


def select_channels(x_f16, k: int):
    """Top-k input channels by activation magnitude, sorted ascending."""
    return top_k(channel_scores(x_f16), k)
