"""Refined GEMV: low-bit resident weights plus refinement bits on chosen channels.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

rag-lover.com StrataFlux summary, explainer dialogue (解説), and the paper's
abstract (arXiv 2611.08363): the resident low-bit weight is used everywhere; for
the input channels whose refinement is present on the GPU (selected by activation
magnitude and found in the cache) the refined value is used instead.  Limitations
section of the same summary: a channel whose refinement is missing stays at
resident precision.

y[b][n] = sum_k x[b][k] * Weff[n][k],
Weff[:, k] = full (b+r)-bit value if k in E else resident value,
with E = selected channels that hit.  Accumulated in fp64 from the exact fp16 x.
"""
from __future__ import annotations

import numpy as np

from . import nested


def effective_weight(q, refined_channels):
    """Dense fp64 [N][K] weight with the refined value on ``refined_channels``."""
    w_res = nested.dequant_resident(q)
    w_full = nested.dequant_full(q)
    mask = np.zeros(w_res.shape[1], dtype=bool)
    mask[np.asarray(list(refined_channels), dtype=np.int64)] = True
    return np.where(mask[None, :], w_full, w_res)


def refined_gemv(q, x_f16, refined_channels):
    """y fp64 [batch][N] for input x fp16 [batch][K]."""
    x = np.asarray(x_f16, dtype=np.float16).astype(np.float64)
    if x.ndim == 1:
        x = x[None, :]
    w = effective_weight(q, refined_channels)
    return x @ w.T


def lag_delta(q, x_f16, late_channels):
    """Fetch lag: the contribution of refinements that arrive after their GEMV.

    rag-lover.com StrataFlux summary, explainer dialogue (解説), fetch lead / fetch
    lag passage: the addition of a refinement to the output may be delayed until a
    later update, so that its transfer overlaps computation.  Reading: for the
    channels in ``late_channels`` (selected, missing when the GEMV ran, fetched
    afterwards) the output misses x_k * (full - resident)[n][k]; that amount is
    added at a later update of the same output.  Returns it, fp64 [batch][N]:
      delta[b][n] = sum_{k in late} x[b][k] * (Wfull[n][k] - Wres[n][k]).
    """
    x = np.asarray(x_f16, dtype=np.float16).astype(np.float64)
    if x.ndim == 1:
        x = x[None, :]
    late = np.asarray(sorted(set(int(k) for k in late_channels)), dtype=np.int64)
    n_out = q["codes"].shape[0]
    if late.size == 0:
        return np.zeros((x.shape[0], n_out))
    d = nested.dequant_full(q)[:, late] - nested.dequant_resident(q)[:, late]
    return x[:, late] @ d.T
