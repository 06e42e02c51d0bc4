"""Refined GQA decode attention over a low-bit KV cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

rag-lover.com StrataFlux summary, explainer dialogue (解説): the KV cache is
resident in low-bit form; the tokens that receive refinement bits are chosen by
the attention weight computed from the low-bit keys.  Limitations section: a
token whose refinement is missing stays at resident precision.

Readings (the pages give no formula):
* query head h reads KV head floor(h / G), G = n_q_heads / n_kv_heads;
* one selection per (batch, kv head): a token's score is the softmax weight of the
  low-bit logits summed over the G query heads that read that KV head, where a
  weight below e^-64 of its head's largest counts as zero;
* for the selected tokens that hit, both the key (for the logit) and the value use
  the (b+r)-bit dequantised vectors; every other token uses the resident b-bit
  ones; the softmax is taken over all T tokens after that replacement.
"""
from __future__ import annotations

import numpy as np

from . import nested, selection


def quantize_kv(k_or_v, b: int, r: int):
    """Quantise K or V [batch][n_kv][T][d] per token-head (one group of d values)."""
    x = np.asarray(k_or_v, dtype=np.float32)
    d = x.shape[-1]
    return nested.quantize(x.reshape(-1, d), b, r, group=d)


def _softmax_rows(logits):
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=-1, keepdims=True)


# A head's softmax weight below e^-64 of its largest weight counts as zero in the
# selection score (reading: such weights carry no usable signal, and kernels that
# form the weights in fp32 cannot rank them; tokens whose score is zero tie, and
# ties go to the lower token).
SCORE_CUTOFF = -64.0


def token_scores(q_f16, k_res, scale):
    """Selection scores of one (batch, kv head).

    q_f16 [G][d], k_res [T][d] (resident keys, fp64) -> per token
    sum over the G heads of softmax_t(scale * q_h . k_t), where a head contributes
    nothing for a token whose logit lies more than 64 below that head's maximum.
    """
    q = np.asarray(q_f16, dtype=np.float16).astype(np.float64)
    logits = scale * (q @ k_res.T)  # [G][T]
    w = _softmax_rows(logits)
    rel = logits - logits.max(axis=-1, keepdims=True)
    return np.where(rel >= SCORE_CUTOFF, w, 0.0).sum(axis=0)


def refined_attention(q_f16, qk, qv, shape, scale, k_sel, sel_in=None, hits=None):
    """Refined decode attention.

    q_f16   fp16 [batch][n_q][d]
    qk, qv  ``nested.quantize`` results of K and V with rows ordered
            (batch, kv head, token)
    shape   (batch, n_kv, T, d)
    sel_in  optional external selection: dict (b, kvh) -> token ids
    hits    optional dict (b, kvh) -> set of token ids whose refinement is present
            (default: every token's refinement is present)

    Returns (out fp64 [batch][n_q][d], selected dict (b, kvh) -> sorted token ids).
    """
    batch, n_kv, T, d = shape
    q_all = np.asarray(q_f16, dtype=np.float16)
    n_q = q_all.shape[1]
    G = n_q // n_kv
    k_res = nested.dequant_resident(qk).reshape(batch, n_kv, T, d)
    k_full = nested.dequant_full(qk).reshape(batch, n_kv, T, d)
    v_res = nested.dequant_resident(qv).reshape(batch, n_kv, T, d)
    v_full = nested.dequant_full(qv).reshape(batch, n_kv, T, d)
    out = np.zeros((batch, n_q, d), dtype=np.float64)
    chosen = {}
    for bi in range(batch):
        for g in range(n_kv):
            heads = list(range(g * G, (g + 1) * G))
            qg = q_all[bi, heads]
            if sel_in is not None:
                sel = sorted(int(t) for t in sel_in[(bi, g)])
            else:
                sel = selection.top_k(token_scores(qg, k_res[bi, g], scale), k_sel)
            chosen[(bi, g)] = sel
            present = set(range(T)) if hits is None else set(hits.get((bi, g), ()))
            refined = np.zeros(T, dtype=bool)
            for t in sel:
                if t in present:
                    refined[t] = True
            k_eff = np.where(refined[:, None], k_full[bi, g], k_res[bi, g])
            v_eff = np.where(refined[:, None], v_full[bi, g], v_res[bi, g])
            qf = qg.astype(np.float64)
            w = _softmax_rows(scale * (qf @ k_eff.T))  # [G][T]
            out[bi, heads] = w @ v_eff
    return out, chosen
