"""The methods the StrataFlux pages compare against, on the same resident data.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

rag-lover.com StrataFlux summary, "既存手法との違い" (differences from existing
methods) and the explainer dialogue: besides nested refinement, the paper compares
fetching FP16 values instead of refinement bits (FP16 fetch), replacing the
selected tokens by their FP16 keys and values (SpeCache), dropping the tokens that
were not selected (sparse attention) and choosing the refined units at random
(random selection).  The pages define none of them further; the readings here keep
everything but the named difference equal to the refined path:

* same selection rule (channel top-k by max |x|; token top-k by the summed low-bit
  softmax weight), same cache semantics (E = the selected units that hit);
* FP16 fetch (weights): for k in E the weight column is fp16(W[:, k]) (one
  nearest-even rounding of the original fp32 weight) instead of the (b+r)-bit
  value; every other column stays resident;
* SpeCache-style replacement (KV): for t in E the key and value are fp16(K[t]),
  fp16(V[t]) instead of the (b+r)-bit vectors; the softmax runs over all tokens;
* sparse attention: only the selected tokens are attended (softmax over S), with
  the (b+r)-bit key and value where they hit and the resident ones where they
  missed; unselected tokens are dropped instead of kept at resident precision;
* random selection: the selected set is drawn at random (an input, see
  ``bit_decode_selective_amd.inputs.random_selection``) and fed to the refined
  GEMV / attention as an external selection: no arithmetic of its own.
"""
from __future__ import annotations

import numpy as np

from . import attention, nested, selection


def fp16_fetch_gemv(W, q, x_f16, hit_channels):
    """y fp64 [batch][N]: resident weights except fp16(W) on the columns in E.

    W fp32 [N][K] (the weights the store was made from), q = nested.quantize(W, ..)."""
    x = np.asarray(x_f16, dtype=np.float16).astype(np.float64)
    if x.ndim == 1:
        x = x[None, :]
    w = nested.dequant_resident(q)
    cols = np.asarray(sorted(set(int(k) for k in hit_channels)), dtype=np.int64)
    if cols.size:
        w[:, cols] = np.asarray(W, dtype=np.float32)[:, cols].astype(np.float16).astype(np.float64)
    return x @ w.T


def _selection(qg, k_res, scale, k_sel, sel_in, key):
    if sel_in is not None:
        return sorted(int(t) for t in sel_in[key])
    return selection.top_k(attention.token_scores(qg, k_res, scale), k_sel)


def sparse_attention(q_f16, qk, qv, shape, scale, k_sel, sel_in=None, hits=None):
    """Attention over the selected tokens only (unselected tokens dropped).

    Arguments as ``attention.refined_attention``.  Returns (out [batch][n_q][d],
    selected dict)."""
    batch, n_kv, T, d = shape
    q_all = np.asarray(q_f16, dtype=np.float16)
    G = q_all.shape[1] // n_kv
    k_res = nested.dequant_resident(qk).reshape(batch, n_kv, T, d)
    k_full = nested.dequant_full(qk).reshape(batch, n_kv, T, d)
    v_res = nested.dequant_resident(qv).reshape(batch, n_kv, T, d)
    v_full = nested.dequant_full(qv).reshape(batch, n_kv, T, d)
    out = np.zeros((batch, q_all.shape[1], d))
    chosen = {}
    for bi in range(batch):
        for g in range(n_kv):
            heads = list(range(g * G, (g + 1) * G))
            qg = q_all[bi, heads]
            sel = _selection(qg, k_res[bi, g], scale, k_sel, sel_in, (bi, g))
            chosen[(bi, g)] = sel
            if not sel:
                continue
            present = set(range(T)) if hits is None else set(hits.get((bi, g), ()))
            idx = np.asarray(sel, dtype=np.int64)
            hit = np.array([t in present for t in sel])
            k_eff = np.where(hit[:, None], k_full[bi, g, idx], k_res[bi, g, idx])
            v_eff = np.where(hit[:, None], v_full[bi, g, idx], v_res[bi, g, idx])
            logits = scale * (qg.astype(np.float64) @ k_eff.T)  # [G][|S|]
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            out[bi, heads] = (e / e.sum(axis=1, keepdims=True)) @ v_eff
    return out, chosen


def fp16_token_attention(q_f16, qk, qv, K, V, shape, scale, k_sel, sel_in=None, hits=None):
    """SpeCache-style: the selected tokens that hit use fp16(K[t]), fp16(V[t]).

    K, V fp32 [batch][n_kv][T][d] (what the cache was quantised from); other
    arguments as ``attention.refined_attention``."""
    batch, n_kv, T, d = shape
    q_all = np.asarray(q_f16, dtype=np.float16)
    G = q_all.shape[1] // n_kv
    k_res = nested.dequant_resident(qk).reshape(batch, n_kv, T, d)
    v_res = nested.dequant_resident(qv).reshape(batch, n_kv, T, d)
    k16 = np.asarray(K, dtype=np.float32).astype(np.float16).astype(np.float64)
    v16 = np.asarray(V, dtype=np.float32).astype(np.float16).astype(np.float64)
    out = np.zeros((batch, q_all.shape[1], d))
    chosen = {}
    for bi in range(batch):
        for g in range(n_kv):
            heads = list(range(g * G, (g + 1) * G))
            qg = q_all[bi, heads]
            sel = _selection(qg, k_res[bi, g], scale, k_sel, sel_in, (bi, g))
            chosen[(bi, g)] = sel
            present = set(range(T)) if hits is None else set(hits.get((bi, g), ()))
            rep = np.zeros(T, dtype=bool)
            for t in sel:
                rep[t] = t in present
            k_eff = np.where(rep[:, None], k16[bi, g], k_res[bi, g])
            v_eff = np.where(rep[:, None], v16[bi, g], v_res[bi, g])
            logits = scale * (qg.astype(np.float64) @ k_eff.T)
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            out[bi, heads] = (e / e.sum(axis=1, keepdims=True)) @ v_eff
    return out, chosen
