"""Decode-step glue around the refined ops, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The pages describe the refined GEMV and attention but not the rest of a decoder
step.  The glue here follows the public definitions of the two model families the
workloads are shaped after (Llama-3.1 and Qwen3 decoder layers); the readings
taken are:

* RMSNorm: ``y = x / sqrt(mean(x^2) + eps) * w`` over the last axis;
* Qwen3 normalises each query and key head with its own RMSNorm (weight of length
  head_dim) before the rotary embedding; Llama does not;
* rotary embedding in the rotate-half form: dims ``i`` and ``i + d/2`` of a head
  form a pair rotated by the angle ``pos * theta^(-2i/d)``;
* SwiGLU feed-forward: ``act = silu(gate) * up`` with ``silu(x) = x / (1 + e^-x)``;
* the residual stream is kept in fp32; every GEMV input is the fp16 rounding
  (nearest-even) of its fp32/fp64 value;
* greedy decoding: ``argmax`` returns the lowest index among equal maxima.

One decoder layer (as the decode-step tests compose these functions with the
refined GEMV and attention) reads ``h``, and in order: ``x = fp16(rmsnorm(h))``,
q/k/v = refined GEMVs of x, q/k head norms (Qwen3) and rotary embedding at ``pos``,
the new k, v appended to the cache, refined attention of fp16(q) over the cache,
``h += W_o fp16(attn)``, ``x2 = fp16(rmsnorm(h))``, ``act = fp16(swiglu(W_g x2,
W_u x2))``, ``h += W_d act``.
"""
from __future__ import annotations

import numpy as np


def rmsnorm(x, w, eps):
    """x / sqrt(mean(x^2) + eps) * w over the last axis, fp64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope(x, pos, theta):
    """Rotary embedding (rotate-half pairs (i, i + d/2)) of x [..., d] at position pos."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    ang = pos * np.power(float(theta), -2.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu(gate, up):
    return silu(gate) * np.asarray(up, dtype=np.float64)


def embed(table_f16, ids):
    """Rows of the fp16 embedding table, as fp64 [len(ids)][hidden]."""
    return np.asarray(table_f16, dtype=np.float16)[np.asarray(ids, dtype=np.int64)].astype(np.float64)


def argmax(logits):
    """Per row, the index of the largest value (lowest index among equals)."""
    logits = np.asarray(logits, dtype=np.float64)
    return np.argmax(logits, axis=-1)  # numpy returns the first occurrence


def to_f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def qk_heads(q, k, n_q, n_kv, d, q_norm_w, k_norm_w, eps, pos, theta):
    """q [batch][n_q*d], k [batch][n_kv*d] (GEMV outputs) -> per-head normalised (if
    weights are given) and rotated q [batch][n_q][d], k [batch][n_kv][d], fp64."""
    q = np.asarray(q, dtype=np.float64).reshape(-1, n_q, d)
    k = np.asarray(k, dtype=np.float64).reshape(-1, n_kv, d)
    if q_norm_w is not None:
        q = rmsnorm(q, q_norm_w, eps)
    if k_norm_w is not None:
        k = rmsnorm(k, k_norm_w, eps)
    return rope(q, pos, theta), rope(k, pos, theta)
