"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module draws random numbers only: it holds none of the method's arithmetic
(no quantisation, selection, attention or cache logic), so the HIP path and the
CPU oracle can both be fed from it without sharing any computation.

The pages measure on trained Llama-3.1-8B-Instruct / Qwen3-8B weights and on
WikiText-2, PG-19 and AIME text; none of that is available here, so every input is
random with the model shapes of those runs:

* weights  N(0, 0.02) fp32, drawn per (config, layer, tensor);
* activations N(0, 1) fp32 with ceil(1% * K) outlier channels scaled by 20 (the
  same channels for every batch row and step), then rounded to fp16;
* K and V N(0, 1) fp32; K carries 4 high-variance dimensions per (layer, kv head)
  scaled by 8;
* queries N(0, 1) rounded to fp16.

Seeds: ``numpy.random.Generator(PCG64(SeedSequence([config, layer, tensor, step])))``.
"""
from __future__ import annotations

import numpy as np

# tensor ids used in seed keys
Q_PROJ, K_PROJ, V_PROJ, O_PROJ, GATE, UP, DOWN = range(7)
KV_CACHE, QUERY, OUTLIERS, HIDDEN, TOKENS, EMBED, LM_HEAD, NORM, RANDOM_SEL = range(7, 16)
KV_HOT_DIMS = 16


def rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def weight(cfg, layer, tensor, n_out, k_in, std=0.02):
    """fp32 [n_out][k_in] ~ N(0, std)."""
    g = rng(cfg, layer, tensor, 0)
    return (g.standard_normal((n_out, k_in), dtype=np.float32) * np.float32(std)).astype(np.float32)


def outlier_channels(cfg, layer, tensor, k_in, percent=1):
    """ceil(percent% * k_in) channels, uniform without replacement, sorted."""
    n = (percent * k_in + 99) // 100
    g = rng(cfg, layer, tensor, OUTLIERS)
    return np.sort(g.choice(k_in, size=n, replace=False))


def activation(cfg, layer, tensor, step, batch, k_in, outlier_scale=20.0, percent=1):
    """fp16 [batch][k_in]: N(0,1) with outlier channels x outlier_scale."""
    g = rng(cfg, layer, tensor, 1000 + step)
    x = g.standard_normal((batch, k_in), dtype=np.float32)
    if percent:
        idx = outlier_channels(cfg, layer, tensor, k_in, percent)
        x[:, idx] *= np.float32(outlier_scale)
    return x.astype(np.float16)


def kv(cfg, layer, batch, n_kv, T, d, hot_dims=4, hot_scale=8.0):
    """K, V fp32 [batch][n_kv][T][d] ~ N(0,1); per kv head, ``hot_dims`` dims of K x hot_scale."""
    g = rng(cfg, layer, KV_CACHE, 0)
    K = g.standard_normal((batch, n_kv, T, d), dtype=np.float32)
    V = g.standard_normal((batch, n_kv, T, d), dtype=np.float32)
    gh = rng(cfg, layer, KV_CACHE, KV_HOT_DIMS)
    for h in range(n_kv):
        dims = gh.choice(d, size=hot_dims, replace=False)
        K[:, h][..., dims] *= np.float32(hot_scale)
    return K, V


def query(cfg, layer, step, batch, n_q, d):
    """fp16 [batch][n_q][d] ~ N(0,1)."""
    g = rng(cfg, layer, QUERY, step)
    return g.standard_normal((batch, n_q, d), dtype=np.float32).astype(np.float16)


def hidden(cfg, step, batch, dim):
    """fp32 [batch][dim] ~ N(0,1): a synthetic residual-stream state."""
    g = rng(cfg, 0, HIDDEN, step)
    return g.standard_normal((batch, dim), dtype=np.float32)


def tokens(cfg, steps, batch, vocab):
    """int64 [steps][batch] uniform token ids (teacher-forced inputs)."""
    g = rng(cfg, 0, TOKENS, 0)
    return g.integers(0, vocab, size=(steps, batch), dtype=np.int64)


def norm_gain(cfg, layer, which, dim, percent=1, scale=20.0):
    """fp32 [dim] RMSNorm gains: 1, except ceil(percent% * dim) channels x scale."""
    gvec = np.ones(dim, dtype=np.float32)
    if percent:
        g = rng(cfg, layer, NORM, which)
        n = (percent * dim + 99) // 100
        gvec[g.choice(dim, size=n, replace=False)] = np.float32(scale)
    return gvec


# --- device-side bulk variants (throughput runs only; same distributions) ---------

def torch_weight(gen, n_out, k_in, std=0.02, device="cuda"):
    import torch

    return torch.randn((n_out, k_in), generator=gen, device=device, dtype=torch.float32) * std


def torch_activation(gen, batch, k_in, outliers, outlier_scale=20.0, device="cuda"):
    import torch

    x = torch.randn((batch, k_in), generator=gen, device=device, dtype=torch.float32)
    if outliers is not None and len(outliers):
        idx = torch.as_tensor(np.asarray(outliers), device=device, dtype=torch.long)
        x[:, idx] *= outlier_scale
    return x.to(torch.float16)


def torch_kv(gen, batch, n_kv, T, d, hot_dims=4, hot_scale=8.0, device="cuda"):
    import torch

    K = torch.randn((batch, n_kv, T, d), generator=gen, device=device, dtype=torch.float32)
    V = torch.randn((batch, n_kv, T, d), generator=gen, device=device, dtype=torch.float32)
    for h in range(n_kv):
        dims = torch.randperm(d, generator=gen, device=device)[:hot_dims]
        K[:, h, :, dims] *= hot_scale
    return K, V


def random_selection(cfg, layer, tensor, step, n, k):
    """Random selection (the pages' ablation): k of n unit ids, uniform without
    replacement, ascending, int32."""
    g = rng(cfg, layer, tensor, RANDOM_SEL, step)
    return np.sort(g.choice(n, size=k, replace=False)).astype(np.int32)


def random_token_selection(cfg, layer, step, batch, n_kv, T, k):
    """Random token selection per (batch, kv head): int32 [batch][n_kv][k], each row
    k of T tokens, uniform without replacement, ascending."""
    out = np.zeros((batch, n_kv, k), dtype=np.int32)
    for bi in range(batch):
        for h in range(n_kv):
            out[bi, h] = random_selection(cfg, layer, KV_CACHE, step * 1000003 + bi * 4096 + h, T, k)
    return out
