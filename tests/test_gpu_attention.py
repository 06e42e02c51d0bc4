"""GPU parity: refined GQA decode attention.  Token selection must be the oracle's
top-k (exactly, when the k-th and (k+1)-th oracle scores are separated by more than
1e-4 relative; otherwise a valid top-k within that margin), and the output must match
the oracle evaluated on the kernel's selection within 1e-3 rel / 1e-4 abs."""
import math

import numpy as np
import pytest
import torch

from bit_decode_selective_amd import binding, inputs
from oracle import attention as o_attn
from oracle import nested, selection

from gpu_util import assert_close, topk_is_valid

pytestmark = pytest.mark.gpu


def _case(cfg, batch, n_kv, G, T, b=2, r=2, q_scale=1.0):
    K, V = inputs.kv(cfg, 0, batch, n_kv, T, 128)
    q = (inputs.query(cfg, 0, 0, batch, n_kv * G, 128).astype(np.float32) * q_scale).astype(np.float16)
    kv = binding.QuantKV.from_host(K, V, b, r)
    qk = o_attn.quantize_kv(K, b, r)
    qv = o_attn.quantize_kv(V, b, r)
    return K, V, q, kv, qk, qv


def _check(q, kv, qk, qv, shape, k_sel, cache="resident", exact_required=False):
    batch, n_kv, T, d = shape
    scale = 1.0 / math.sqrt(d)
    if cache == "resident":
        cache = binding.RefineCache([kv.resident_pool_desc()])
    out, sel, hit = binding.refined_attention(q, kv, scale, k_sel, cache=cache)
    torch.cuda.synchronize()
    out, sel, hit = out.cpu().numpy(), sel.cpu().numpy(), hit.cpu().numpy()
    k_res = nested.dequant_resident(qk).reshape(batch, n_kv, T, d)
    G = q.shape[1] // n_kv
    n_exact = 0
    for bi in range(batch):
        for g in range(n_kv):
            sc = o_attn.token_scores(q[bi, g * G:(g + 1) * G], k_res[bi, g], scale)
            s = sel[bi, g].tolist()
            assert s == sorted(s)
            ok, separated = topk_is_valid(sc, s, k_sel)
            assert ok, (bi, g)
            if separated:
                assert s == selection.top_k(sc, k_sel), (bi, g)
                n_exact += 1
    if exact_required:
        assert n_exact == batch * n_kv
    hits = None
    if cache is None:
        hits = {}
    sel_map = {(bi, g): sel[bi, g].tolist() for bi in range(batch) for g in range(n_kv)}
    if cache is not None and cache != "resident":
        hits = {(bi, g): {t for t, h in zip(sel[bi, g], hit[bi, g]) if h >= 0}
                for bi in range(batch) for g in range(n_kv)}
    ref, _ = o_attn.refined_attention(q, qk, qv, shape, scale, k_sel, sel_in=sel_map, hits=hits)
    assert_close(out, ref, what=f"attention T={T} k={k_sel}")
    return out, sel, hit


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_small(G):
    batch, n_kv, T = 2, 2, 300
    K, V, q, kv, qk, qv = _case(20 + G, batch, n_kv, G, T)
    for k_sel in (0, 1, 7, T):
        _check(q, kv, qk, qv, (batch, n_kv, T, 128), k_sel)


@pytest.mark.parametrize("b,r", [(1, 1), (4, 4), (2, 1)])
def test_formats(b, r):
    K, V, q, kv, qk, qv = _case(30 + b, 1, 2, 4, 777, b, r)
    _check(q, kv, qk, qv, (1, 2, 777, 128), 16)


def test_single_token_and_tiny():
    for T in (1, 2, 65):
        K, V, q, kv, qk, qv = _case(40 + T, 1, 1, 4, T)
        _check(q, kv, qk, qv, (1, 1, T, 128), min(T, 3))


def test_uniform_query_selects_first_tokens():
    K, V, q, kv, qk, qv = _case(50, 1, 2, 4, 200)
    q = np.zeros_like(q)
    out, sel, _ = _check(q, kv, qk, qv, (1, 2, 200, 128), 5)
    assert sel[0, 0].tolist() == [0, 1, 2, 3, 4]


def test_misses_fall_back_to_resident():
    K, V, q, kv, qk, qv = _case(51, 1, 2, 4, 500)
    _, sel, hit = _check(q, kv, qk, qv, (1, 2, 500, 128), 10, cache=None)
    assert np.all(hit == -1)


def test_external_selection():
    batch, n_kv, G, T = 1, 2, 4, 400
    K, V, q, kv, qk, qv = _case(52, batch, n_kv, G, T)
    rng = np.random.default_rng(1)
    ext = np.stack([np.sort(rng.choice(T, 9, replace=False)) for _ in range(n_kv)])[None].astype(np.int32)
    cache = binding.RefineCache([kv.resident_pool_desc()])
    out, sel, hit = binding.refined_attention(q, kv, 1 / math.sqrt(128), 9, cache=cache, sel_in=ext)
    assert np.array_equal(sel.cpu().numpy(), ext)
    ref, _ = o_attn.refined_attention(q, qk, qv, (batch, n_kv, T, 128), 1 / math.sqrt(128), 9,
                                      sel_in={(0, g): ext[0, g].tolist() for g in range(n_kv)})
    assert_close(out.cpu().numpy(), ref)


def test_full_size_32k():
    """32 query heads, 8 KV heads, head dim 128, T = 32768, 2 + 2 bit KV, top 2% tokens."""
    batch, n_kv, G, T = 1, 8, 4, 32768
    K, V, q, kv, qk, qv = _case(3, batch, n_kv, G, T)
    _check(q, kv, qk, qv, (batch, n_kv, T, 128), selection.k_select(2, T))


def test_ragged_long_context():
    """T = 40000: ten selection chunks, the last one ragged."""
    batch, n_kv, G, T = 1, 1, 4, 40000
    K, V, q, kv, qk, qv = _case(53, batch, n_kv, G, T)
    _check(q, kv, qk, qv, (batch, n_kv, T, 128), selection.k_select(2, T))
