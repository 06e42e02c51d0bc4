"""GPU parity of the refinement slot cache over several decode steps, through the C
ABI: host-pinned refinement stores, pools smaller than the units they serve, fills
by the side-stream copy.  Each step's hit set must equal the oracle LRU's (oracle
``cache.LRUPool``, deterministic mode), the outputs must match the oracle evaluated
with exactly those hits, and the resident sets must agree after every fill.  Async
mode is checked for consistency given the kernel-reported hits and for eventually
serving a repeated selection."""
import math

import numpy as np
import pytest
import torch

from bit_decode_selective_amd import binding, inputs
from oracle import attention as o_attn
from oracle import cache as o_cache
from oracle import gemv as o_gemv
from oracle import nested, selection

from gpu_util import assert_close

pytestmark = pytest.mark.gpu


def _weight(cfg, n_out, k_in, b, r, tensor=0):
    W = inputs.weight(cfg, 0, tensor, n_out, k_in)
    return binding.QuantWeight.from_host(W, b, r), nested.quantize(W, b, r, 128)


def _step_x(cfg, step, k_in, batch=1):
    # half of the steps repeat an earlier activation so that the pool sees reuse
    return inputs.activation(cfg, 0, 0, step // 2, batch, k_in)


@pytest.mark.parametrize("capacity,max_fill", [(24, 0), (24, 5), (0, 0), (512, 0)])
def test_gemv_lru_over_steps(capacity, max_fill):
    k_in, n_out, ks = 512, 256, 16
    qw, q = _weight(60, n_out, k_in, 2, 2)
    store = qw.host_store()
    cache = binding.RefineCache([binding.host_pool_desc(store, capacity)], max_fill=max_fill, keep=[store])
    pool = o_cache.LRUPool(capacity)
    for t in range(8):
        x = _step_x(60 + t % 3, t, k_in)
        (y,), sel, (hit,) = binding.refined_gemv([(qw, 0)], x, ks, cache=cache)
        torch.cuda.synchronize()
        sel = sel.cpu().numpy().tolist()
        hit = hit.cpu().numpy()
        assert sel == selection.select_channels(x, ks), t
        want_hits = pool.lookup(sel, t)
        assert (hit >= 0).tolist() == want_hits, t
        hit_channels = [k for k, h in zip(sel, want_hits) if h]
        assert_close(y.cpu().numpy(), o_gemv.refined_gemv(q, x, hit_channels), what=f"step {t}")
        cache.fill()
        pool.fill(t, max_fill or None)
        assert cache.resident(0, max(1, capacity)) == pool.resident(), t
    st = cache.stats(0)
    assert st["lookups"] == 8 * ks
    assert st["h2d_bytes"] == st["installed"] * qw.unit_bytes


def test_gemv_fused_ops_have_their_own_pools():
    k_in, ks = 512, 20
    (qa, qa_o), (qb, qb_o) = _weight(61, 256, k_in, 2, 2, 0), _weight(61, 96, k_in, 2, 2, 1)
    sa, sb = qa.host_store(), qb.host_store()
    caps = (30, 8)
    cache = binding.RefineCache([binding.host_pool_desc(sa, caps[0]), binding.host_pool_desc(sb, caps[1])],
                                keep=[sa, sb])
    pools = [o_cache.LRUPool(c) for c in caps]
    for t in range(6):
        x = _step_x(61, t, k_in)
        ys, sel, hits = binding.refined_gemv([(qa, 0), (qb, 1)], x, ks, cache=cache)
        torch.cuda.synchronize()
        sel = sel.cpu().numpy().tolist()
        for i, (qo, y, h) in enumerate(zip((qa_o, qb_o), ys, hits)):
            want = pools[i].lookup(sel, t)
            assert (h.cpu().numpy() >= 0).tolist() == want, (t, i)
            assert_close(y.cpu().numpy(), o_gemv.refined_gemv(qo, x, [k for k, w in zip(sel, want) if w]))
        cache.fill()
        for p in pools:
            p.fill(t)
        for i, p in enumerate(pools):
            assert cache.resident(i, caps[i]) == p.resident()


def test_attention_lru_over_steps():
    batch, n_kv, G, T, b, r, ks = 1, 2, 4, 600, 2, 2, 12
    K, V = inputs.kv(62, 0, batch, n_kv, T, 128)
    kv = binding.QuantKV.from_host(K, V, b, r)
    qk, qv = o_attn.quantize_kv(K, b, r), o_attn.quantize_kv(V, b, r)
    store = kv.host_store()
    capacity = 20
    cache = binding.RefineCache([binding.host_pool_desc(store, capacity)], keep=[store])
    pool = o_cache.LRUPool(capacity)
    scale = 1.0 / math.sqrt(128)
    for t in range(6):
        q = inputs.query(62, 0, t // 2, batch, n_kv * G, 128)
        out, sel, hit = binding.refined_attention(q, kv, scale, ks, cache=cache)
        torch.cuda.synchronize()
        out, sel, hit = out.cpu().numpy(), sel.cpu().numpy(), hit.cpu().numpy()
        units = [(bi * n_kv + g) * kv.t_cap + int(tok) for bi in range(batch) for g in range(n_kv) for tok in sel[bi, g]]
        want = pool.lookup(units, t)
        assert (hit.reshape(-1) >= 0).tolist() == want, t
        hits = {(bi, g): {int(tok) for tok, h in zip(sel[bi, g], hit[bi, g]) if h >= 0}
                for bi in range(batch) for g in range(n_kv)}
        sel_map = {(bi, g): sel[bi, g].tolist() for bi in range(batch) for g in range(n_kv)}
        ref, _ = o_attn.refined_attention(q, qk, qv, (batch, n_kv, T, 128), scale, ks, sel_in=sel_map, hits=hits)
        assert_close(out, ref, what=f"attention step {t}")
        cache.fill()
        pool.fill(t)
        assert cache.resident(0, capacity) == pool.resident(), t


def test_async_fills_are_consistent_and_land():
    k_in, n_out, ks = 512, 256, 16
    qw, q = _weight(63, n_out, k_in, 2, 2)
    store = qw.host_store()
    cache = binding.RefineCache([binding.host_pool_desc(store, 64)], mode=binding.SF_CACHE_ASYNC, keep=[store])
    x = _step_x(63, 0, k_in)
    seen_all = False
    for t in range(6):
        (y,), sel, (hit,) = binding.refined_gemv([(qw, 0)], x, ks, cache=cache)
        torch.cuda.synchronize()
        sel, hit = sel.cpu().numpy().tolist(), hit.cpu().numpy()
        # whatever the kernel saw, the output is the oracle's for exactly those hits
        assert_close(y.cpu().numpy(), o_gemv.refined_gemv(q, x, [k for k, h in zip(sel, hit) if h >= 0]))
        seen_all = seen_all or bool(np.all(hit >= 0))
        cache.fill()
    torch.cuda.synchronize()
    assert seen_all, "a repeated selection is served once its fill has landed"


def test_pageable_store_is_refused():
    """Fills read the store from the device: a pool over pageable memory is an error
    at create time (SF_EINVAL), before any kernel could touch it."""
    qw, _ = _weight(61, 256, 512, 2, 2)
    pinned = qw.host_store()
    pageable = torch.empty_like(pinned, device="cpu", pin_memory=False)
    pageable.copy_(pinned)
    with pytest.raises(binding.SFError):
        binding.RefineCache([binding.host_pool_desc(pageable, 8)], keep=[pageable])
    # a pool without slots never reads its store
    binding.RefineCache([binding.host_pool_desc(pageable, 0)], keep=[pageable])
