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
@pytest.mark.parametrize("given", [False, True])
def test_gemv_lru_over_steps(capacity, max_fill, given):
    """given: the selection comes in as sel_in (as a producer kernel hands it over),
    so each tile looks its hits up itself and the first tile logs the lookups."""
    k_in, n_out, ks = 512, 256, 16
    qw, q = _weight(60, n_out, k_in, 2, 2)
    store = qw.host_store()
    cache = binding.RefineCache([binding.host_pool_desc(store, capacity)], max_fill=max_fill, keep=[store])
    pool = o_cache.LRUPool(capacity)
    for t in range(8):
        x = _step_x(60 + t % 3, t, k_in)
        sel_in = np.array(selection.select_channels(x, ks), dtype=np.int32) if given else None
        (y,), sel, (hit,) = binding.refined_gemv([(qw, 0)], x, ks, cache=cache, sel_in=sel_in)
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


@pytest.mark.parametrize("mode", [binding.SF_CACHE_DETERMINISTIC, binding.SF_CACHE_ASYNC])
def test_ssd_tier_matches_host_store(tmp_path, mode):
    """The same weight pool served from a store file (read per unit, direct I/O where
    the file system allows) and from pinned host memory: identical hit sets, resident
    sets and outputs (bit for bit) every step; deterministic mode also against the
    oracle LRU; every installed unit read from the file once."""
    k_in, n_out, ks, capacity = 512, 256, 16, 24
    qw, q = _weight(64, n_out, k_in, 2, 2)
    store = qw.host_store()
    path = str(tmp_path / "units.bin")
    binding.write_store_file(path, store)
    c_ram = binding.RefineCache([binding.host_pool_desc(store, capacity)], mode=mode, keep=[store])
    c_ssd = binding.RefineCache([binding.file_pool_desc(path, qw.unit_bytes, k_in, capacity)], mode=mode)
    pool = o_cache.LRUPool(capacity)
    for t in range(8):
        x = _step_x(64 + t % 3, t, k_in)
        outs = []
        for c in (c_ram, c_ssd):
            (y,), sel, (hit,) = binding.refined_gemv([(qw, 0)], x, ks, cache=c)
            torch.cuda.synchronize()
            outs.append((y.cpu().numpy(), sel.cpu().numpy().tolist(), (hit.cpu().numpy() >= 0).tolist()))
        assert outs[0][1] == outs[1][1] and outs[0][2] == outs[1][2], t
        assert np.array_equal(outs[0][0], outs[1][0]), t
        sel, hits = outs[1][1], outs[1][2]
        if mode == binding.SF_CACHE_DETERMINISTIC:
            assert hits == pool.lookup(sel, t), t
        assert_close(outs[1][0], o_gemv.refined_gemv(q, x, [k for k, h in zip(sel, hits) if h]), what=f"step {t}")
        c_ram.fill()
        c_ssd.fill()
        if mode == binding.SF_CACHE_DETERMINISTIC:
            pool.fill(t)
            assert c_ssd.resident(0, capacity) == pool.resident(), t
    torch.cuda.synchronize()
    io = c_ssd.io_stats(0)
    st = c_ssd.stats(0)
    assert io["reads"] == st["installed"] > 0
    assert io["bytes"] == st["installed"] * qw.unit_bytes
    assert io["p99_us"] >= io["p50_us"] > 0
    assert c_ram.io_stats()["reads"] == 0


def test_ssd_tier_kv_pool(tmp_path):
    """KV refinement units (64 bytes each, far below a disk block) from a store file
    at an offset: hit sets against the oracle LRU and outputs against the oracle."""
    batch, n_kv, G, T, b, r, ks = 1, 2, 4, 600, 2, 2, 12
    K, V = inputs.kv(65, 0, batch, n_kv, T, 128)
    kv = binding.QuantKV.from_host(K, V, b, r)
    qk, qv = o_attn.quantize_kv(K, b, r), o_attn.quantize_kv(V, b, r)
    store = kv.host_store()
    path = str(tmp_path / "kv_units.bin")
    with open(path, "wb") as f:
        f.write(b"\x5a" * 1000)  # the units start at byte 1000
    with open(path, "ab") as f:
        f.write(store.numpy().tobytes())
    capacity = 20
    cache = binding.RefineCache([binding.file_pool_desc(path, kv.unit_bytes, kv.n_units, capacity, offset=1000)])
    pool = o_cache.LRUPool(capacity)
    scale = 1.0 / math.sqrt(128)
    for t in range(6):
        q = inputs.query(65, 0, t // 2, batch, n_kv * G, 128)
        out, sel, hit = binding.refined_attention(q, kv, scale, ks, cache=cache)
        torch.cuda.synchronize()
        out, sel, hit = out.cpu().numpy(), sel.cpu().numpy(), hit.cpu().numpy()
        units = [(bi * n_kv + g) * kv.t_cap + int(tok) for bi in range(batch) for g in range(n_kv) for tok in sel[bi, g]]
        assert (hit.reshape(-1) >= 0).tolist() == pool.lookup(units, t), t
        hits = {(bi, g): {int(tok) for tok, h in zip(sel[bi, g], hit[bi, g]) if h >= 0}
                for bi in range(batch) for g in range(n_kv)}
        sel_map = {(bi, g): sel[bi, g].tolist() for bi in range(batch) for g in range(n_kv)}
        ref, _ = o_attn.refined_attention(q, qk, qv, (batch, n_kv, T, 128), scale, ks, sel_in=sel_map, hits=hits)
        assert_close(out, ref, what=f"attention step {t}")
        cache.fill()
        pool.fill(t)
        assert cache.resident(0, capacity) == pool.resident(), t


@pytest.mark.parametrize("b,r,batch", [(2, 2, 1), (3, 1, 3), (1, 3, 2)])
def test_lag_delta_completes_missed_refinements(b, r, batch):
    """sf_refine_lag_delta after a GEMV whose pool holds 10 of the channels: the late
    contribution of the channels that missed equals the oracle's, and the GEMV's
    output plus it equals the oracle GEMV refined on the whole selection."""
    k_in, n_out, ks, capacity = 640, 224, 40, 10
    qw, q = _weight(66, n_out, k_in, b, r)
    store = qw.host_store()
    cache = binding.RefineCache([binding.host_pool_desc(store, capacity)], keep=[store])
    x0 = inputs.activation(66, 0, 0, 0, batch, k_in)
    binding.refined_gemv([(qw, 0)], x0, ks, cache=cache)
    cache.fill()  # the first selection's top channels are now resident
    x = inputs.activation(66, 0, 0, 1, batch, k_in)
    (y,), sel, (hit,) = binding.refined_gemv([(qw, 0)], x, ks, cache=cache)
    delta = binding.refine_lag_delta(cache, 0, qw, x, sel, hit)
    torch.cuda.synchronize()
    sel_l, hit_l = sel.cpu().numpy().tolist(), hit.cpu().numpy().tolist()
    late = [k for k, h in zip(sel_l, hit_l) if h < 0]
    assert 0 < len(late) < ks
    assert_close(delta.cpu().numpy(), o_gemv.lag_delta(q, x, late), what="late contribution")
    assert_close(y.cpu().numpy() + delta.cpu().numpy(), o_gemv.refined_gemv(q, x, sel_l), what="y + late")


def test_lag_delta_edges():
    """Nothing missed (a resident pool) gives 0; k_sel = 0 gives 0; a store file is
    not supported; residual_add adds in place."""
    qw, q = _weight(67, 256, 512, 2, 2)
    cache = binding.RefineCache([qw.resident_pool_desc()])
    x = inputs.activation(67, 0, 0, 0, 1, 512)
    (y,), sel, (hit,) = binding.refined_gemv([(qw, 0)], x, 16, cache=cache)
    d = binding.refine_lag_delta(cache, 0, qw, x, sel, hit)
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    d0 = binding.refine_lag_delta(cache, 0, qw, x, empty, empty)
    torch.cuda.synchronize()
    assert not d.abs().max().item() and not d0.abs().max().item()
    h = torch.arange(256, dtype=torch.float32, device="cuda")
    binding.residual_add(h, torch.full_like(h, 0.5))
    assert torch.equal(h.cpu(), torch.arange(256, dtype=torch.float32) + 0.5)


@pytest.mark.parametrize("lead,capacity", [(16, 12), (10, 0), (40, 30)])
def test_lead_prefetch_over_steps(lead, capacity):
    """Fetch lead on one weight pool over 10 steps: a prefetch of a predicted
    selection (every other step the GEMV's own, otherwise another step's) on a side
    stream, then the GEMV: hit sets, outputs and LRU resident sets against the
    oracle policy (LRU slots plus lead slots)."""
    k_in, n_out, ks = 512, 256, 16
    qw, q = _weight(68, n_out, k_in, 2, 2)
    store = qw.host_store()
    cache = binding.RefineCache([binding.host_pool_desc(store, capacity, lead_slots=lead)], keep=[store])
    pool = o_cache.LeadPool(capacity, lead)
    side = torch.cuda.Stream()
    for t in range(10):
        x = _step_x(68, t, k_in)
        pred = selection.select_channels(_step_x(68, t + 1, k_in), ks)
        ev = torch.cuda.Event()
        with torch.cuda.stream(side):
            cache.prefetch(0, torch.as_tensor(pred, dtype=torch.int32, device="cuda"), stream=side)
            ev.record(side)
        torch.cuda.current_stream().wait_event(ev)
        pool.prefetch(pred)
        (y,), sel, (hit,) = binding.refined_gemv([(qw, 0)], x, ks, cache=cache)
        torch.cuda.synchronize()
        sel = sel.cpu().numpy().tolist()
        hits = (hit.cpu().numpy() >= 0).tolist()
        assert hits == pool.lookup(sel, t), t
        assert_close(y.cpu().numpy(), o_gemv.refined_gemv(q, x, [k for k, h in zip(sel, hits) if h]),
                     what=f"step {t}")
        cache.fill()
        pool.fill(t)
        assert cache.resident(0, max(1, capacity)) == pool.resident(), t
    st = cache.stats(0)
    assert st["lookups"] == 10 * ks and st["hits"] > 0


def test_lead_prefetch_edges():
    """A pool without lead slots refuses prefetches; an empty prefetch empties the
    ring; prefetched units that the LRU already holds are not fetched again."""
    qw, q = _weight(69, 256, 512, 2, 2)
    store = qw.host_store()
    with pytest.raises(binding.SFError):
        c0 = binding.RefineCache([binding.host_pool_desc(store, 8)], keep=[store])
        c0.prefetch(0, torch.arange(4, dtype=torch.int32, device="cuda"))
    cache = binding.RefineCache([binding.host_pool_desc(store, 8, lead_slots=8)], keep=[store])
    pool = o_cache.LeadPool(8, 8)
    ids = torch.arange(8, dtype=torch.int32, device="cuda")
    slots = cache.lookup(0, ids)
    pool.lookup(list(range(8)), 0)
    cache.fill()
    pool.fill(0)  # units 0..7 in LRU slots
    cache.prefetch(0, torch.arange(4, 12, dtype=torch.int32, device="cuda"))
    assert pool.prefetch(list(range(4, 12))) == [8, 9, 10, 11]
    slots = cache.lookup(0, torch.arange(16, dtype=torch.int32, device="cuda")).cpu().numpy()
    assert (slots >= 0).tolist() == pool.lookup(list(range(16)), 1)
    assert set(slots[8:12].tolist()) <= set(range(8, 16)) and slots[:8].max() < 8  # ring slots follow the LRU's
    cache.prefetch(0, torch.empty(0, dtype=torch.int32, device="cuda"))
    pool.prefetch([])
    slots = cache.lookup(0, torch.arange(16, dtype=torch.int32, device="cuda")).cpu().numpy()
    assert (slots >= 0).tolist() == pool.lookup(list(range(16)), 2)
    torch.cuda.synchronize()


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


def test_lookup_call_matches_oracle_lru():
    """sf_refine_cache_lookup on its own: the slot of every resident unit and -1 for
    the rest, in the order asked; its lookups are logged like the kernels' own, so
    the fills that follow install the same units as the oracle LRU (two lookup calls
    per step, repeated and duplicate ids, a pool smaller than one step's lookups)."""
    qw, _ = _weight(64, 256, 512, 2, 2)
    store = qw.host_store()
    cap = 24
    cache = binding.RefineCache([binding.host_pool_desc(store, cap, max_lookup=64)], keep=[store])
    pool = o_cache.LRUPool(cap)
    rng = np.random.default_rng(5)
    for t in range(10):
        for call in range(2):
            ids = rng.choice(48, 20, replace=False).astype(np.int32)
            if call == 1:
                ids[:3] = ids[3]  # the same unit three times in one call
            slots = cache.lookup(0, torch.as_tensor(ids, device="cuda")).cpu().numpy()
            want = pool.lookup(ids.tolist(), t)
            assert (slots >= 0).tolist() == want, (t, call)
            hit_slots = slots[slots >= 0]
            assert np.all(hit_slots < cap)
            # a unit has one slot, and different units have different slots
            by_unit = {}
            for u, s in zip(ids.tolist(), slots.tolist()):
                if s >= 0:
                    assert by_unit.setdefault(u, s) == s
            assert len(set(by_unit.values())) == len(by_unit)
        cache.fill()
        pool.fill(t)
        assert cache.resident(0, cap) == pool.resident(), t
    assert cache.stats(0)["lookups"] == 10 * 2 * 20
