"""GPU parity of the pages' comparison variants, through the C ABI, against
``oracle.variants`` (and the refined-path oracle for random selection): random
selection, FP16 fetch of weight columns, SpeCache-style FP16 token replacement and
sparse attention over the selected tokens.  Selections bit-exact, outputs within
1e-3 rel / 1e-4 abs."""
import math

import numpy as np
import pytest
import torch

from bit_decode_selective_amd import binding, inputs
from oracle import attention as o_attn
from oracle import cache as o_cache
from oracle import gemv as o_gemv
from oracle import nested, selection, variants

from gpu_util import assert_close, separated_query

pytestmark = pytest.mark.gpu

D = 128
SCALE = 1.0 / math.sqrt(D)


# ---- random selection ---------------------------------------------------------
def test_random_selection_gemv_4096():
    """A 4096 x 4096 2+2-bit GEMV refined on 205 random channels (every unit resident)."""
    W = inputs.weight(21, 0, 0, 4096, 4096)
    qw = binding.QuantWeight.from_host(W, 2, 2)
    q = nested.quantize(W, 2, 2, 128)
    x = inputs.activation(21, 0, 0, 0, 1, 4096)
    sel = inputs.random_selection(21, 0, 0, 0, 4096, 205)
    cache = binding.RefineCache([qw.resident_pool_desc()])
    (y,), got, _ = binding.refined_gemv([(qw, 0)], x, 205, cache=cache, sel_in=sel)
    torch.cuda.synchronize()
    assert got.cpu().numpy().tolist() == sel.tolist()
    assert_close(y.cpu().numpy(), o_gemv.refined_gemv(q, x, sel.tolist()), what="random selection GEMV")


def test_random_selection_attention_32k():
    """Attention at T = 32768, 8 KV heads, 656 random tokens per KV head."""
    T, n_kv = 32768, 8
    K, V = inputs.kv(22, 0, 1, n_kv, T, D)
    kv = binding.QuantKV.from_host(K, V, 2, 2)
    qk, qv = o_attn.quantize_kv(K, 2, 2), o_attn.quantize_kv(V, 2, 2)
    q = inputs.query(22, 0, 0, 1, 32, D)
    ks = selection.k_select(2, T)
    sel = inputs.random_token_selection(22, 0, 0, 1, n_kv, T, ks)
    cache = binding.RefineCache([kv.resident_pool_desc()])
    out, got, _ = binding.refined_attention(q, kv, SCALE, ks, cache=cache, sel_in=sel)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), sel)
    ref, _ = o_attn.refined_attention(q, qk, qv, (1, n_kv, T, D), SCALE, ks,
                                      sel_in={(0, g): sel[0, g].tolist() for g in range(n_kv)})
    assert_close(out.cpu().numpy(), ref, what="random token selection")


# ---- FP16 fetch ---------------------------------------------------------------
@pytest.mark.parametrize("b,r,batch", [(2, 2, 1), (3, 1, 2), (4, 4, 3), (1, 3, 1)])
def test_fp16_fetch_resident(b, r, batch):
    """Every selected column present as fp16: the selected columns take fp16(W)."""
    n_out, k_in, ks = 224, 640, 37
    W = inputs.weight(23, 0, 0, n_out, k_in)
    qw = binding.QuantWeight.from_host(W, b, r)
    q = nested.quantize(W, b, r, 128)
    units = binding.fp16_weight_units(W)
    cache = binding.RefineCache([binding.device_pool_desc(units)])
    x = inputs.activation(23, 0, 0, 0, batch, k_in)
    y, sel, slots = binding.fp16_fetch_gemv(qw, x, ks, cache, 0)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy().tolist()
    assert sel == selection.select_channels(x, ks)
    assert (slots.cpu().numpy() >= 0).all()
    assert_close(y.cpu().numpy(), variants.fp16_fetch_gemv(W, q, x, sel), what=f"fp16 fetch b{b} r{r}")


def test_fp16_fetch_lru_over_steps():
    """FP16 columns from a pinned host store through LRU slots (capacity 24): hit
    sets against the oracle LRU, outputs against the oracle on those hits."""
    n_out, k_in, ks, cap = 256, 512, 16, 24
    W = inputs.weight(24, 0, 0, n_out, k_in)
    qw = binding.QuantWeight.from_host(W, 2, 2)
    q = nested.quantize(W, 2, 2, 128)
    store = binding.fp16_weight_units(W, device="cpu").pin_memory()
    cache = binding.RefineCache([binding.host_pool_desc(store, cap)], keep=[store])
    pool = o_cache.LRUPool(cap)
    for t in range(8):
        x = inputs.activation(24 + t % 3, 0, 0, t // 2, 1, k_in)
        y, sel, slots = binding.fp16_fetch_gemv(qw, x, ks, cache, 0)
        torch.cuda.synchronize()
        sel = sel.cpu().numpy().tolist()
        hits = (slots.cpu().numpy() >= 0).tolist()
        assert hits == pool.lookup(sel, t), t
        assert_close(y.cpu().numpy(), variants.fp16_fetch_gemv(W, q, x, [k for k, h in zip(sel, hits) if h]),
                     what=f"fp16 fetch step {t}")
        cache.fill()
        pool.fill(t)


def test_fp16_fetch_full_size():
    """4096 -> 14336 (gate width), 123 channels (3%), every column present."""
    W = inputs.weight(25, 0, 0, 14336, 4096)
    qw = binding.QuantWeight.from_host(W, 2, 2)
    q = nested.quantize(W, 2, 2, 128)
    units = binding.fp16_weight_units(W)
    cache = binding.RefineCache([binding.device_pool_desc(units)])
    x = inputs.activation(25, 0, 0, 0, 1, 4096)
    ks = selection.k_select(3, 4096)
    y, sel, _ = binding.fp16_fetch_gemv(qw, x, ks, cache, 0)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy().tolist()
    assert sel == selection.select_channels(x, ks)
    assert_close(y.cpu().numpy(), variants.fp16_fetch_gemv(W, q, x, sel), what="fp16 fetch 14336x4096")


# ---- attention variants ----------------------------------------------------------
class KVCase:
    def __init__(self, cfg, batch, n_kv, G, T, b=2, r=2):
        self.batch, self.n_kv, self.G, self.T, self.cfg = batch, n_kv, G, T, cfg
        self.K, self.V = inputs.kv(cfg, 0, batch, n_kv, T, D)
        self.kv = binding.QuantKV.from_host(self.K, self.V, b, r)
        self.qk, self.qv = o_attn.quantize_kv(self.K, b, r), o_attn.quantize_kv(self.V, b, r)
        self.k_res = nested.dequant_resident(self.qk).reshape(batch, n_kv, T, D)
        self.shape = (batch, n_kv, T, D)

    def query(self, k_sel):
        q, _ = separated_query(self.cfg, 0, self.batch, self.n_kv, self.G, D, lambda bi, g: self.k_res[bi, g],
                               SCALE, k_sel)
        return q

    def check_selection(self, q, sel, k_sel):
        for bi in range(self.batch):
            for g in range(self.n_kv):
                sc = o_attn.token_scores(q[bi, g * self.G:(g + 1) * self.G], self.k_res[bi, g], SCALE)
                assert sel[bi, g].tolist() == selection.top_k(sc, k_sel), (bi, g)


@pytest.mark.parametrize("T,G,k_sel", [(300, 4, 7), (777, 2, 40), (1, 4, 1), (65, 8, 65)])
def test_fp16_tokens_resident(T, G, k_sel):
    case = KVCase(31, 2, 2, G, T)
    units = binding.fp16_kv_units(case.K, case.V)
    cache = binding.RefineCache([binding.device_pool_desc(units)])
    q = case.query(k_sel)
    out, sel, hit = binding.refined_attention(q, case.kv, SCALE, k_sel, cache=cache,
                                              variant=binding.SF_ATTN_FP16_TOKENS)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    case.check_selection(q, sel, k_sel)
    ref, _ = variants.fp16_token_attention(q, case.qk, case.qv, case.K, case.V, case.shape, SCALE, k_sel)
    assert_close(out.cpu().numpy(), ref, what=f"fp16 tokens T={T}")


def test_fp16_tokens_with_misses():
    """A pool holding 20 fp16 token units (LRU): misses stay resident."""
    case = KVCase(32, 1, 2, 4, 600)
    store = binding.fp16_kv_units(case.K, case.V, device="cpu").pin_memory()
    cache = binding.RefineCache([binding.host_pool_desc(store, 20)], keep=[store])
    pool = o_cache.LRUPool(20)
    for t in range(4):
        q = inputs.query(32, 0, t // 2, 1, 8, D)
        out, sel, hit = binding.refined_attention(q, case.kv, SCALE, 12, cache=cache,
                                                  variant=binding.SF_ATTN_FP16_TOKENS)
        torch.cuda.synchronize()
        out, sel, hit = out.cpu().numpy(), sel.cpu().numpy(), hit.cpu().numpy()
        units = [g * case.T + int(tok) for g in range(2) for tok in sel[0, g]]
        assert (hit.reshape(-1) >= 0).tolist() == pool.lookup(units, t), t
        hits = {(0, g): {int(tok) for tok, h in zip(sel[0, g], hit[0, g]) if h >= 0} for g in range(2)}
        ref, _ = variants.fp16_token_attention(q, case.qk, case.qv, case.K, case.V, case.shape, SCALE, 12,
                                               sel_in={(0, g): sel[0, g].tolist() for g in range(2)}, hits=hits)
        assert_close(out, ref, what=f"fp16 tokens step {t}")
        cache.fill()
        pool.fill(t)


@pytest.mark.parametrize("T,G,k_sel", [(300, 4, 7), (777, 2, 40), (1, 4, 1), (65, 8, 65), (2000, 1, 1)])
def test_sparse_attention(T, G, k_sel):
    case = KVCase(33, 2, 2, G, T)
    cache = binding.RefineCache([case.kv.resident_pool_desc()])
    q = case.query(k_sel)
    out, sel, hit = binding.refined_attention(q, case.kv, SCALE, k_sel, cache=cache,
                                              variant=binding.SF_ATTN_DROP_UNSELECTED)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    case.check_selection(q, sel, k_sel)
    ref, _ = variants.sparse_attention(q, case.qk, case.qv, case.shape, SCALE, k_sel)
    assert_close(out.cpu().numpy(), ref, what=f"sparse attention T={T} k={k_sel}")


def test_sparse_attention_with_misses_and_edges():
    """No pool: every selected token at resident precision; k_sel = 0 is refused."""
    case = KVCase(34, 1, 2, 4, 500)
    q = case.query(9)
    out, sel, _ = binding.refined_attention(q, case.kv, SCALE, 9, cache=None, variant=binding.SF_ATTN_DROP_UNSELECTED)
    torch.cuda.synchronize()
    ref, _ = variants.sparse_attention(q, case.qk, case.qv, case.shape, SCALE, 9, hits={})
    assert_close(out.cpu().numpy(), ref, what="sparse attention, all misses")
    with pytest.raises(binding.SFError):
        binding.refined_attention(q, case.kv, SCALE, 0, variant=binding.SF_ATTN_DROP_UNSELECTED)


@pytest.mark.parametrize("variant", [binding.SF_ATTN_FP16_TOKENS, binding.SF_ATTN_DROP_UNSELECTED])
def test_attention_variants_32k(variant):
    """T = 32768, 8 KV heads, top 656 tokens per KV head, every unit resident."""
    case = KVCase(35, 1, 8, 4, 32768)
    ks = selection.k_select(2, 32768)
    if variant == binding.SF_ATTN_FP16_TOKENS:
        units = binding.fp16_kv_units(case.K, case.V)
        cache = binding.RefineCache([binding.device_pool_desc(units)])
    else:
        cache = binding.RefineCache([case.kv.resident_pool_desc()])
    q = case.query(ks)
    out, sel, _ = binding.refined_attention(q, case.kv, SCALE, ks, cache=cache, variant=variant)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    case.check_selection(q, sel, ks)
    if variant == binding.SF_ATTN_FP16_TOKENS:
        ref, _ = variants.fp16_token_attention(q, case.qk, case.qv, case.K, case.V, case.shape, SCALE, ks)
    else:
        ref, _ = variants.sparse_attention(q, case.qk, case.qv, case.shape, SCALE, ks)
    assert_close(out.cpu().numpy(), ref, what=f"variant {variant} at 32K")
