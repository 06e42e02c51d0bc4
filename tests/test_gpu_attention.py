"""GPU parity: refined GQA decode attention, through the C ABI.

Queries are drawn without near-ties: for every (batch, kv head) the k-th and
(k+1)-th oracle token scores differ by at least 1e-4 relative (the group's heads
are redrawn from the next step's query until they do), so the selected index set
is unique and must equal the oracle's exactly.  Outputs must match the oracle
within 1e-3 rel / 1e-4 abs; with every selected unit resident in the cache the
oracle runs on its own selection, so a wrong choice shows in the output too."""
import math

import numpy as np
import pytest
import torch

from bit_decode_selective_amd import binding, inputs
from oracle import attention as o_attn
from oracle import nested, selection

from gpu_util import assert_close, separated_query

pytestmark = pytest.mark.gpu

D = 128
SCALE = 1.0 / math.sqrt(D)


class Case:
    """Seeded K/V of one layer, quantised on the GPU and in the oracle."""

    def __init__(self, cfg, batch, n_kv, G, T, b=2, r=2, t_cap=None):
        self.cfg, self.batch, self.n_kv, self.G, self.T, self.b, self.r = cfg, batch, n_kv, G, T, b, r
        K, V = inputs.kv(cfg, 0, batch, n_kv, T, D)
        self.kv = binding.QuantKV.from_host(K, V, b, r, t_cap=t_cap)
        self.qk = o_attn.quantize_kv(K, b, r)
        self.qv = o_attn.quantize_kv(V, b, r)
        self.k_res = nested.dequant_resident(self.qk).reshape(batch, n_kv, T, D)

    @property
    def shape(self):
        return (self.batch, self.n_kv, self.T, D)

    def query(self, k_sel):
        q, _ = separated_query(self.cfg, 0, self.batch, self.n_kv, self.G, D, lambda bi, g: self.k_res[bi, g],
                               SCALE, k_sel)
        return q


def _run(case, q, k_sel, cache="resident", sel_in=None):
    if cache == "resident":
        cache = binding.RefineCache([case.kv.resident_pool_desc()])
    out, sel, hit = binding.refined_attention(q, case.kv, SCALE, k_sel, cache=cache, sel_in=sel_in)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sel.cpu().numpy(), hit.cpu().numpy()


def _check(case, q, k_sel, cache="resident"):
    """Exact selection per (batch, kv head) and the output against the oracle's own
    refined attention (every hit when the pool is resident, else the reported hits)."""
    out, sel, hit = _run(case, q, k_sel, cache)
    G = case.G
    for bi in range(case.batch):
        for g in range(case.n_kv):
            sc = o_attn.token_scores(q[bi, g * G:(g + 1) * G], case.k_res[bi, g], SCALE)
            assert sel[bi, g].tolist() == selection.top_k(sc, k_sel), (bi, g)
    if cache == "resident":
        ref, chosen = o_attn.refined_attention(q, case.qk, case.qv, case.shape, SCALE, k_sel)
        assert all(chosen[(bi, g)] == sel[bi, g].tolist() for bi in range(case.batch) for g in range(case.n_kv))
    else:
        hits = {(bi, g): {int(t) for t, h in zip(sel[bi, g], hit[bi, g]) if h >= 0}
                for bi in range(case.batch) for g in range(case.n_kv)}
        sel_map = {(bi, g): sel[bi, g].tolist() for bi in range(case.batch) for g in range(case.n_kv)}
        ref, _ = o_attn.refined_attention(q, case.qk, case.qv, case.shape, SCALE, k_sel, sel_in=sel_map, hits=hits)
    assert_close(out, ref, what=f"attention T={case.T} k={k_sel}")
    return out, sel, hit


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_small(G):
    case = Case(20 + G, 2, 2, G, 300)
    for k_sel in (0, 1, 7, 300):
        _check(case, case.query(k_sel), k_sel)


@pytest.mark.parametrize("b,r", [(1, 1), (4, 4), (2, 1)])
def test_formats(b, r):
    case = Case(30 + b, 1, 2, 4, 777, b, r)
    _check(case, case.query(16), 16)


def test_single_token_and_tiny():
    for T in (1, 2, 65):
        case = Case(40 + T, 1, 1, 4, T)
        k = min(T, 3)
        _check(case, case.query(k), k)


def test_uniform_query_selects_first_tokens():
    """q = 0: every logit is 0 and every score equal, so the lowest tokens win."""
    case = Case(50, 1, 2, 4, 200)
    q = np.zeros((1, 8, D), dtype=np.float16)
    out, sel, _ = _check(case, q, 5)
    assert sel[0, 0].tolist() == sel[0, 1].tolist() == [0, 1, 2, 3, 4]


@pytest.mark.parametrize("T,k", [(12000, 700), (9000, 4100), (4097, 2)])
def test_uniform_query_ties_across_chunks(T, k):
    """q = 0 over several 4096-token chunks: every score is equal, so the first k
    tokens win, taken across chunk boundaries in token order."""
    case = Case(53, 1, 2, 4, T)
    q = np.zeros((1, 8, D), dtype=np.float16)
    out, sel, _ = _check(case, q, k)
    assert sel[0, 0].tolist() == sel[0, 1].tolist() == list(range(k))


def test_misses_fall_back_to_resident():
    case = Case(51, 1, 2, 4, 500)
    _, sel, hit = _check(case, case.query(10), 10, cache=None)
    assert np.all(hit == -1)


def test_external_selection():
    case = Case(52, 1, 2, 4, 400)
    rng = np.random.default_rng(1)
    ext = np.stack([np.sort(rng.choice(400, 9, replace=False)) for _ in range(2)])[None].astype(np.int32)
    q = inputs.query(52, 0, 0, 1, 8, D)
    out, sel, _ = _run(case, q, 9, sel_in=ext)
    assert np.array_equal(sel, ext)
    ref, _ = o_attn.refined_attention(q, case.qk, case.qv, case.shape, SCALE, 9,
                                      sel_in={(0, g): ext[0, g].tolist() for g in range(2)})
    assert_close(out, ref)


def test_full_size_32k():
    """32 query heads, 8 KV heads, head dim 128, T = 32768, 2 + 2 bit KV, top 2% tokens."""
    case = Case(3, 1, 8, 4, 32768)
    ks = selection.k_select(2, 32768)
    _check(case, case.query(ks), ks)


def test_ragged_long_context():
    """T = 40000: ten selection chunks, the last one ragged."""
    case = Case(53, 1, 1, 4, 40000)
    ks = selection.k_select(2, 40000)
    _check(case, case.query(ks), ks)


def test_batch8_context_8k():
    """Batch 8 at context 8192 (the batch-8 full-step shape): 64 (batch, kv head)
    selections of 164 tokens each."""
    case = Case(4, 8, 8, 4, 8192)
    ks = selection.k_select(2, 8192)
    _check(case, case.query(ks), ks)


def test_full_size_128k():
    """T = 131072, 8 KV heads, 2 + 2 bit KV, top 2% (2622 tokens per KV head): every
    selection exact; the output of every KV head against the oracle, one KV head at a
    time (the oracle's dequantised cache of all heads would not fit a test's memory)."""
    T, n_kv, G = 131072, 8, 4
    K, V = inputs.kv(5, 0, 1, n_kv, T, D)
    kv = binding.QuantKV.from_host(K, V, 2, 2)
    ks = selection.k_select(2, T)
    per_head = []
    for g in range(n_kv):
        qk = o_attn.quantize_kv(K[:, g:g + 1], 2, 2)
        qv = o_attn.quantize_kv(V[:, g:g + 1], 2, 2)
        per_head.append((qk, qv, nested.dequant_resident(qk)))
    del K, V
    q, _ = separated_query(5, 0, 1, n_kv, G, D, lambda bi, g: per_head[g][2], SCALE, ks)
    cache = binding.RefineCache([kv.resident_pool_desc()])
    out, sel, hit = binding.refined_attention(q, kv, SCALE, ks, cache=cache)
    torch.cuda.synchronize()
    out, sel = out.cpu().numpy(), sel.cpu().numpy()
    for g in range(n_kv):
        qk, qv, k_res = per_head[g]
        qg = q[:, g * G:(g + 1) * G]
        assert sel[0, g].tolist() == selection.top_k(o_attn.token_scores(qg[0], k_res, SCALE), ks), g
        ref, _ = o_attn.refined_attention(qg, qk, qv, (1, 1, T, D), SCALE, ks)
        assert_close(out[:, g * G:(g + 1) * G], ref, what=f"128K kv head {g}")


def test_max_context_1m():
    """The largest context the call accepts, T = 1,048,576 (256 selection chunks, one
    per CU, all resident together): one KV head, top 2% (20,972 tokens), exact
    selection and the output against the oracle."""
    T, n_kv, G = 1 << 20, 1, 4
    K, V = inputs.kv(6, 0, 1, n_kv, T, D)
    kv = binding.QuantKV.from_host(K, V, 2, 2)
    ks = selection.k_select(2, T)
    qk = o_attn.quantize_kv(K, 2, 2)
    qv = o_attn.quantize_kv(V, 2, 2)
    del K, V
    k_res = nested.dequant_resident(qk).reshape(1, n_kv, T, D)
    q, _ = separated_query(6, 0, 1, n_kv, G, D, lambda bi, g: k_res[bi, g], SCALE, ks)
    cache = binding.RefineCache([kv.resident_pool_desc()])
    out, sel, hit = binding.refined_attention(q, kv, SCALE, ks, cache=cache)
    torch.cuda.synchronize()
    out, sel = out.cpu().numpy(), sel.cpu().numpy()
    assert sel[0, 0].tolist() == selection.top_k(o_attn.token_scores(q[0], k_res[0, 0], SCALE), ks)
    ref, _ = o_attn.refined_attention(q, qk, qv, (1, n_kv, T, D), SCALE, ks)
    assert_close(out, ref, what="attention T=1048576")


def test_refinement_that_removes_the_dominant_token():
    """KV head 0's token 0 holds nearly all of the softmax mass at resident precision
    and loses it once refined (its refinement bits sit where the query is negative),
    so the refined output is set by the other tokens; KV head 1 is ordinary.  Both
    heads must match the oracle."""
    T, n_kv, G = 96, 2, 2
    K, V = inputs.kv(54, 0, 1, n_kv, T, D)
    K[0, 0, 1:] *= np.float32(0.05)  # the other tokens of KV head 0: small keys, small logits
    # token 0 of KV head 0: codes 15, 0, then 3 everywhere (z = 0, s = 1 exactly):
    # resident values 12, 0, 0, ..; refined 15, 0, 3, ..
    K[0, 0, 0, :] = 3.0
    K[0, 0, 0, 0] = 15.0
    K[0, 0, 0, 1] = 0.0
    q = inputs.query(54, 0, 0, 1, n_kv * G, D).astype(np.float32)
    q[0, :G, :] = -1.0
    q[0, :G, 0] = 16.0
    q = q.astype(np.float16)
    kv = binding.QuantKV.from_host(K, V, 2, 2)
    qk, qv = o_attn.quantize_kv(K, 2, 2), o_attn.quantize_kv(V, 2, 2)
    k_res = nested.dequant_resident(qk).reshape(1, n_kv, T, D)
    k_full = nested.dequant_full(qk).reshape(1, n_kv, T, D)
    l_res = SCALE * (q[0, 0].astype(np.float64) @ k_res[0, 0].T)
    l_full = SCALE * (q[0, 0].astype(np.float64) @ k_full[0, 0].T)
    assert l_res[0] - np.max(l_res[1:]) > 8 and l_full[0] < np.max(l_full[1:]) - 8  # the construction holds
    ks = 3
    from gpu_util import token_gap
    for g in range(n_kv):
        assert token_gap(o_attn.token_scores(q[0, g * G:(g + 1) * G], k_res[0, g], SCALE), ks) >= 1e-4
    cache = binding.RefineCache([kv.resident_pool_desc()])
    out, sel, hit = binding.refined_attention(q, kv, SCALE, ks, cache=cache)
    torch.cuda.synchronize()
    ref, chosen = o_attn.refined_attention(q, qk, qv, (1, n_kv, T, D), SCALE, ks)
    assert sel.cpu().numpy()[0, 0].tolist() == chosen[(0, 0)] and 0 in chosen[(0, 0)]
    assert_close(out.cpu().numpy(), ref, what="dominant token refined away")


@pytest.mark.parametrize("b,r,G,T0", [(2, 2, 4, 300), (1, 1, 2, 40), (4, 4, 8, 700), (2, 2, 4, 4096 + 255), (2, 1, 1, 0)])
def test_fused_append_matches_append_then_attention(b, r, G, T0):
    """sf_refined_attn_decode_append against sf_kv_append of the same token followed by
    sf_refined_attn_decode: the cache (codes, sz words, refinement units), the
    selection and the hits bit for bit; the outputs to fp32 rounding (the value-sum
    records are added atomically, in no fixed order), and the fp16 output as the fp32
    one rounded to nearest even.  T0 = 0: the new token is the whole cache."""
    batch, n_kv = 2, 2
    K, V = inputs.kv(60 + b + G, 0, batch, n_kv, T0 + 1, D)
    q = inputs.query(60 + b + G, 0, 0, batch, n_kv * G, D)
    ks = max(1, selection.k_select(2, T0 + 1))
    res = []
    for fused in (False, True):
        kv = binding.QuantKV(batch, n_kv, T0 + 8, b, r)
        if T0 > 0:
            kv.append(K[:, :, :T0], V[:, :, :T0])
        cache = binding.RefineCache([kv.resident_pool_desc()])
        kn, vn = K[:, :, T0], V[:, :, T0]
        if fused:
            o16 = torch.empty((batch, n_kv * G, D), dtype=torch.int16, device="cuda")
            out, sel, hit = binding.refined_attention_append(q, kv, kn, vn, SCALE, ks, cache=cache, out_f16=o16)
        else:
            kv.append(kn[:, :, None], vn[:, :, None])
            out, sel, hit = binding.refined_attention(q, kv, SCALE, ks, cache=cache)
        torch.cuda.synchronize()
        assert kv.t_len == T0 + 1
        res.append(([t.cpu().numpy() for t in (kv.k_res, kv.k_sz, kv.v_res, kv.v_sz, kv.refine)],
                    out.cpu().numpy(), sel.cpu().numpy(), hit.cpu().numpy()))
    (bufs_a, out_a, sel_a, hit_a), (bufs_b, out_b, sel_b, hit_b) = res
    for x, y in zip(bufs_a, bufs_b):
        assert np.array_equal(x, y)
    assert np.array_equal(sel_a, sel_b) and np.array_equal(hit_a, hit_b)
    assert_close(out_b, out_a, rtol=1e-6, atol=1e-7, what="fused append")
    # the fp16 copy: the fp32 output rounded to nearest even
    assert np.array_equal(o16.cpu().numpy().view(np.float16), out_b.astype(np.float16))
