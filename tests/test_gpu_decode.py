"""GPU parity of the decode-step glue and of whole decode steps, through the C ABI.

Glue operations are compared with the fp64 oracle on the same inputs: exact where
the result is an integer, a gather or one fp32 add / fp16 rounding; within one fp16
ulp (rtol 2e-3) where the GPU rounds an fp32 result to fp16 and the oracle rounds
an fp64 one; within 1e-5 where the result stays fp32.

A decode step is checked operation by operation, each fed with the GPU's own inputs
(teacher forcing): the residual stream is rebuilt in fp64 from the GPU's GEMV
outputs, every GEMV's selection must be the oracle's top-k of the GPU's fp16 input
and its output the oracle GEMV on those channels, the appended KV codes are the
oracle's quantisation of the GPU's rotated key and value, and attention is the
oracle's on the KV head's selection, which must be a valid top-k."""
import math

import numpy as np
import pytest
import torch

from bit_decode_selective_amd import binding, decode, inputs
from oracle import attention as o_attn
from oracle import cache as o_cache
from oracle import decode as o_dec
from oracle import gemv as o_gemv
from oracle import nested, selection

from gpu_util import assert_close, topk_is_valid

pytestmark = pytest.mark.gpu

F16 = dict(rtol=2e-3, atol=1e-4)


def _f16(t):
    return t.cpu().view(torch.float16).numpy().astype(np.float64)


def test_embed_and_argmax():
    table = (np.random.default_rng(0).standard_normal((1000, 96)) * 3).astype(np.float16)
    dt = binding._f16_bits(table, "cuda")
    ids = np.array([5, 999, 0, -1, 1000], dtype=np.int32)
    h = binding.embed(dt, ids).cpu().numpy()
    want = np.zeros((5, 96))
    want[:3] = o_dec.embed(table, ids[:3])
    assert np.array_equal(h, want)
    for vocab in (1000, 151936):
        lg = np.random.default_rng(vocab).standard_normal((3, vocab)).astype(np.float32)
        lg[1, [7, 300, vocab - 1]] = 50.0  # equal maxima: the lowest index wins
        lg[2, :] = -3.0
        got = binding.argmax(torch.as_tensor(lg, device="cuda")).cpu().numpy()
        assert got.tolist() == o_dec.argmax(lg).tolist() and got[1] == 7 and got[2] == 0


@pytest.mark.parametrize("hidden", [256, 4096, 5000, 4098, 20480])
def test_add_rmsnorm(hidden):
    rng = np.random.default_rng(hidden)
    h = rng.standard_normal((3, hidden)).astype(np.float32)
    y = (rng.standard_normal((3, hidden)) * 0.5).astype(np.float32)
    w = inputs.norm_gain(9, 0, 0, hidden)
    ht = torch.as_tensor(h, device="cuda")
    x = binding.add_rmsnorm(ht, torch.as_tensor(y, device="cuda"), torch.as_tensor(w, device="cuda"), 1e-5)
    assert np.array_equal(ht.cpu().numpy(), h + y)  # one fp32 add
    assert_close(_f16(x), o_dec.rmsnorm((h + y).astype(np.float64), w, 1e-5), what="add+rmsnorm", **F16)
    x2 = binding.add_rmsnorm(ht, None, torch.as_tensor(w, device="cuda"), 1e-6)
    assert_close(_f16(x2), o_dec.rmsnorm((h + y).astype(np.float64), w, 1e-6), what="rmsnorm", **F16)


@pytest.mark.parametrize("norms", [False, True])
@pytest.mark.parametrize("pos", [0, 7, 8191, 131071])
def test_qk_rope(norms, pos):
    rng = np.random.default_rng(pos + norms)
    B, nq, nkv = 2, 8, 2
    q = rng.standard_normal((B, nq * 128)).astype(np.float32)
    k = (rng.standard_normal((B, nkv * 128)) * 2).astype(np.float32)
    wq = inputs.norm_gain(3, 0, 2, 128) if norms else None
    wk = inputs.norm_gain(3, 0, 3, 128) if norms else None
    T = lambda a: torch.as_tensor(a, device="cuda") if a is not None else None
    theta = 1e6 if norms else 5e5
    qh, ko = binding.qk_rope(T(q), T(k), nq, nkv, T(wq), T(wk), 1e-6, pos, theta)
    wq_, wk_ = o_dec.qk_heads(q.astype(np.float64), k.astype(np.float64), nq, nkv, 128, wq, wk, 1e-6, pos, theta)
    assert_close(_f16(qh), wq_, what="q", **F16)
    assert_close(ko.cpu().numpy(), wk_, rtol=1e-5, atol=1e-6, what="k")


def test_swiglu_and_to_f16():
    rng = np.random.default_rng(5)
    g = (rng.standard_normal(12288 * 2) * 4).astype(np.float32)
    u = rng.standard_normal(12288 * 2).astype(np.float32)
    act = binding.swiglu(torch.as_tensor(g, device="cuda"), torch.as_tensor(u, device="cuda"))
    assert_close(_f16(act), o_dec.swiglu(g.astype(np.float64), u.astype(np.float64)), what="swiglu", **F16)
    x = (rng.standard_normal(4099) * 100).astype(np.float32)
    assert np.array_equal(_f16(binding.to_f16(torch.as_tensor(x, device="cuda"))),
                          x.astype(np.float16).astype(np.float64))


TINY_LLAMA = decode.Spec("tiny-llama", 2, 256, 4, 2, 512, 1024, False, 500000.0, 1e-5)
TINY_QWEN = decode.Spec("tiny-qwen", 2, 256, 4, 2, 384, 1280, True, 1000000.0, 1e-6)


class Quants:
    """Oracle quantisation of each host weight, computed once per test."""

    def __init__(self, model):
        self.model, self.q = model, {}

    def __call__(self, key):
        if key not in self.q:
            m = self.model
            self.q[key] = nested.quantize(m.host[key], m.b, m.r, 128)
        return self.q[key]


def _pool_of(model, li, name):
    if li >= model.spec.layers:
        return model.pool_lm
    return model.layers[li].get("pool_" + name, -1)


def _gemv_check(model, li, names, x16, ys, sel_t, k_in, what, quants, lru=None, step=0, outputs=True):
    """Selection = oracle top-k of the GPU's fp16 input; the hit set of each matrix =
    the oracle LRU's (or every channel for resident pools); outputs = oracle GEMV on
    the hit channels."""
    ks = decode.k_select(model.ch_pct, k_in)
    x = x16.astype(np.float16)
    sel = sel_t.cpu().numpy()[:ks].tolist()
    assert sel == selection.select_channels(x, ks), what
    for name, y in zip(names, ys):
        key = (li, name)
        hit = model.hits[(li if li < model.spec.layers else -1, name if li < model.spec.layers else "lm_head")]
        got_hits = (hit.cpu().numpy()[:ks] >= 0).tolist()
        if lru is None:
            want_hits = [True] * ks  # resident pools
        else:
            want_hits = lru[_pool_of(model, li, name)].lookup(sel, step)
        assert got_hits == want_hits, f"{what} {name} hits"
        if outputs:
            chans = [k for k, h in zip(sel, want_hits) if h]
            assert_close(y, o_gemv.refined_gemv(quants(key), x, chans), what=f"{what} {name}")


TENSOR = {"q": inputs.Q_PROJ, "k": inputs.K_PROJ, "v": inputs.V_PROJ, "o": inputs.O_PROJ, "gate": inputs.GATE,
          "up": inputs.UP, "down": inputs.DOWN}


def _lag_check(model, li, name, x16, quants, what):
    """The late contribution the GPU computed for this GEMV (its lag buffer) against
    the oracle's on the GEMV's own misses; returns the GPU's (fp64)."""
    bf = model.buf[li]
    k_in = model.layers[li][name].k_in
    ks = decode.k_select(model.ch_pct, k_in)
    sel = bf["sel_" + name].cpu().numpy()[:ks]
    hit = model.hits[(li, name)].cpu().numpy()[:ks]
    late = [int(k) for k, h in zip(sel, hit) if h < 0]
    got = bf["lag_" + name].cpu().numpy().astype(np.float64)
    assert_close(got, o_gemv.lag_delta(quants((li, name)), x16.astype(np.float16), late), what=f"{what} late {name}")
    return got


def _run_steps(spec, batch, T0, steps, cfg, b=2, r=2, pool_frac=None, output_steps=None, fetch_lag=False,
               fetch_lead=False, producer_select=False):
    """Teacher-forced decode steps; every operation of every step checked against the
    oracle on the GPU's own inputs.  With pool_frac, the LRU pools of every weight,
    KV cache and lm_head are replayed by the oracle (``cache.LRUPool``): each GEMV's
    and each attention's hit set must be the oracle's, and every pool's resident set
    must agree after each step's fill.  output_steps: the steps whose operation
    outputs are compared (all by default); selections and hit sets are checked at
    every step."""
    src = decode.HostWeights(cfg)
    model = decode.DecodeModel(spec, batch, T0 + steps, src, b=b, r=r, pool_frac=pool_frac, fetch_lag=fetch_lag,
                               fetch_lead=fetch_lead, producer_select=producer_select)
    assert model.fetch_lag == fetch_lag and model.fetch_lead == fetch_lead
    for li in range(spec.layers):
        for name, t in TENSOR.items():
            model.host[(li, name)] = model.host[(li, t)]
    model.host[(spec.layers, "lm_head")] = model.host[(spec.layers, inputs.LM_HEAD)]
    model.fill_kv(T0, src)
    quants = Quants(model)
    lru = None
    if pool_frac is not None:
        lru = {i: o_cache.LeadPool(int(p.capacity), int(p.lead_slots)) for i, p in enumerate(model._pools)}
    S, d = spec, spec.head_dim
    kv_host = {li: model.host[("kv", li)] for li in range(S.layers)}
    appended = {li: ([], []) for li in range(S.layers)}
    ids = inputs.tokens(cfg, steps, batch, S.vocab)
    for step in range(steps):
        outs = output_steps is None or step in output_steps
        pos = model.pos
        nxt = model.step(ids[step])
        torch.cuda.synchronize()
        binding.check_workspaces()
        # rebuild the residual stream in fp64 from the GPU's op outputs
        h = o_dec.embed(model.host["embed"], ids[step])
        late_o = late_down = None  # the previous layer's late contributions (fetch lag)
        for li, L in enumerate(model.layers):
            bf = {k: v for k, v in model.buf[li].items()}
            if late_o is not None:
                h = h + late_o
            x = _f16(bf["x_attn"])
            assert_close(x, o_dec.to_f16(o_dec.rmsnorm(h, L["attn_norm"].cpu().numpy(), S.eps)).astype(np.float64),
                         what=f"layer {li} attn norm", **F16)
            if fetch_lead and li + 1 < S.layers:
                # layer li + 1's channels predicted from this residual stream, then
                # prefetched into its pools' lead slots (in the GPU's order)
                nx, bn = model.layers[li + 1], model.buf[li + 1]
                ks_h = decode.k_select(model.ch_pct, S.hidden)
                for norm_key, sfx, names in (("attn_norm", "attn", ("q", "k", "v")), ("ffn_norm", "ffn", ("gate", "up"))):
                    xp = _f16(bn["x_pred_" + sfx])
                    assert_close(xp, o_dec.to_f16(o_dec.rmsnorm(h, nx[norm_key].cpu().numpy(), S.eps)).astype(np.float64),
                                 what=f"layer {li} prediction for {li + 1} ({sfx})", **F16)
                    sp = bn["sel_pred_" + sfx].cpu().numpy()[:ks_h].tolist()
                    assert sp == selection.select_channels(xp.astype(np.float16), ks_h), (step, li, sfx)
                    for n in names:
                        lru[nx["pool_" + n]].prefetch(sp)
            ys = [bf[n].cpu().numpy() for n in ("q", "k", "v")]
            _gemv_check(model, li, ("q", "k", "v"), x, ys, bf["sel_attn"], S.hidden, f"step {step} layer {li} qkv",
                        quants, lru, step, outs)
            qn = L["q_norm"].cpu().numpy() if S.qk_norm else None
            kn = L["k_norm"].cpu().numpy() if S.qk_norm else None
            qh, kh = o_dec.qk_heads(ys[0], ys[1], S.n_q, S.n_kv, d, qn, kn, S.eps, pos, S.theta)
            q16 = _f16(bf["q16"])
            assert_close(q16, qh, what="q rope", **F16)
            k_rot = bf["k_rot"].cpu().numpy()
            assert_close(k_rot, kh, rtol=1e-5, atol=1e-6, what="k rope")
            # the cache: synthetic prefix + the GPU's rotated keys / values of the steps so far
            appended[li][0].append(k_rot.reshape(batch, S.n_kv, 1, d))
            appended[li][1].append(ys[2].reshape(batch, S.n_kv, 1, d))
            K = np.concatenate([kv_host[li][0]] + appended[li][0], axis=2)
            V = np.concatenate([kv_host[li][1]] + appended[li][1], axis=2)
            T = pos + 1
            qk = o_attn.quantize_kv(K, model.kv_b, model.kv_r)
            qv = o_attn.quantize_kv(V, model.kv_b, model.kv_r)
            kt = decode.k_select(model.tok_pct, T)
            n_sel = batch * S.n_kv * kt
            sel = bf["sel_tok"].reshape(-1)[:n_sel].reshape(batch, S.n_kv, kt).cpu().numpy()
            hit = bf["hit_tok"].reshape(-1)[:n_sel].reshape(batch, S.n_kv, kt).cpu().numpy()
            scale = 1.0 / math.sqrt(d)
            k_res = nested.dequant_resident(qk).reshape(batch, S.n_kv, T, d)
            G = S.n_q // S.n_kv
            for bi in range(batch):
                for g in range(S.n_kv):
                    sc = o_attn.token_scores(q16.astype(np.float16)[bi, g * G:(g + 1) * G], k_res[bi, g], scale)
                    ok, separated = topk_is_valid(sc, sel[bi, g].tolist(), kt)
                    assert ok, (step, li, bi, g)
                    if separated:
                        assert sel[bi, g].tolist() == selection.top_k(sc, kt), (step, li, bi, g)
            sel_map = {(bi, g): sel[bi, g].tolist() for bi in range(batch) for g in range(S.n_kv)}
            hits = None
            if lru is not None:
                units = [(bi * S.n_kv + g) * model.t_cap + int(t) for bi in range(batch) for g in range(S.n_kv)
                         for t in sel[bi, g]]
                want = lru[L["pool_kv"]].lookup(units, step)
                assert (hit.reshape(-1) >= 0).tolist() == want, f"step {step} layer {li} KV hits"
                hits = {(bi, g): {int(t) for t, hh in zip(sel[bi, g], hit[bi, g]) if hh >= 0}
                        for bi in range(batch) for g in range(S.n_kv)}
            attn = bf["attn"].cpu().numpy()
            if outs:
                ref, _ = o_attn.refined_attention(q16.astype(np.float16), qk, qv, (batch, S.n_kv, T, d), scale, kt,
                                                  sel_in=sel_map, hits=hits)
                assert_close(attn, ref, what=f"step {step} layer {li} attention")
            a16 = _f16(bf["a16"])
            assert np.array_equal(a16, attn.reshape(batch, -1).astype(np.float16).astype(np.float64))
            o = bf["o"].cpu().numpy()
            _gemv_check(model, li, ("o",), a16, [o], bf["sel_o"], S.n_q * d, f"step {step} layer {li} o", quants, lru,
                        step, outs)
            h = h + o.astype(np.float64)
            if late_down is not None:
                h = h + late_down
            if fetch_lag:
                late_o = _lag_check(model, li, "o", a16, quants, f"step {step} layer {li}")
            x2 = _f16(bf["x_ffn"])
            assert_close(x2, o_dec.to_f16(o_dec.rmsnorm(h, L["ffn_norm"].cpu().numpy(), S.eps)).astype(np.float64),
                         what=f"layer {li} ffn norm", **F16)
            gu = [bf[n].cpu().numpy() for n in ("gate", "up")]
            _gemv_check(model, li, ("gate", "up"), x2, gu, bf["sel_ffn"], S.hidden, f"step {step} layer {li} gate/up",
                        quants, lru, step, outs)
            act = _f16(bf["act"])
            assert_close(act, o_dec.swiglu(gu[0], gu[1]), what="swiglu", **F16)
            dn = bf["down"].cpu().numpy()
            _gemv_check(model, li, ("down",), act, [dn], bf["sel_down"], S.ffn, f"step {step} layer {li} down", quants,
                        lru, step, outs)
            h = h + dn.astype(np.float64)
            if fetch_lag and li < S.layers - 1:
                late_down = _lag_check(model, li, "down", act, quants, f"step {step} layer {li}")
        if late_o is not None:
            h = h + late_o
        xf = _f16(model.x_final)
        assert_close(xf, o_dec.to_f16(o_dec.rmsnorm(h, model.final_norm.cpu().numpy(), S.eps)).astype(np.float64),
                     what="final norm", **F16)
        logits = model.logits.cpu().numpy()
        _gemv_check(model, S.layers, ("lm_head",), xf, [logits], model.sel_lm, S.hidden, f"step {step} lm_head",
                    quants, lru, step, outs)
        assert nxt.cpu().numpy().tolist() == o_dec.argmax(logits).tolist()
        if lru is not None:
            for i, p in lru.items():
                p.fill(step)
                assert model.cache.resident(i, max(1, p.capacity)) == p.resident(), (step, i)


TINY_LLAMA = decode.Spec("tiny-llama", 2, 256, 4, 2, 512, 1024, False, 500000.0, 1e-5)
TINY_QWEN = decode.Spec("tiny-qwen", 2, 256, 4, 2, 384, 1280, True, 1000000.0, 1e-6)


@pytest.mark.parametrize("spec", [TINY_LLAMA, TINY_QWEN], ids=lambda s: s.name)
@pytest.mark.parametrize("batch", [1, 2])
@pytest.mark.parametrize("producer_select", [False, True], ids=["gemv-selects", "producer-selects"])
def test_decode_steps(spec, batch, producer_select):
    _run_steps(spec, batch, 40, 2, 70 + batch, producer_select=producer_select)


@pytest.mark.parametrize("spec", [TINY_LLAMA, TINY_QWEN], ids=lambda s: s.name)
def test_decode_steps_batch8(spec):
    """Batch 8: every GEMV on the batched MFMA kernel, its channels selected by the
    launch's own first workgroup over all eight rows."""
    _run_steps(spec, 8, 40, 2, 78)


@pytest.mark.parametrize("spec", [TINY_LLAMA, TINY_QWEN], ids=lambda s: s.name)
@pytest.mark.parametrize("producer_select", [False, True], ids=["gemv-selects", "producer-selects"])
def test_decode_steps_lru_pools(spec, producer_select):
    """Small decoders with LRU pools holding 25% of every tensor's units over 8 steps."""
    _run_steps(spec, 2, 60, 8, 80, pool_frac=0.25, producer_select=producer_select)


@pytest.mark.parametrize("spec", [TINY_LLAMA, TINY_QWEN], ids=lambda s: s.name)
def test_decode_steps_fetch_lag(spec):
    """Fetch lag with 25% LRU pools over 6 steps: each o / down projection's late
    contribution (its missed channels, read from the host store on the side stream)
    against the oracle, and every later operation against the oracle on a residual
    stream that carries it from the next update on."""
    _run_steps(spec, 2, 60, 6, 85, pool_frac=0.25, fetch_lag=True)


@pytest.mark.parametrize("spec", [TINY_LLAMA, TINY_QWEN], ids=lambda s: s.name)
def test_decode_steps_fetch_lead(spec):
    """Fetch lead with 25% LRU pools over 6 steps (3 layers): each layer's q/k/v and
    gate/up channels for the next layer predicted from its residual stream (checked
    against the oracle), prefetched into lead slots, and every later lookup's hit set
    equal to the oracle policy's (LRU slots plus lead slots)."""
    spec3 = decode.Spec(spec.name, 3, spec.hidden, spec.n_q, spec.n_kv, spec.ffn, spec.vocab, spec.qk_norm,
                        spec.theta, spec.eps)
    _run_steps(spec3, 2, 60, 6, 86, pool_frac=0.25, fetch_lead=True)


def test_decode_full_width_llama_fetch_lead_and_lag():
    """Full-width Llama layers (2+2 bits, 10% pools) with fetch lead and fetch lag
    together, 4 steps; outputs checked on the last."""
    _run_steps(WIDE_LLAMA, 1, 128, 4, 87, pool_frac=0.10, output_steps={3}, fetch_lag=True, fetch_lead=True)


# full hidden width, two layers, a 4096-token vocabulary (the lm_head's shape aside,
# every matrix has the model's own size)
WIDE_LLAMA = decode.Spec("llama-3.1-8b-width-2-layers", 2, 4096, 32, 8, 14336, 4096, False, 500000.0, 1e-5)
WIDE_QWEN = decode.Spec("qwen3-8b-width-2-layers", 2, 4096, 32, 8, 12288, 4096, True, 1000000.0, 1e-6)


def test_decode_full_width_qwen3_pools25():
    """The Qwen3-8B workload's step at full width: 2+2-bit weights and KV, pools of 25%
    with LRU replacement and deterministic fills, 8 steps; every operation's output
    checked on the first and last step, selections and hit sets on all."""
    _run_steps(WIDE_QWEN, 1, 192, 8, 90, pool_frac=0.25, output_steps={0, 7})


def test_decode_full_width_qwen3_batch8_pools25():
    """The Qwen3-8B workload's step at full width and batch 8 (the batched MFMA GEMVs,
    64 token selections per layer), pools of 25%, 4 steps; outputs checked on the first
    and last step, selections and hit sets on all."""
    _run_steps(WIDE_QWEN, 8, 160, 4, 92, pool_frac=0.25, output_steps={0, 3})


def test_decode_full_width_llama_w3r1_pools10():
    """The 128K workload's formats at full width: 3-bit weights + 1 refinement bit,
    2+2-bit KV, pools of 10%, 8 steps (short context)."""
    _run_steps(WIDE_LLAMA, 1, 192, 8, 91, b=3, r=1, pool_frac=0.10, output_steps={0, 7})


@pytest.mark.parametrize("batch", [1, 3, 16])
@pytest.mark.parametrize("n,k_sel", [(4096, 123), (14336, 431), (12288, 369), (256, 128), (4096, 0), (1024, 1024),
                                     (40, 1)])
def test_producers_select_their_channels(batch, n, k_sel):
    """sf_add_rmsnorm_select / sf_swiglu_select / sf_to_f16_select: the fp16 output as
    the oracle forms it (one fp16 rounding: within one ulp; the cast exactly), and the
    selection exactly the oracle top-k by max-over-rows |x| of that output."""
    rng = np.random.default_rng(n + batch + k_sel)
    T = lambda a: torch.as_tensor(a, device="cuda")
    h = rng.standard_normal((batch, n)).astype(np.float32)
    y = (rng.standard_normal((batch, n)) * 0.5).astype(np.float32)
    w = inputs.norm_gain(9, 1, 0, n)
    ht = T(h)
    x, sel = binding.add_rmsnorm_select(ht, T(y), T(w), 1e-5, k_sel)
    assert np.array_equal(ht.cpu().numpy(), h + y)
    xg = _f16(x)
    assert_close(xg, o_dec.rmsnorm((h + y).astype(np.float64), w, 1e-5), what="norm", **F16)
    assert sel.cpu().numpy().tolist() == selection.select_channels(xg.astype(np.float16), k_sel)
    g = (rng.standard_normal((batch, n)) * 4).astype(np.float32)
    u = rng.standard_normal((batch, n)).astype(np.float32)
    act, sel = binding.swiglu_select(T(g), T(u), k_sel)
    ag = _f16(act)
    assert_close(ag, o_dec.swiglu(g.astype(np.float64), u.astype(np.float64)), what="swiglu", **F16)
    assert sel.cpu().numpy().tolist() == selection.select_channels(ag.astype(np.float16), k_sel)
    v = (rng.standard_normal((batch, n)) * 30).astype(np.float32)
    c, sel = binding.to_f16_select(T(v), k_sel)
    cg = _f16(c)
    assert np.array_equal(cg, v.astype(np.float16).astype(np.float64))
    assert sel.cpu().numpy().tolist() == selection.select_channels(cg.astype(np.float16), k_sel)


def test_producer_ties_go_to_lower_channels():
    """Equal magnitudes (including signs) at the k-th place: the lower channels win."""
    v = np.zeros((2, 512), dtype=np.float32)
    v[0, [7, 100, 300, 301]] = [2.0, -2.0, 2.0, 1.0]
    v[1, [5, 300]] = [-2.0, 3.0]
    c, sel = binding.to_f16_select(torch.as_tensor(v, device="cuda"), 3)
    assert sel.cpu().numpy().tolist() == [5, 7, 300]
