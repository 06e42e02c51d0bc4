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


def _gemv_check(model, li, names, x16, ys, sel_t, k_in, what):
    """Selection = oracle top-k of the GPU's fp16 input; outputs = oracle GEMV on it."""
    ks = decode.k_select(model.ch_pct, k_in)
    x = x16.astype(np.float16)
    sel = sel_t.cpu().numpy()[:ks].tolist()
    assert sel == selection.select_channels(x, ks), what
    for name, y in zip(names, ys):
        W = model.host[(li, name)]
        hit = model.hits[(li if li < model.spec.layers else -1, name if li < model.spec.layers else "lm_head")]
        assert np.all(hit.cpu().numpy()[:ks] >= 0)  # resident pools
        q = nested.quantize(W, model.b, model.r, 128)
        assert_close(y, o_gemv.refined_gemv(q, x, sel), what=f"{what} {name}")


TENSOR = {"q": inputs.Q_PROJ, "k": inputs.K_PROJ, "v": inputs.V_PROJ, "o": inputs.O_PROJ, "gate": inputs.GATE,
          "up": inputs.UP, "down": inputs.DOWN}


@pytest.mark.parametrize("spec", [TINY_LLAMA, TINY_QWEN], ids=lambda s: s.name)
@pytest.mark.parametrize("batch", [1, 2])
def test_decode_steps(spec, batch):
    src = decode.HostWeights(70 + batch)
    T0, steps = 40, 2
    model = decode.DecodeModel(spec, batch, T0 + steps, src)
    # host weight keys by name
    for li in range(spec.layers):
        for name, t in TENSOR.items():
            model.host[(li, name)] = model.host[(li, t)]
    model.host[(spec.layers, "lm_head")] = model.host[(spec.layers, inputs.LM_HEAD)]
    model.fill_kv(T0, src)
    S, d = spec, spec.head_dim
    kv_host = {li: model.host[("kv", li)] for li in range(S.layers)}
    appended = {li: ([], []) for li in range(S.layers)}
    ids = inputs.tokens(70, steps, batch, S.vocab)
    for step in range(steps):
        pos = model.pos
        nxt = model.step(ids[step])
        torch.cuda.synchronize()
        # rebuild the residual stream in fp64 from the GPU's op outputs
        h = o_dec.embed(model.host["embed"], ids[step])
        for li, L in enumerate(model.layers):
            bf = {k: v for k, v in model.buf[li].items()}
            x = _f16(bf["x_attn"])
            assert_close(x, o_dec.to_f16(o_dec.rmsnorm(h, L["attn_norm"].cpu().numpy(), S.eps)).astype(np.float64),
                         what=f"layer {li} attn norm", **F16)
            ys = [bf[n].cpu().numpy() for n in ("q", "k", "v")]
            _gemv_check(model, li, ("q", "k", "v"), x, ys, bf["sel_attn"], S.hidden, f"step {step} layer {li} qkv")
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
            sel = bf["sel_tok"].reshape(-1)[: batch * S.n_kv * kt].reshape(batch, S.n_kv, kt).cpu().numpy()
            scale = 1.0 / math.sqrt(d)
            k_res = nested.dequant_resident(qk).reshape(batch, S.n_kv, T, d)
            G = S.n_q // S.n_kv
            for bi in range(batch):
                for g in range(S.n_kv):
                    sc = o_attn.token_scores(q16.astype(np.float16)[bi, g * G:(g + 1) * G], k_res[bi, g], scale)
                    ok, _ = topk_is_valid(sc, sel[bi, g].tolist(), kt)
                    assert ok, (step, li, bi, g)
            sel_map = {(bi, g): sel[bi, g].tolist() for bi in range(batch) for g in range(S.n_kv)}
            ref, _ = o_attn.refined_attention(q16.astype(np.float16), qk, qv, (batch, S.n_kv, T, d), scale, kt,
                                              sel_in=sel_map)
            attn = bf["attn"].cpu().numpy()
            assert_close(attn, ref, what=f"step {step} layer {li} attention")
            a16 = _f16(bf["a16"])
            assert np.array_equal(a16, attn.reshape(batch, -1).astype(np.float16).astype(np.float64))
            o = bf["o"].cpu().numpy()
            _gemv_check(model, li, ("o",), a16, [o], bf["sel_o"], S.n_q * d, f"layer {li} o")
            h = h + o.astype(np.float64)
            x2 = _f16(bf["x_ffn"])
            assert_close(x2, o_dec.to_f16(o_dec.rmsnorm(h, L["ffn_norm"].cpu().numpy(), S.eps)).astype(np.float64),
                         what=f"layer {li} ffn norm", **F16)
            gu = [bf[n].cpu().numpy() for n in ("gate", "up")]
            _gemv_check(model, li, ("gate", "up"), x2, gu, bf["sel_ffn"], S.hidden, f"layer {li} gate/up")
            act = _f16(bf["act"])
            assert_close(act, o_dec.swiglu(gu[0], gu[1]), what="swiglu", **F16)
            dn = bf["down"].cpu().numpy()
            _gemv_check(model, li, ("down",), act, [dn], bf["sel_down"], S.ffn, f"layer {li} down")
            h = h + dn.astype(np.float64)
        xf = _f16(model.x_final)
        assert_close(xf, o_dec.to_f16(o_dec.rmsnorm(h, model.final_norm.cpu().numpy(), S.eps)).astype(np.float64),
                     what="final norm", **F16)
        logits = model.logits.cpu().numpy()
        _gemv_check(model, S.layers, ("lm_head",), xf, [logits], model.sel_lm, S.hidden, "lm_head")
        assert nxt.cpu().numpy().tolist() == o_dec.argmax(logits).tolist()
