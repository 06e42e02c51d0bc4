"""One greedy decode step of a Llama-3.1- or Qwen3-shaped model through the C ABI.

Host orchestration only: every operation of the step is a library call (embedding,
residual add + RMSNorm, refined GEMVs, q/k head norm + rotary embedding, KV append,
refined attention, SwiGLU, lm_head GEMV, argmax).  The argument tuples of a step are
built once per position, so a step is a fixed sequence of launches on one stream
(capturable as a HIP graph).  Every intermediate has its own buffer per layer, so a
finished step can be inspected operation by operation.

Weights are random (no trained checkpoints are available); their shapes are the
public model shapes.  The KV cache before the first step is filled with synthetic
keys and values (not by running the model on a prompt).
"""
from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass

import numpy as np

from . import binding, inputs


@dataclass(frozen=True)
class Spec:
    name: str
    layers: int
    hidden: int
    n_q: int
    n_kv: int
    ffn: int
    vocab: int
    qk_norm: bool
    theta: float
    eps: float
    head_dim: int = 128


LLAMA31_8B = Spec("llama-3.1-8b", 32, 4096, 32, 8, 14336, 128256, False, 500000.0, 1e-5)
QWEN3_8B = Spec("qwen3-8b", 36, 4096, 32, 8, 12288, 151936, True, 1000000.0, 1e-6)


def k_select(percent, n):
    return (percent * n + 99) // 100


class HostWeights:
    """Seeded numpy weights (small models for the step tests)."""

    def __init__(self, cfg):
        self.cfg = cfg

    def matrix(self, layer, tensor, n_out, k_in):
        return inputs.weight(self.cfg, layer, tensor, n_out, k_in)

    def gain(self, layer, which, dim):
        return inputs.norm_gain(self.cfg, layer, which, dim)

    def embedding(self, vocab, hidden):
        return inputs.weight(self.cfg, 0, inputs.EMBED, vocab, hidden, std=1.0).astype(np.float16)

    def kv(self, layer, batch, n_kv, T, d):
        return inputs.kv(self.cfg, layer, batch, n_kv, T, d)


class DeviceWeights:
    """The same distributions drawn on the device (full-size models)."""

    def __init__(self, seed, device):
        import torch

        self.g = torch.Generator(device=device)
        self.g.manual_seed(seed)
        self.device = device

    def matrix(self, layer, tensor, n_out, k_in):
        return inputs.torch_weight(self.g, n_out, k_in, device=self.device)

    def gain(self, layer, which, dim):
        return inputs.norm_gain(int(self.g.initial_seed()), layer, which, dim)

    def embedding(self, vocab, hidden):
        import torch

        return torch.randn((vocab, hidden), generator=self.g, device=self.device, dtype=torch.float32).half()

    def kv(self, layer, batch, n_kv, T, d):
        return inputs.torch_kv(self.g, batch, n_kv, T, d, device=self.device)


# gain ids of the norms (``inputs.norm_gain`` keys)
ATTN_NORM, FFN_NORM, Q_NORM, K_NORM, FINAL_NORM = range(5)


class DecodeModel:
    """Quantised weights, KV caches, refinement cache and per-layer buffers.

    b, r       weight format; kv_b, kv_r the KV format
    ch_pct     percent of input channels selected per GEMV (also the lm_head)
    tok_pct    percent of tokens selected per (batch, kv head)
    pool_frac  None: every refinement unit resident on the device (pools never
               miss); else the device slots per pool as a fraction of its units,
               filled from pinned host stores by the cache (LRU)
    head       False: the layers only (no embedding, final norm, lm_head or argmax);
               the step then starts from the residual state in ``h``
    producer_select
               the kernel that forms each GEMV input also selects its channels
               (sf_add_rmsnorm_select, sf_to_f16_select, sf_swiglu_select) and the
               GEMV takes that selection as sel_in (batch <= 16).  Off by default:
               each GEMV then selects its channels itself, in one workgroup while
               the others stream the resident codes, which hides the selection
               (a producer's selection runs on one workgroup before the GEMV starts)
    store_dir  with pool_frac: weight pools read their units from files in this
               directory (the SSD tier); KV pools stay in pinned host memory
    fetch_lead with pool_frac: at each layer l but the last, layer l + 1's q/k/v and
               gate/up channels are predicted from the residual stream entering
               layer l (its RMSNorms with layer l + 1's gains, then top-k) and
               prefetched on the side stream into lead slots of those pools
               (sf_refine_cache_prefetch); layer l + 1's q/k/v GEMV waits for them
    fetch_lag  with pool_frac: the selected channels of the o and down projections
               that missed are read from the host store on the side stream
               (sf_refine_lag_delta) and their contribution is added to the
               residual stream at its next update (the next layer's residual add,
               or the final norm); the last layer's down has no later update
    """

    def __init__(self, spec, batch, t_cap, src, b=2, r=2, kv_b=2, kv_r=2, ch_pct=3, tok_pct=2, pool_frac=None,
                 cache_mode=binding.SF_CACHE_DETERMINISTIC, device="cuda", head=True, producer_select=False,
                 store_dir=None, fetch_lag=False, fetch_lead=False):
        import torch

        self.torch, self.spec, self.batch, self.t_cap = torch, spec, batch, t_cap
        self.head = head
        self.producer_select = producer_select and batch <= 16
        # fetch lag: the o and down projections' missed refinements are read on the
        # side stream and added at the residual stream's next update
        self.fetch_lag = bool(fetch_lag) and pool_frac is not None and r > 0 and store_dir is None
        # fetch lead: layer l + 1's q/k/v and gate/up channels are predicted from the
        # residual stream entering layer l and prefetched into lead slots meanwhile
        self.fetch_lead = bool(fetch_lead) and pool_frac is not None and r > 0 and store_dir is None
        self.b, self.r, self.kv_b, self.kv_r = b, r, kv_b, kv_r
        self.ch_pct, self.tok_pct = ch_pct, tok_pct
        dev = torch.device(device)
        self.dev = dev
        S, H, d = spec, spec.hidden, spec.head_dim
        self.host = {}  # fp32 weights kept for the oracle checks (HostWeights only)
        keep_host = isinstance(src, HostWeights)
        pools = []
        stores = {}  # pool index -> pinned host store

        def quant(layer, tensor, n, k):
            W = src.matrix(layer, tensor, n, k)
            if keep_host:
                self.host[(layer, tensor)] = W
            qw = binding.QuantWeight.from_host(W, b, r) if keep_host else binding.QuantWeight.from_device(W, b, r)
            return qw

        lead_of = lambda n_lookup: n_lookup if self.fetch_lead else 0

        def add_pool(unit_bytes_obj, n_lookup, static=True, lead=0):
            """n_lookup: unit ids one step looks up in the pool (sizes its lookup log).
            With store_dir, a static pool (a weight matrix) reads its units from a
            file there (the SSD tier); KV units change every step and stay in RAM."""
            if pool_frac is None:
                pools.append(unit_bytes_obj.resident_pool_desc())
            elif store_dir is not None and static:
                path = os.path.join(store_dir, f"refine_pool{len(pools)}.bin")
                binding.write_store_file(path, unit_bytes_obj.refine)
                n = unit_bytes_obj.refine.shape[0]
                pools.append(binding.file_pool_desc(path, unit_bytes_obj.unit_bytes, n, max(0, int(pool_frac * n)),
                                                    max_lookup=n_lookup))
            else:
                st = unit_bytes_obj.host_store()
                stores[len(pools)] = st
                cap = max(0, int(pool_frac * st.shape[0]))
                pools.append(binding.host_pool_desc(st, cap, max_lookup=n_lookup, lead_slots=lead))
            return len(pools) - 1

        self.layers = []
        for li in range(S.layers):
            L = {}
            L["q"] = quant(li, inputs.Q_PROJ, S.n_q * d, H)
            L["k"] = quant(li, inputs.K_PROJ, S.n_kv * d, H)
            L["v"] = quant(li, inputs.V_PROJ, S.n_kv * d, H)
            L["o"] = quant(li, inputs.O_PROJ, H, S.n_q * d)
            L["gate"] = quant(li, inputs.GATE, S.ffn, H)
            L["up"] = quant(li, inputs.UP, S.ffn, H)
            L["down"] = quant(li, inputs.DOWN, H, S.ffn)
            if r > 0:
                for name in ("q", "k", "v", "o", "gate", "up", "down"):
                    n_look = k_select(ch_pct, L[name].k_in)
                    lead = lead_of(n_look) if name in ("q", "k", "v", "gate", "up") and li > 0 else 0
                    L["pool_" + name] = add_pool(L[name], n_look, lead=lead)
            L["attn_norm"] = torch.as_tensor(src.gain(li, ATTN_NORM, H), device=dev)
            L["ffn_norm"] = torch.as_tensor(src.gain(li, FFN_NORM, H), device=dev)
            if S.qk_norm:
                L["q_norm"] = torch.as_tensor(src.gain(li, Q_NORM, d), device=dev)
                L["k_norm"] = torch.as_tensor(src.gain(li, K_NORM, d), device=dev)
            L["index"] = li
            kv = binding.QuantKV(batch, S.n_kv, t_cap, kv_b, kv_r, device=dev)
            L["kv"] = kv
            if kv_r > 0:
                # store taken before any token: refilled from the device copy in fill_kv
                L["pool_kv"] = add_pool(kv, batch * S.n_kv * k_select(tok_pct, t_cap), static=False)
            self.layers.append(L)
            torch.cuda.synchronize()
        self.final_norm = torch.as_tensor(src.gain(S.layers, FINAL_NORM, H), device=dev)
        self.pool_lm = -1
        if head:
            emb = src.embedding(S.vocab, H)
            if keep_host:
                self.host["embed"] = emb
            self.embed = binding._f16_bits(emb, dev)
            self.lm_head = quant(S.layers, inputs.LM_HEAD, S.vocab, H)
            self.pool_lm = add_pool(self.lm_head, k_select(ch_pct, H)) if r > 0 else -1
        self._pool_frac = pool_frac
        self._pools, self._stores = pools, stores
        self.cache = binding.RefineCache(pools, mode=cache_mode, device=dev, keep=list(stores.values())) if pools else None
        self.side = torch.cuda.Stream(device=dev)
        self._alloc_buffers()
        self.pos = 0

    # ---- KV prefix -------------------------------------------------------------------
    def fill_kv(self, T0, src):
        """Synthetic keys/values for positions [0, T0) of every layer (not a prefill)."""
        for li, L in enumerate(self.layers):
            K, V = src.kv(li, self.batch, self.spec.n_kv, T0, self.spec.head_dim)
            if isinstance(src, HostWeights):
                self.host[("kv", li)] = (K, V)
            L["kv"].append(K, V)
            if self._pool_frac is not None and self.kv_r > 0:
                # the host store holds the prefix's refinement units too (one store per pool)
                st = self._stores[L["pool_kv"]]
                st.copy_(L["kv"].refine.reshape(st.shape).to("cpu"))
        self.pos = T0
        self.torch.cuda.synchronize()

    # ---- buffers -----------------------------------------------------------------------
    def _alloc_buffers(self):
        torch, S, B, d = self.torch, self.spec, self.batch, self.spec.head_dim
        f32 = dict(dtype=torch.float32, device=self.dev)
        i16 = dict(dtype=torch.int16, device=self.dev)
        self.h = torch.zeros((B, S.hidden), **f32)
        self.ids = torch.zeros(B, dtype=torch.int32, device=self.dev)
        self.next_ids = torch.zeros(B, dtype=torch.int32, device=self.dev)
        self.buf = []
        for _ in range(S.layers):
            self.buf.append({
                "x_attn": torch.empty((B, S.hidden), **i16),
                "q": torch.empty((B, S.n_q * d), **f32),
                "k": torch.empty((B, S.n_kv * d), **f32),
                "k_rot": torch.empty((B, S.n_kv, d), **f32),
                "v": torch.empty((B, S.n_kv * d), **f32),
                "q16": torch.empty((B, S.n_q, d), **i16),
                "attn": torch.empty((B, S.n_q, d), **f32),
                "a16": torch.empty((B, S.n_q * d), **i16),
                "o": torch.empty((B, S.hidden), **f32),
                "x_ffn": torch.empty((B, S.hidden), **i16),
                "gate": torch.empty((B, S.ffn), **f32),
                "up": torch.empty((B, S.ffn), **f32),
                "act": torch.empty((B, S.ffn), **i16),
                "x_pred_attn": torch.zeros((B, S.hidden), **i16),
                "x_pred_ffn": torch.zeros((B, S.hidden), **i16),
                "sel_pred_attn": torch.zeros(max(1, k_select(self.ch_pct, S.hidden)), dtype=torch.int32,
                                             device=self.dev),
                "sel_pred_ffn": torch.zeros(max(1, k_select(self.ch_pct, S.hidden)), dtype=torch.int32,
                                            device=self.dev),
                "lag_o": torch.zeros((B, S.hidden), **f32),
                "lag_down": torch.zeros((B, S.hidden), **f32),
                "down": torch.empty((B, S.hidden), **f32),
                "sel_attn": torch.empty(max(1, k_select(self.ch_pct, S.hidden)), dtype=torch.int32, device=self.dev),
                "sel_o": torch.empty(max(1, k_select(self.ch_pct, S.n_q * d)), dtype=torch.int32, device=self.dev),
                "sel_ffn": torch.empty(max(1, k_select(self.ch_pct, S.hidden)), dtype=torch.int32, device=self.dev),
                "sel_down": torch.empty(max(1, k_select(self.ch_pct, S.ffn)), dtype=torch.int32, device=self.dev),
                # [batch][n_kv][k_sel] for the step's k_sel, packed (room for k_sel up to t_cap)
                "sel_tok": torch.empty(B * S.n_kv * max(1, self.t_cap), dtype=torch.int32, device=self.dev),
                "hit_tok": torch.empty(B * S.n_kv * max(1, self.t_cap), dtype=torch.int32, device=self.dev),
            })
        self.x_final = torch.empty((B, S.hidden), **i16)
        self.logits = torch.empty((B, S.vocab if self.head else 1), **f32)
        self.sel_lm = torch.empty(max(1, k_select(self.ch_pct, S.hidden)), dtype=torch.int32, device=self.dev)
        self.hits = {}  # (layer index or -1, op name) -> hit tensor [k_sel] of each GEMV op

    def workspace_bytes(self, T):
        L = binding.lib()
        S = self.spec
        best = L.sf_workspace_bytes_attn(self.batch, S.n_q, S.n_kv, T, k_select(self.tok_pct, T))
        for li in (0,):
            for names, k_in in ((("q", "k", "v"), S.hidden), (("o",), S.n_q * S.head_dim), (("gate", "up"), S.hidden),
                                (("down",), S.ffn)):
                arr = (binding.sf_gemv_op * len(names))()
                for i, n in enumerate(names):
                    arr[i] = binding.sf_gemv_op(self.layers[li][n].desc(), -1, None, None)
                best = max(best, L.sf_workspace_bytes_gemv(arr, len(names), self.batch, k_select(self.ch_pct, k_in)))
        if not self.head:
            return best
        arr = (binding.sf_gemv_op * 1)(binding.sf_gemv_op(self.lm_head.desc(), -1, None, None))
        return max(best, L.sf_workspace_bytes_gemv(arr, 1, self.batch, k_select(self.ch_pct, S.hidden)))

    # ---- one step ------------------------------------------------------------------------
    def build_step(self, pos, refined=True):
        """Prebuilt (function, args) list of the step that reads position ``pos`` (the
        new token's K/V land at ``pos``; attention covers ``pos + 1`` tokens)."""
        torch, S, B, d = self.torch, self.spec, self.batch, self.spec.head_dim
        if pos + 1 > self.t_cap:
            raise ValueError("the KV cache is full")
        Lb = binding.lib()
        P = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None
        cache = self.cache.handle if self.cache is not None else None
        ws = binding.workspace(self.workspace_bytes(pos + 1), self.dev)
        self._ws = ws
        keep = []
        calls = []

        ps = self.producer_select

        def ksel(k_in):
            return k_select(self.ch_pct, k_in) if refined and self.r > 0 else 0

        def gemv(names, layer, x, ys, k_in, sel, tag):
            """The selection is in `sel` already when its producer made it (sel_in);
            otherwise the GEMV computes it and writes it there (sel_out)."""
            ks = ksel(k_in)
            arr = (binding.sf_gemv_op * len(names))()
            for i, (n, y) in enumerate(zip(names, ys)):
                W = layer[n] if isinstance(n, str) else n
                pool = (layer.get("pool_" + n, -1) if isinstance(n, str) else self.pool_lm) if cache is not None else -1
                hit = torch.empty(max(1, ks), dtype=torch.int32, device=self.dev)
                self.hits[(layer.get("index", -1), n if isinstance(n, str) else "lm_head")] = hit
                keep.append(hit)
                arr[i] = binding.sf_gemv_op(W.desc(), pool, y.data_ptr(), hit.data_ptr())
            keep.append(arr)
            sel_in, sel_out = (P(sel), None) if (ps and ks > 0) else (None, P(sel))
            calls.append((Lb.sf_refined_gemv, [arr, len(names), P(x), B, ks, sel_in, sel_out, cache, ws.handle, None], tag))

        def norm(y, w, x, sel, k_in, tag):
            if ps:
                calls.append((Lb.sf_add_rmsnorm_select, [P(self.h), P(y), P(w), B, S.hidden, S.eps, P(x), ksel(k_in),
                                                         P(sel), None], tag))
            else:
                calls.append((Lb.sf_add_rmsnorm, [P(self.h), P(y), P(w), B, S.hidden, S.eps, P(x), None], tag))

        torch_ = self.torch
        pending = {}  # update -> late contribution waiting for it

        def lag(li, name, x, sel):
            """Side stream: the late contribution of this GEMV's missed channels; the
            returned call adds it to h on the compute stream once it is done."""
            L, bf = self.layers[li], self.buf[li]
            ev_in, ev_out = torch_.cuda.Event(), torch_.cuda.Event()
            dsc = L[name].desc()
            out = bf["lag_" + name]
            keep.extend([ev_in, ev_out, dsc])
            args = (cache, L["pool_" + name], C.byref(dsc), P(x), B, ksel(L[name].k_in), P(sel),
                    P(self.hits[(li, name)]), P(out), C.c_void_p(self.side.cuda_stream))

            def launch(stream):
                ev_in.record(stream)
                self.side.wait_event(ev_in)
                binding.check(Lb.sf_refine_lag_delta(*args))
                ev_out.record(self.side)

            def apply(stream):
                stream.wait_event(ev_out)
                binding.check(Lb.sf_residual_add(P(self.h), P(out), B * S.hidden, C.c_void_p(stream.cuda_stream)))

            calls.append((launch, None, "lag"))
            return apply

        def late_into(update):
            if update in pending:
                calls.append((pending.pop(update), None, "lag_add"))

        lag_on = self.fetch_lag and refined
        lead_on = self.fetch_lead and refined
        lead_wait = {}  # ("qkv" | "ffn-write", layer) -> call that makes the compute stream wait

        def lead(li):
            """Predict layer li + 1's channels from the residual stream entering layer li
            (side stream: the two norms' selections, then the prefetches) and register
            the waits: the compute stream's next write of h waits for the prediction,
            layer li + 1's q/k/v GEMV for the prefetches."""
            nx, bn = self.layers[li + 1], self.buf[li + 1]
            ks = ksel(S.hidden)
            ev_in, ev_pred, ev_done = torch_.cuda.Event(), torch_.cuda.Event(), torch_.cuda.Event()
            keep.extend([ev_in, ev_pred, ev_done])
            side = C.c_void_p(self.side.cuda_stream)
            preds = [(nx["attn_norm"], bn["x_pred_attn"], bn["sel_pred_attn"]),
                     (nx["ffn_norm"], bn["x_pred_ffn"], bn["sel_pred_ffn"])]
            fetch = [(nx["pool_" + n], bn["sel_pred_attn"] if n in ("q", "k", "v") else bn["sel_pred_ffn"])
                     for n in ("q", "k", "v", "gate", "up")]

            def launch(stream):
                ev_in.record(stream)
                self.side.wait_event(ev_in)
                for gain, xp, sp in preds:
                    binding.check(Lb.sf_add_rmsnorm_select(P(self.h), None, P(gain), B, S.hidden, S.eps, P(xp), ks,
                                                           P(sp), side))
                ev_pred.record(self.side)
                for pool, sp in fetch:
                    binding.check(Lb.sf_refine_cache_prefetch(cache, pool, P(sp), ks, side))
                ev_done.record(self.side)

            calls.append((launch, None, "lead"))
            lead_wait[("ffn-write", li)] = lambda stream: stream.wait_event(ev_pred)
            lead_wait[("qkv", li + 1)] = lambda stream: stream.wait_event(ev_done)
        if self.head:
            calls.append((Lb.sf_embed, [P(self.embed), S.vocab, S.hidden, P(self.ids), B, P(self.h), None], "embed"))
        for li, L in enumerate(self.layers):
            bf = self.buf[li]
            prev = self.buf[li - 1]["down"] if li > 0 else None
            late_into(("attn", li))
            norm(prev, L["attn_norm"], bf["x_attn"], bf["sel_attn"], S.hidden, "norm")
            if lead_on and li + 1 < len(self.layers):
                lead(li)
            if ("qkv", li) in lead_wait:
                calls.append((lead_wait.pop(("qkv", li)), None, "lead_wait"))
            gemv(("q", "k", "v"), L, bf["x_attn"], (bf["q"], bf["k"], bf["v"]), S.hidden, bf["sel_attn"], "qkv")
            calls.append((Lb.sf_qk_rope, [P(bf["q"]), P(bf["k"]), B, S.n_q, S.n_kv, P(L.get("q_norm")), P(L.get("k_norm")),
                                          S.eps, pos, S.theta, P(bf["q16"]), P(bf["k_rot"]), None], "rope"))
            kv = L["kv"]
            # the new token's refinement units: into the device copy, or straight into the
            # pinned host store the cache fills from (device-visible memory)
            if self._pool_frac is not None and self.kv_r > 0:
                dst = self._stores[L["pool_kv"]].data_ptr() + pos * kv.unit_bytes
            else:
                dst = kv.refine.data_ptr() + pos * kv.unit_bytes
            dsc = kv.desc(pos + 1)
            keep.append(dsc)
            kt = k_select(self.tok_pct, pos + 1) if refined and self.kv_r > 0 else 0
            pool_kv = L.get("pool_kv", -1) if cache is not None else -1
            # the append and the attention in one call (the attention's first pass
            # quantises the new token); without producer selection the attention also
            # writes the o projection's fp16 input
            calls.append((Lb.sf_refined_attn_decode_append,
                          [P(bf["q16"]), S.n_q, C.byref(dsc), P(bf["k_rot"]), P(bf["v"]), C.c_void_p(dst), kv.t_cap,
                           1.0 / math.sqrt(d), kt, None, cache, pool_kv, P(bf["attn"]), None if ps else P(bf["a16"]),
                           P(bf["sel_tok"]), P(bf["hit_tok"]), ws.handle, None], "attn"))
            if ps:
                calls.append((Lb.sf_to_f16_select, [P(bf["attn"]), B, S.n_q * d, P(bf["a16"]), ksel(S.n_q * d),
                                                    P(bf["sel_o"]), None], "cast"))
            gemv(("o",), L, bf["a16"], (bf["o"],), S.n_q * d, bf["sel_o"], "o")
            last = li == len(self.layers) - 1
            if lag_on and (not last or self.head):  # o's next update: the next layer's, or the final norm
                pending[("attn", li + 1)] = lag(li, "o", bf["a16"], bf["sel_o"])
            if ("ffn-write", li) in lead_wait:  # the prediction read h: its next write waits
                calls.append((lead_wait.pop(("ffn-write", li)), None, "lead_wait"))
            late_into(("ffn", li))
            norm(bf["o"], L["ffn_norm"], bf["x_ffn"], bf["sel_ffn"], S.hidden, "norm")
            gemv(("gate", "up"), L, bf["x_ffn"], (bf["gate"], bf["up"]), S.hidden, bf["sel_ffn"], "gateup")
            if ps:
                calls.append((Lb.sf_swiglu_select, [P(bf["gate"]), P(bf["up"]), B, S.ffn, P(bf["act"]), ksel(S.ffn),
                                                    P(bf["sel_down"]), None], "swiglu"))
            else:
                calls.append((Lb.sf_swiglu, [P(bf["gate"]), P(bf["up"]), B * S.ffn, P(bf["act"]), None], "swiglu"))
            gemv(("down",), L, bf["act"], (bf["down"],), S.ffn, bf["sel_down"], "down")
            if lag_on and not last:  # down's next update: the next layer's ffn residual add
                pending[("ffn", li + 1)] = lag(li, "down", bf["act"], bf["sel_down"])
        late_into(("attn", len(self.layers)))
        if self.head:
            norm(self.buf[-1]["down"], self.final_norm, self.x_final, self.sel_lm, S.hidden, "norm")
            gemv((self.lm_head,), {}, self.x_final, (self.logits,), S.hidden, self.sel_lm, "lm_head")
            calls.append((Lb.sf_argmax, [P(self.logits), B, S.vocab, P(self.next_ids), None], "argmax"))
        return calls, keep

    def enqueue(self, calls, stream, timer=None):
        """Launch the calls on `stream`; timer(tag) -> (start, end) events recorded
        around each call when given."""
        s = C.c_void_p(stream.cuda_stream)
        for fn, args, tag in calls:
            if args is None:  # stream-ordering step (events, side-stream work)
                fn(stream)
                continue
            a = list(args)
            a[-1] = s
            ev = timer(tag) if timer is not None else None
            if ev is not None:
                ev[0].record(stream)
            st = fn(*a)
            if ev is not None:
                ev[1].record(stream)
            if st != 0:
                binding.check(st)

    def step(self, ids, stream=None, refined=True):
        """One decode step at the current position: ids int [batch] -> next ids (device)."""
        torch = self.torch
        stream = stream or torch.cuda.current_stream()
        self.ids.copy_(torch.as_tensor(np.asarray(ids), dtype=torch.int32))
        calls, keep = self.build_step(self.pos, refined)
        self.enqueue(calls, stream)
        if self.cache is not None:
            binding.check(binding.lib().sf_refine_cache_fill(self.cache.handle, C.c_void_p(stream.cuda_stream),
                                                             C.c_void_p(self.side.cuda_stream), None))
        self._keep = keep
        self.pos += 1
        return self.next_ids
