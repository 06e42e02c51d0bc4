#!/usr/bin/env python3
"""Refined low-bit decode-step benchmark on one MI355X.

Default workload (llama8b-step): the GEMVs and attention of one decode step of a
Llama-3.1-8B-shaped model at batch 1, 32 layers, each:
  q/k/v refined GEMV (one fused launch, top 3% input channels refined),
  KV append (the new token quantised into the 2+2-bit cache) and refined GQA
  attention over the 32768-token context (32 query / 8 KV heads, head dim 128, top
  2% tokens refined) in one call,
  o refined GEMV, gate/up refined GEMV (one fused launch), down refined GEMV.
Every GEMV input is a seeded synthetic fp16 vector, N(0, 1) with 1% of channels
x20; W ~ N(0, 0.02); K and V ~ N(0, 1) with 4 dims of K x8; q ~ N(0, 1) (no trained
weights or datasets).  Weights and KV are 2-bit resident + 2-bit refinement, group
128.  Every refinement pool holds all of its units on the device, so every
selected unit hits.

Timing: the step is captured once as a HIP graph and replayed; inputs are resident
in HBM before the timed region.  Every call of the step is also timed on its own
with HIP events in eager passes over the same step (every layer's own matrices and
cache, so nothing is timed hot); the call with the largest share of the step gives
the roofline line.  The CPU baseline is the fp64 oracle on a bounded sample.

Other workloads (--workload): llama8b-layers runs whole decoder layers (RMSNorm,
RoPE, SwiGLU and casts between the GEMVs, each GEMV input produced by the layer);
qwen3-8b-decode and llama8b-128k-decode run full greedy decode steps with embedding
and lm_head, a Qwen3-8B-shaped model at context 8192 with 25% LRU pools or a
Llama-3.1-8B-shaped model at context 131072 with 3+1-bit weights and 10% pools with
asynchronous fills.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
HD = 128
# kernel sources of the attention call (its kernels and the headers they include)
ATTN_SOURCES = ("bit_decode_selective_amd/csrc/attention.hip", "bit_decode_selective_amd/csrc/group_quant.h",
                "bit_decode_selective_amd/csrc/sf_internal.h")
# HBM bytes per call of the dominant call of the default workload, from two rocprofv3
# --pmc runs (FETCH_SIZE, then WRITE_SIZE) scaled by the same counters on a plain copy
# of known size (--copy-calibration); reported only while the kernel sources have
# the hash they were measured on, and only for the call and workload (batch, context)
# they were measured for.
TRAFFIC = {
    # attn call (with the new token's append), T = 32768, 8 KV heads: split + select + pv,
    # medians over 32 calls each
    # (profiles/decode_step_llama8b_2bit_t32k_hbm_counters.md)
    "call": "attn",
    "workload": "llama8b-step",
    "batch": 1,
    "context": 32768,
    "sources_sha256": "1409320ba4786b1569199114f7d3b8b6eb576b7237270215564f0b370c3b8ae3",
    "fetch_bytes": 9655022 + 6832404 + 16914617,
    "write_bytes": 4691763 + 738406 + 1409024,
}
COPY_CALIBRATION_BYTES = 256 << 20


def k_select(percent, n):
    return (percent * n + 99) // 100


def sources_hash(files=ATTN_SOURCES):
    h = hashlib.sha256()
    for s in files:
        with open(os.path.join(ROOT, s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# ---- algorithmic bytes ----------------------------------------------------------------
def gemv_bytes(shapes, k_in, k_sel, b, r, batch):
    """One fused refined GEMV call: resident codes, scale/zero words, refinement bits
    of the applied (hit) channels, x, y, the selected indices."""
    tot = 0
    for n_out in shapes:
        tot += n_out * k_in * b // 8 + n_out * (k_in // 128) * 4 + k_sel * n_out * r // 8 + n_out * 4 * batch
    return tot + k_in * 2 * batch + k_sel * 4


def attn_bytes(T, k_sel, b, r, batch, n_q, n_kv):
    """One refined attention call: resident K and V codes with their scale/zero words,
    refinement units of the applied tokens, q, out, the selected indices."""
    per_th = 2 * (HD * b // 8 + 4)
    return batch * (n_kv * T * per_th + n_kv * k_sel * (2 * HD * r // 8) + n_q * HD * 2 + n_q * HD * 4
                    + n_kv * k_sel * 4)


def append_bytes(b, r, batch, n_kv):
    return batch * n_kv * (2 * HD * 4 + 2 * (HD * b // 8 + 4) + 2 * HD * r // 8)


def call_bytes(model, tag, T, refined):
    """Algorithmic bytes of one call with this tag in a step of `model` at context T."""
    S, B = model.spec, model.batch
    ks = (lambda n: k_select(model.ch_pct, n)) if refined and model.r > 0 else (lambda n: 0)
    kt = k_select(model.tok_pct, T) if refined and model.kv_r > 0 else 0
    H, QD = S.hidden, S.n_q * HD
    if tag == "qkv":
        return gemv_bytes([QD, S.n_kv * HD, S.n_kv * HD], H, ks(H), model.b, model.r, B)
    if tag == "o":
        return gemv_bytes([H], QD, ks(QD), model.b, model.r, B)
    if tag == "gateup":
        return gemv_bytes([S.ffn, S.ffn], H, ks(H), model.b, model.r, B)
    if tag == "down":
        return gemv_bytes([H], S.ffn, ks(S.ffn), model.b, model.r, B)
    if tag == "lm_head":
        return gemv_bytes([S.vocab], H, ks(H), model.b, model.r, B)
    if tag == "attn":  # with the new token's append (one call)
        return attn_bytes(T, kt, model.kv_b, model.kv_r, B, S.n_q, S.n_kv) + append_bytes(model.kv_b, model.kv_r, B,
                                                                                           S.n_kv)
    if tag == "append":
        return append_bytes(model.kv_b, model.kv_r, B, S.n_kv)
    if tag == "norm":  # h (+ y) read, h written, gains, x written, selection
        return B * H * (4 + 4 + 4 + 2) + H * 4 + ks(H) * 4
    if tag == "cast":
        return B * QD * (4 + 2) + ks(QD) * 4
    if tag == "swiglu":
        return B * S.ffn * (4 + 4 + 2) + ks(S.ffn) * 4
    if tag == "rope":
        return B * (S.n_q + S.n_kv) * HD * 4 + B * S.n_q * HD * 2 + B * S.n_kv * HD * 4
    if tag == "embed":
        return B * H * (2 + 4)
    if tag == "argmax":
        return B * S.vocab * 4 + B * 4
    return 0


def step_bytes(model, calls, T, refined):
    return sum(call_bytes(model, tag, T, refined) for _, _, tag in calls)


# ---- timing ----------------------------------------------------------------------------
class CallTimer:
    """HIP events around every call of a step, by tag."""

    def __init__(self, torch):
        self.torch, self.ev = torch, {}

    def __call__(self, tag):
        e = (self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True))
        self.ev.setdefault(tag, []).append(e)
        return e

    def us(self):
        return {t: [1000.0 * a.elapsed_time(b) for a, b in v] for t, v in self.ev.items()}


def capture(torch, model, calls, stream, before=None):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        if before is not None:
            before()
        model.enqueue(calls, stream)
    return g


def time_replays(torch, g, stream, steps, warmup, after=None):
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            g.replay()
            if after is not None:
                after()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(steps):
            g.replay()
            if after is not None:
                after()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_call(torch, model, calls, stream, passes, before=None):
    """Per-tag call durations (us) over `passes` eager passes of the step.  Each pass
    is queued behind a GPU sleep longer than the host needs to enqueue the whole
    pass, so the events around a call time its kernels, not the host's launches."""
    timer = CallTimer(torch)
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        if before is not None:
            before()
        model.enqueue(calls, stream)  # untimed: the host's enqueue time of one pass
        host_s = time.perf_counter() - t0
        torch.cuda.synchronize()
        for _ in range(passes):
            torch.cuda._sleep(int(max(host_s, 1e-3) * 4 * 2.4e9))
            if before is not None:
                before()
            model.enqueue(calls, stream, timer)
            torch.cuda.synchronize()
    return timer.us()


def call_table(model, calls, T, refined, us):
    """Per tag: launches per step, average us, bytes per call, GB/s, fraction of the
    HBM peak, and the tag's share of the step's summed call time."""
    count = {}
    for _, _, tag in calls:
        if tag in us:  # stream-ordering steps are not timed
            count[tag] = count.get(tag, 0) + 1
    total = sum(np.mean(us[t]) * count[t] for t in count)
    out = {}
    for t in count:
        a = float(np.mean(us[t]))
        by = call_bytes(model, t, T, refined)
        out[t] = {"per_step": count[t], "avg_us": a, "bytes": by, "gbps": by / (a * 1e3),
                  "frac": by / (a * 1e3) / HBM_PEAK_GBPS, "share": a * count[t] / total}
    return out


KERNELS = {  # the kernels one call of a tag launches (batch 1-2)
    "qkv": "gemv_split_kernel", "o": "gemv_split_kernel", "down": "gemv_split_kernel",
    "gateup": "gemv_split_kernel", "lm_head": "gemv_split_kernel",
    "attn": "attn_split_kernel (appending the new token) + attn_select_kernel + attn_pv_kernel",
    "norm": "produce_select_kernel<PROD_NORM>", "cast": "produce_select_kernel<PROD_CAST>",
    "swiglu": "produce_select_kernel<PROD_SWIGLU>", "rope": "qk_rope_kernel", "append": "kv_append_kernel",
}


def cpu_baseline(T, ch_pct, tok_pct, b, r, gemv_step_bytes, attn_step_bytes, batch, budget_s=8.0):
    """The fp64 oracle on a bounded sample: a 4096 x 4096 refined GEMV and refined
    attention over all 8 KV heads (32 query heads) at the full context, each repeated
    for about `budget_s` seconds (median per call); rates are scaled to the whole step
    by algorithmic bytes."""
    from bit_decode_selective_amd import inputs
    from oracle import attention as o_attn
    from oracle import gemv as o_gemv
    from oracle import nested, selection

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1

    def timed(fn):
        fn()
        times = []
        while len(times) < 3 or sum(times) < budget_s:
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
        times.sort()
        return times[len(times) // 2], len(times)

    H = 4096
    W = inputs.weight(2, 0, inputs.Q_PROJ, H, H)
    q = nested.quantize(W, b, r, 128)
    x = inputs.activation(2, 0, inputs.Q_PROJ, 0, batch, H)
    ks = selection.k_select(ch_pct, H)
    tg, ng = timed(lambda: o_gemv.refined_gemv(q, x, selection.select_channels(x, ks)))
    gb = gemv_bytes([H], H, ks, b, r, batch)
    K, V = inputs.kv(3, 0, 1, 8, T, HD)
    qh = inputs.query(3, 0, 0, 1, 32, HD)
    qk, qv = o_attn.quantize_kv(K, b, r), o_attn.quantize_kv(V, b, r)
    del K, V
    kt = selection.k_select(tok_pct, T)
    ta, na = timed(lambda: o_attn.refined_attention(qh, qk, qv, (1, 8, T, HD), 1 / math.sqrt(HD), kt))
    ab = attn_bytes(T, kt, b, r, 1, 32, 8)
    step_s = gemv_step_bytes / (gb / tg) + attn_step_bytes / (ab / ta)
    return {
        "value": batch / step_s,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle, median of {ng} calls of one {H}x{H} {b}+{r}-bit refined GEMV with top-{ks} "
                   f"channel selection ({tg:.3f} s each) and of {na} calls of refined attention, batch 1, 32 query / "
                   f"8 KV heads x {T} tokens, top-{kt} tokens ({ta:.3f} s each); scaled to the step's GEMV and "
                   f"attention bytes (GEMV {gb / tg / 1e6:.1f} MB/s, attention {ab / ta / 1e6:.1f} MB/s); host "
                   f"cpu_count={os.cpu_count()}"),
    }


# ---- workloads -------------------------------------------------------------------------
class SyntheticStep:
    """The default workload: 32 Llama-3.1-8B-shaped layers with synthetic GEMV inputs.

    Per layer, in launch order: the q/k/v GEMVs (one fused launch over one input),
    the new token's KV append and refined attention over the layer's own cache (one
    call), o, gate/up
    (one fused launch), down.  Every GEMV input is its own seeded fp16 vector of
    N(0, 1) with 1% of channels x20 (the GEMV configuration's activations), so each
    GEMV selects its own channels; q ~ N(0, 1); K and V ~ N(0, 1) with 4 dims of K x8.
    Every refinement pool holds all of its units on the device (every selected unit
    hits)."""

    def __init__(self, layers, T, batch, b=2, r=2, ch_pct=3, tok_pct=2, seed=1234):
        import torch

        from bit_decode_selective_amd import binding, decode, inputs

        self.torch, self.binding = torch, binding
        base = decode.LLAMA31_8B
        self.spec = decode.Spec(base.name, layers, base.hidden, base.n_q, base.n_kv, base.ffn, base.vocab,
                                base.qk_norm, base.theta, base.eps)
        S = self.spec
        self.layers, self.T, self.batch = layers, T, batch
        self.b, self.r, self.kv_b, self.kv_r, self.ch_pct, self.tok_pct = b, r, b, r, ch_pct, tok_pct
        dev = torch.device("cuda", 0)
        self.dev = dev
        g = torch.Generator(device=dev)
        H, QD, KD = S.hidden, S.n_q * HD, S.n_kv * HD
        pools, self.groups, self.kvs = [], [], []
        for li in range(layers):
            g.manual_seed(seed + li)
            mats = {}
            for name, (n, k) in (("q", (QD, H)), ("k", (KD, H)), ("v", (KD, H)), ("o", (H, QD)),
                                 ("gate", (S.ffn, H)), ("up", (S.ffn, H)), ("down", (H, S.ffn))):
                W = inputs.torch_weight(g, n, k, device=dev)
                mats[name] = binding.QuantWeight.from_device(W, b, r)
                del W
            grp = []
            for tag, names in (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gateup", ("gate", "up")),
                               ("down", ("down",))):
                ops = []
                for nm in names:
                    ops.append((mats[nm], len(pools)))
                    pools.append(mats[nm].resident_pool_desc())
                grp.append((tag, ops, mats[names[0]].k_in))
            self.groups.append(grp)
            kv = binding.QuantKV(batch, S.n_kv, T, b, r, device=dev)
            for t0 in range(0, T - 1, 8192):
                K, V = inputs.torch_kv(g, batch, S.n_kv, min(8192, T - 1 - t0), HD, device=dev)
                kv.append(K, V)
                del K, V
            self.kvs.append((kv, len(pools)))
            pools.append(kv.resident_pool_desc())
            torch.cuda.synchronize()
        self.cache = binding.RefineCache(pools, device=dev)
        self.x, self.y, self.q, self.knew, self.out = [], [], [], [], []
        for li in range(layers):
            g.manual_seed(seed + 1000 + li)
            xs, ys = [], []
            for tag, ops, k_in in self.groups[li]:
                outl = torch.randperm(k_in, generator=g, device=dev)[: (k_in + 99) // 100].cpu().numpy()
                xs.append(binding._f16_bits(inputs.torch_activation(g, batch, k_in, outl, device=dev), dev))
                ys.append([torch.empty((batch, w.n_out), dtype=torch.float32, device=dev) for w, _ in ops])
            self.x.append(xs)
            self.y.append(ys)
            self.q.append(binding._f16_bits(torch.randn((batch, S.n_q, HD), generator=g, device=dev).half(), dev))
            K, V = inputs.torch_kv(g, batch, S.n_kv, 1, HD, device=dev)
            self.knew.append((K.contiguous(), V.contiguous()))
            self.out.append(torch.empty((batch, S.n_q, HD), dtype=torch.float32, device=dev))
        L = binding.lib()
        wsb = [L.sf_workspace_bytes_attn(batch, S.n_q, S.n_kv, T, k_select(tok_pct, T))]
        for grp in self.groups:
            for tag, ops, k_in in grp:
                arr = (binding.sf_gemv_op * len(ops))(*[binding.sf_gemv_op(w.desc(), p, None, None) for w, p in ops])
                wsb.append(L.sf_workspace_bytes_gemv(arr, len(ops), batch, k_select(ch_pct, k_in)))
        self.ws = binding.workspace(max(wsb), dev)
        torch.cuda.synchronize()

    def build_step(self, refined=True):
        """(function, args, tag) of every launch of one step; `keep` holds the ctypes
        objects the argument tuples point into."""
        b, L, S, T = self.binding, self.binding.lib(), self.spec, self.T
        calls, keep = [], []
        for li in range(self.layers):
            kv, kv_pool = self.kvs[li]
            Kn, Vn = self.knew[li]
            dst = kv.refine.data_ptr() + (T - 1) * kv.unit_bytes
            for gi, (tag, ops, k_in) in enumerate(self.groups[li]):
                ks = k_select(self.ch_pct, k_in) if refined else 0
                arr = (b.sf_gemv_op * len(ops))(*[b.sf_gemv_op(w.desc(), p, self.y[li][gi][i].data_ptr(), None)
                                                   for i, (w, p) in enumerate(ops)])
                keep.append(arr)
                calls.append((L.sf_refined_gemv, (arr, len(ops), C.c_void_p(self.x[li][gi].data_ptr()), self.batch,
                                                  ks, None, None, self.cache.handle, self.ws.handle, None), tag))
                if tag == "qkv":
                    dsc = kv.desc(T)
                    keep.append(dsc)
                    kt = k_select(self.tok_pct, T) if refined else 0
                    # the new token's KV append and the attention in one call
                    calls.append((L.sf_refined_attn_decode_append,
                                  (C.c_void_p(self.q[li].data_ptr()), S.n_q, C.byref(dsc), C.c_void_p(Kn.data_ptr()),
                                   C.c_void_p(Vn.data_ptr()), C.c_void_p(dst), kv.t_cap, 1.0 / math.sqrt(HD), kt,
                                   None, self.cache.handle, kv_pool, C.c_void_p(self.out[li].data_ptr()), None, None,
                                   None, self.ws.handle, None), "attn"))
        return calls, keep

    def enqueue(self, calls, stream, timer=None):
        s = C.c_void_p(stream.cuda_stream)
        for fn, args, tag in calls:
            a = list(args)
            a[-1] = s
            ev = timer(tag) if timer is not None else None
            if ev is not None:
                ev[0].record(stream)
            st = fn(*a)
            if ev is not None:
                ev[1].record(stream)
            if st != 0:
                self.binding.check(st)


def copy_calibration():
    """A plain device copy of known size (256 MiB read + 256 MiB written): its HBM
    counters scale those of the other kernels."""
    import torch

    src_t = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
    dst_t = torch.empty_like(src_t)
    for _ in range(3):
        torch.neg(src_t, out=dst_t)
    torch.cuda.synchronize()
    print(f"# copy calibration: 3 x torch.neg over {COPY_CALIBRATION_BYTES} bytes", file=sys.stderr, flush=True)


def measure(torch, model, calls, calls0, stream, args, before=None):
    """Graph-replayed step times (refined, unrefined) and per-call eager timings."""
    from bit_decode_selective_amd import binding

    with torch.cuda.stream(stream):  # first launches outside capture
        for c in (calls, calls0):
            if before is not None:
                before()
            model.enqueue(c, stream)
    torch.cuda.synchronize()
    graph = capture(torch, model, calls, stream, before)
    ms = time_replays(torch, graph, stream, args.steps, args.warmup)
    print(f"# refined step {ms:.3f} ms", file=sys.stderr, flush=True)
    ws = binding.workspace(0, model.dev)
    ws.check()  # raises if a bounded device wait gave up during the timed steps
    unref_ms = None
    if not args.no_unrefined:
        graph0 = capture(torch, model, calls0, stream, before)
        unref_ms = time_replays(torch, graph0, stream, args.steps, args.warmup)
        print(f"# unrefined step {unref_ms:.3f} ms", file=sys.stderr, flush=True)
    us = per_call(torch, model, calls, stream, 3, before)
    ws.check()
    return ms, unref_ms, us


def report(model, calls, T, B, args, ms, unref_ms, us, workload, extra_config):
    table = call_table(model, calls, T, True, us)
    dom = max(table, key=lambda t: table[t]["avg_us"] * table[t]["per_step"])
    sb = step_bytes(model, calls, T, True)
    gbps = sb / (ms * 1e-3) / 1e9
    traffic = None
    if (TRAFFIC is not None and TRAFFIC.get("call") == dom and TRAFFIC.get("workload") == args.workload
            and TRAFFIC.get("batch") == B and TRAFFIC.get("context") == T
            and TRAFFIC.get("sources_sha256") == sources_hash()):
        traffic = TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]
    res = {
        "metric": "refined decode tokens/s + achieved HBM GB/s (% peak), Llama-8B-shape 2-bit",
        "value": B / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 x int2 -> fp32",
        "data": "synthetic (seeded random weights, KV and activations of the model shapes; no trained weights)",
        "config": dict({"workload": workload, "layers": args.layers, "batch": B, "context": T,
                        "weight_bits": "2+2", "kv_bits": "2+2", "refine_channels_pct": 3, "refine_tokens_pct": 2,
                        "refinement_pools": "all units resident on the device", "hip_graph": True}, **extra_config),
        "hbm_gbps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "step_algorithmic_bytes": sb,
        "roofline": {
            "bound": "hbm",
            "kernel": f"{dom} call: {KERNELS.get(dom, dom)}",
            "achieved": table[dom]["gbps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": table[dom]["frac"],
            "traffic": traffic,
            "launch_us": table[dom]["avg_us"],
            "bytes_per_launch": table[dom]["bytes"],
        },
        "calls": {t: {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()} for t, d in table.items()},
    }
    if unref_ms is not None:
        res["unrefined_tokens_per_s"] = B / (unref_ms * 1e-3)
        res["refined_over_unrefined"] = unref_ms / ms
    if not args.no_cpu_baseline:
        gsb = sum(call_bytes(model, t, T, True) for _, _, t in calls if t in ("qkv", "o", "gateup", "down"))
        asb = sum(call_bytes(model, t, T, True) for _, _, t in calls if t == "attn")
        res["cpu_baseline"] = cpu_baseline(T, 3, 2, 2, 2, gsb, asb, B)
    print(json.dumps(res), flush=True)


def synthetic_step(args):
    """The default workload (see SyntheticStep)."""
    import torch

    if args.copy_calibration:
        copy_calibration()
    T, B = args.context, args.batch
    t0 = time.time()
    model = SyntheticStep(args.layers, T, B)
    print(f"# setup {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    stream = torch.cuda.Stream()
    calls, keep = model.build_step(refined=True)
    calls0, keep0 = model.build_step(refined=False)
    torch.cuda.synchronize()
    ms, unref_ms, us = measure(torch, model, calls, calls0, stream, args)
    workload = (f"Llama-3.1-8B-shape refined decode step, batch {B}: {args.layers} layers x (q/k/v GEMV, "
                f"KV append + GQA attention 32q/8kv d128 T={T} in one call, o GEMV, gate/up GEMV, down GEMV) with synthetic GEMV inputs "
                f"(N(0,1), 1% of channels x20) and queries; weights and KV 2+2-bit, top 3% channels / 2% tokens "
                f"refined")
    report(model, calls, T, B, args, ms, unref_ms, us, workload, {"channel_selection": "in each GEMV launch"})


def layer_chain(args):
    """Whole decoder layers of a Llama-3.1-8B-shaped model, each GEMV input produced
    by the layer before it (RMSNorm, RoPE, SwiGLU and casts included)."""
    import torch

    from bit_decode_selective_amd import decode

    if args.copy_calibration:
        copy_calibration()
    T, B = args.context, args.batch
    base = decode.LLAMA31_8B
    spec = decode.Spec(base.name, args.layers, base.hidden, base.n_q, base.n_kv, base.ffn, base.vocab, base.qk_norm,
                       base.theta, base.eps)
    t0 = time.time()
    src = decode.DeviceWeights(1234, "cuda")
    model = decode.DecodeModel(spec, B, T, src, b=2, r=2, kv_b=2, kv_r=2, ch_pct=3, tok_pct=2, pool_frac=None,
                               head=False, producer_select=args.producer_select)
    model.fill_kv(T - 1, src)
    pos = T - 1
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    h0 = torch.randn((B, spec.hidden), generator=g, device="cuda", dtype=torch.float32)
    print(f"# setup {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    stream = torch.cuda.Stream()
    reset = lambda: model.h.copy_(h0)  # the step's input state (in place of the embedding)
    calls, keep = model.build_step(pos, refined=True)
    calls0, keep0 = model.build_step(pos, refined=False)
    torch.cuda.synchronize()
    ms, unref_ms, us = measure(torch, model, calls, calls0, stream, args, reset)
    sel = "by the kernel that produces each GEMV input" if args.producer_select else "in each GEMV launch"
    workload = (f"Llama-3.1-8B-shape refined decoder layers, batch {B}: {args.layers} layers x (RMSNorm, q/k/v GEMV, "
                f"RoPE, KV append + GQA attention 32q/8kv d128 T={T} in one call, fp16 cast, o GEMV, RMSNorm, gate/up GEMV, "
                f"SwiGLU, down GEMV) from a synthetic residual state; weights and KV 2+2-bit, top 3% channels / 2% "
                f"tokens refined")
    report(model, calls, T, B, args, ms, unref_ms, us, workload, {"channel_selection": sel})


def variants_workload(args):
    """The pages' comparison variants beside nested refinement, per call, each over
    distinct matrices / layer caches (more bytes than the 256 MB last-level cache):
    a 4096 -> 14336 2+2-bit GEMV refined on 123 channels (3%) -- nested refinement,
    random selection, FP16 fetch of the columns -- and attention over 32768 tokens,
    32 query / 8 KV heads, 656 tokens per KV head (2%) -- nested refinement, random
    selection, SpeCache-style FP16 tokens, sparse attention over the selected
    tokens.  Every unit is resident on the device; each variant's calls are captured
    in a HIP graph and replayed."""
    import torch

    from bit_decode_selective_amd import binding, inputs

    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    n_mat, n_kv_layers, T, H, F = 24, 16, args.context, 4096, 14336
    ks_c, ks_t = k_select(3, H), k_select(2, T)
    mats = []
    for i in range(n_mat):
        W = inputs.torch_weight(g, F, H, device=dev)
        qw = binding.QuantWeight.from_device(W, 2, 2)
        u16 = W.t().contiguous().half().view(torch.uint8).reshape(H, -1)
        del W
        mats.append((qw, binding.RefineCache([qw.resident_pool_desc()]), binding.RefineCache([binding.device_pool_desc(u16)]),
                     u16))
    x = binding._f16_bits(inputs.torch_activation(g, 1, H, torch.randperm(H, generator=g, device=dev)[:41].cpu().numpy(),
                                                  device=dev), dev)
    rsel = torch.as_tensor(inputs.random_selection(77, 0, 0, 0, H, ks_c), device=dev)
    layers = []
    for i in range(n_kv_layers):
        K, V = inputs.torch_kv(g, 1, 8, T, HD, device=dev)
        kv = binding.QuantKV.from_host(K, V, 2, 2)
        u16 = torch.cat([K, V], dim=-1).half().view(torch.uint8).reshape(-1, 4 * HD)
        del K, V
        layers.append((kv, binding.RefineCache([kv.resident_pool_desc()]), binding.RefineCache([binding.device_pool_desc(u16)]),
                       u16))
    q = binding._f16_bits(torch.randn((1, 32, HD), generator=g, device=dev).half(), dev)
    tsel = torch.as_tensor(inputs.random_token_selection(77, 0, 0, 1, 8, T, ks_t), device=dev)
    sc = 1.0 / math.sqrt(HD)
    V_ = binding
    cases = {
        "gemv_nested": lambda: [V_.refined_gemv([(m[0], 0)], x, ks_c, cache=m[1], want_hits=False) for m in mats],
        "gemv_random_selection": lambda: [V_.refined_gemv([(m[0], 0)], x, ks_c, cache=m[1], sel_in=rsel, want_hits=False)
                                          for m in mats],
        "gemv_fp16_fetch": lambda: [V_.fp16_fetch_gemv(m[0], x, ks_c, m[2], 0) for m in mats],
        "attn_nested": lambda: [V_.refined_attention(q, L[0], sc, ks_t, cache=L[1]) for L in layers],
        "attn_random_selection": lambda: [V_.refined_attention(q, L[0], sc, ks_t, cache=L[1], sel_in=tsel) for L in layers],
        "attn_fp16_tokens": lambda: [V_.refined_attention(q, L[0], sc, ks_t, cache=L[2], variant=V_.SF_ATTN_FP16_TOKENS)
                                     for L in layers],
        "attn_sparse": lambda: [V_.refined_attention(q, L[0], sc, ks_t, cache=L[1], variant=V_.SF_ATTN_DROP_UNSELECTED)
                                for L in layers],
    }
    unit = {"gemv_nested": F * 2 // 8, "gemv_random_selection": F * 2 // 8, "gemv_fp16_fetch": F * 2,
            "attn_nested": 2 * HD * 2 // 8, "attn_random_selection": 2 * HD * 2 // 8, "attn_fp16_tokens": 4 * HD,
            "attn_sparse": 2 * HD * 2 // 8}
    stream = torch.cuda.Stream()
    res = {}
    for name, fn in cases.items():
        with torch.cuda.stream(stream):
            keep = fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            keep = fn()
        n_calls = n_mat if name.startswith("gemv") else n_kv_layers
        ms = time_replays(torch, graph, stream, args.steps, args.warmup)
        per = ms * 1e3 / n_calls
        sel_units = ks_c if name.startswith("gemv") else 8 * ks_t
        res[name] = {"us_per_call": round(per, 2), "selected_units": sel_units, "unit_bytes": unit[name],
                     "selected_bytes": sel_units * unit[name]}
        print(f"# {name}: {per:.2f} us per call", file=sys.stderr, flush=True)
        del graph, keep
    binding.workspace(0, dev).check()
    print(json.dumps({"workload": "comparison variants (per call, every unit resident)", "context": T,
                      "gemv": f"{H} -> {F}, 2+2-bit, {ks_c} channels", "attention": f"32q/8kv d128, {ks_t} tokens per "
                      "KV head", "variants": res}), flush=True)


def decode_workload(args):
    """Full greedy decode steps (embedding .. argmax) of a Qwen3-8B-shaped model at
    context 8192 with pools holding 25% of every tensor's refinement units (LRU,
    deterministic fills), or a Llama-3.1-8B-shaped model at context 131072 with
    3+1-bit weights, 2+2-bit KV and pools of 10% (asynchronous fills).  Each step is
    one graph replay at a fixed position with new token ids, then the cache fill."""
    import torch

    from bit_decode_selective_amd import binding, decode

    if args.workload == "qwen3-8b-decode":
        spec, T, (wb, wr), frac, mode = decode.QWEN3_8B, args.context or 8192, (2, 2), 0.25, binding.SF_CACHE_DETERMINISTIC
    else:
        spec, T, (wb, wr), frac, mode = decode.LLAMA31_8B, args.context or 131072, (3, 1), 0.10, binding.SF_CACHE_ASYNC
    kvb, kvr, ch_pct, tok_pct = 2, 2, 3, 2
    layers = args.layers if args.layers else spec.layers
    spec = decode.Spec(spec.name, layers, spec.hidden, spec.n_q, spec.n_kv, spec.ffn, spec.vocab, spec.qk_norm,
                       spec.theta, spec.eps)
    t0 = time.time()
    src = decode.DeviceWeights(4321, "cuda")
    store_dir = None
    if args.store == "ssd":
        import tempfile

        store_dir = tempfile.mkdtemp(prefix="sf_refine_store_")
    model = decode.DecodeModel(spec, args.batch, T + 1, src, b=wb, r=wr, kv_b=kvb, kv_r=kvr, ch_pct=ch_pct,
                               tok_pct=tok_pct, pool_frac=frac, cache_mode=mode, store_dir=store_dir,
                               fetch_lag=args.fetch_lag, fetch_lead=args.fetch_lead,
                               producer_select=args.producer_select)
    model.fill_kv(T, src)
    print(f"# setup {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    calls, keep = model.build_step(T)
    stream = torch.cuda.Stream(device=model.dev)
    rng = np.random.default_rng(99)

    def fill():
        binding.check(binding.lib().sf_refine_cache_fill(model.cache.handle, C.c_void_p(stream.cuda_stream),
                                                         C.c_void_p(model.side.cuda_stream), None))

    # token ids of every step staged on the device up front: a step's copy is device to
    # device and never waits for the step in flight (a pageable host copy would)
    n_ids = 2 + args.warmup + 2 * args.steps
    ids_all = torch.as_tensor(rng.integers(0, spec.vocab, size=(n_ids, args.batch)), dtype=torch.int32).to(model.dev)
    ids_next = [0]

    def new_ids():
        model.ids.copy_(ids_all[ids_next[0] % n_ids], non_blocking=True)
        ids_next[0] += 1

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        new_ids()
        model.enqueue(calls, stream)
        fill()
    torch.cuda.synchronize()
    g = capture(torch, model, calls, stream)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            new_ids()
            g.replay()
            fill()
    torch.cuda.synchronize()
    st0 = model.cache.stats()
    ms = time_replays(torch, g, stream, args.steps, 0, after=lambda: (new_ids(), fill()))
    st1 = model.cache.stats()
    ms_kernels = time_replays(torch, g, stream, args.steps, 0)
    binding.workspace(0, model.dev).check()
    d = {k: st1[k] - st0[k] for k in st1}
    io = model.cache.io_stats()
    sb = step_bytes(model, calls, T + 1, True)
    secs = ms * 1e-3
    res = {
        "metric": "refined decode tokens/s, full decode step (glue, lm_head, argmax, cache fills)",
        "value": args.batch / secs,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"fp16 x int{wb} -> fp32",
        "data": "synthetic (random-init weights of the model shape, synthetic KV prefix, random token ids)",
        "config": {
            "workload": (f"{spec.name}-shape greedy decode, batch {args.batch}, context {T}, {layers} layers, "
                         f"weights {wb}+{wr}-bit, KV {kvb}+{kvr}-bit, top {ch_pct}% channels / {tok_pct}% tokens, "
                         f"pools {int(frac * 100)}% of each tensor's refinement units, "
                         f"{'deterministic' if mode == binding.SF_CACHE_DETERMINISTIC else 'async'} fills"),
            "batch": args.batch,
            "context": T,
            "layers": layers,
            "hip_graph": True,
        },
        "hbm_gbps": sb / secs / 1e9,
        "hbm_frac": sb / secs / 1e9 / HBM_PEAK_GBPS,
        "step_algorithmic_bytes": sb,
        "ms_per_step_kernels_only": ms_kernels,
        "refinement_hit_rate": d["hits"] / max(1, d["lookups"]),
        "fill_bytes_per_step": d["h2d_bytes"] / args.steps,
        "units_installed_per_step": d["installed"] / args.steps,
    }
    if store_dir is not None:
        res["config"]["weight_refinement_store"] = "files (SSD tier), one per weight pool; KV units in pinned RAM"
        res["ssd_reads"] = io
        import shutil

        shutil.rmtree(store_dir, ignore_errors=True)
    else:
        res["config"]["weight_refinement_store"] = "pinned host RAM"
    res["config"]["channel_selection"] = ("by the kernel that produces each GEMV input" if model.producer_select
                                          else "in each GEMV launch")
    res["config"]["fetch_lag"] = bool(model.fetch_lag)
    res["config"]["fetch_lead"] = bool(model.fetch_lead)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--context", type=int, default=32768)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unrefined", action="store_true")
    ap.add_argument("--workload", default="llama8b-step",
                    choices=["llama8b-step", "llama8b-layers", "qwen3-8b-decode", "llama8b-128k-decode", "variants"],
                    help="llama8b-step (default): the GEMVs and attention of a Llama-3.1-8B-shaped step with "
                         "synthetic inputs; llama8b-layers: whole decoder layers chained through RMSNorm, RoPE and "
                         "SwiGLU; the others run full decode steps with embedding, lm_head and LRU refinement pools")
    ap.add_argument("--store", default="ram", choices=["ram", "ssd"],
                    help="decode workloads: weight refinement stores in pinned host RAM or in files (SSD tier)")
    ap.add_argument("--fetch-lead", action="store_true",
                    help="decode workloads: each layer predicts the next layer's q/k/v and gate/up channels from its "
                         "residual stream and prefetches them on the side stream")
    ap.add_argument("--fetch-lag", action="store_true",
                    help="decode workloads: missed o / down refinements are fetched on the side stream and added at "
                         "the residual stream's next update")
    ap.add_argument("--producer-select", action="store_true",
                    help="the kernels that form each GEMV input also select its channels (else each GEMV selects)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain device copy (256 MiB read + 256 MiB written) whose HBM counters scale "
                         "those of the other kernels")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the refined decode path runs on "
              "a single device; DESIGN.md describes how it would shard)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "llama8b-step":
        synthetic_step(args)
        return
    if args.workload == "llama8b-layers":
        layer_chain(args)
        return
    if args.workload == "variants":
        variants_workload(args)
        return
    if args.layers == 32:
        args.layers = 0  # the model's own depth
    if args.context == 32768:
        args.context = 0  # the workload's own context
    decode_workload(args)


if __name__ == "__main__":
    main()
