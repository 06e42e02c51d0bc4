"""ctypes binding of libstrataflux.so (C ABI in include/strataflux.h).

Argument marshalling only: every step of the decode path runs in the library's HIP
kernels.  PyTorch provides device memory, pinned host memory and streams.  If the
library has not been built, ``lib()`` raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstrataflux.so")
_lib = None
_lock = threading.Lock()

SF_REFINE_CHANNEL_MAJOR = 0
SF_REFINE_ROW_MAJOR = 1
SF_CACHE_DETERMINISTIC = 0
SF_CACHE_ASYNC = 1


class SFError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"strataflux status {status}: {msg}")
        self.status = status


class sf_qfmt(C.Structure):
    _fields_ = [("b", C.c_int32), ("r", C.c_int32), ("group", C.c_int32)]


class sf_qweight(C.Structure):
    _fields_ = [
        ("resident", C.c_void_p),
        ("sz", C.c_void_p),
        ("n_out", C.c_int64),
        ("k_in", C.c_int64),
        ("fmt", sf_qfmt),
    ]


class sf_qkv(C.Structure):
    _fields_ = [
        ("k_res", C.c_void_p),
        ("k_sz", C.c_void_p),
        ("v_res", C.c_void_p),
        ("v_sz", C.c_void_p),
        ("batch", C.c_int32),
        ("n_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("t_len", C.c_int32),
        ("t_cap", C.c_int32),
        ("fmt", sf_qfmt),
    ]


class sf_pool_desc(C.Structure):
    _fields_ = [
        ("unit_bytes", C.c_int64),
        ("n_units", C.c_int64),
        ("capacity", C.c_int64),
        ("host_store", C.c_void_p),
        ("device_store", C.c_void_p),
        ("max_lookup", C.c_int32),
        ("store_file", C.c_char_p),
        ("store_offset", C.c_int64),
        ("lead_slots", C.c_int32),
    ]


class sf_gemv_op(C.Structure):
    _fields_ = [
        ("w", sf_qweight),
        ("pool", C.c_int32),
        ("y", C.c_void_p),
        ("hit_out", C.c_void_p),
    ]


VP, I32, I64, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
_PROTOS = {
    "sf_abi_version": (I32, []),
    "sf_status_string": (C.c_char_p, [I32]),
    "sf_last_error": (C.c_char_p, []),
    "sf_workspace_create": (I32, [SZ, C.POINTER(VP)]),
    "sf_workspace_destroy": (I32, [VP]),
    "sf_workspace_bytes_gemv": (SZ, [C.POINTER(sf_gemv_op), I32, I32, I32]),
    "sf_workspace_bytes_attn": (SZ, [I32, I32, I32, I32, I32]),
    "sf_workspace_check": (I32, [VP]),
    "sf_workspace_set_spin_limit": (I32, [VP, C.c_uint32]),
    "sf_quantize_nested": (I32, [VP, I64, I64, sf_qfmt, I32, VP, VP, VP, VP]),
    "sf_debug_dequantize": (I32, [VP, VP, VP, I64, I64, sf_qfmt, I32, I32, VP, VP]),
    "sf_kv_append": (I32, [VP, VP, I32, I32, C.POINTER(sf_qkv), VP, I64, VP]),
    "sf_refine_cache_create": (I32, [C.POINTER(sf_pool_desc), I32, I32, I32, C.POINTER(VP)]),
    "sf_refine_cache_destroy": (I32, [VP]),
    "sf_refine_cache_lookup": (I32, [VP, I32, VP, I32, VP, VP]),
    "sf_refine_cache_fill": (I32, [VP, VP, VP, C.POINTER(I64)]),
    "sf_refine_cache_stats": (I32, [VP, I32, C.POINTER(I64), C.POINTER(I64), C.POINTER(I64), C.POINTER(I64)]),
    "sf_refine_cache_resident": (I32, [VP, I32, C.POINTER(I64), C.POINTER(I64)]),
    "sf_refine_cache_prefetch": (I32, [VP, I32, VP, I32, VP]),
    "sf_refine_cache_io_stats": (I32, [VP, I32, C.POINTER(I64), C.POINTER(I64), C.POINTER(C.c_double),
                                       C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    "sf_refined_gemv": (I32, [C.POINTER(sf_gemv_op), I32, VP, I32, I32, VP, VP, VP, VP, VP]),
    "sf_refined_gemv_noalloc": (I32, [C.POINTER(sf_gemv_op), I32, VP, I32, I32, VP, VP, VP, VP]),
    "sf_refined_attn_decode": (I32, [VP, I32, C.POINTER(sf_qkv), C.c_float, I32, VP, VP, I32, VP, VP, VP, VP, VP]),
    "sf_refined_attn_decode_append": (I32, [VP, I32, C.POINTER(sf_qkv), VP, VP, VP, I64, C.c_float, I32, VP, VP, I32,
                                            VP, VP, VP, VP, VP, VP]),
    "sf_attn_decode_variant": (I32, [VP, I32, C.POINTER(sf_qkv), C.c_float, I32, VP, VP, I32, VP, VP, VP, VP, VP,
                                     I32]),
    "sf_fp16_fetch_delta": (I32, [VP, I32, C.POINTER(sf_qweight), VP, I32, I32, VP, VP, VP, VP]),
    "sf_embed": (I32, [VP, I64, I32, VP, I32, VP, VP]),
    "sf_add_rmsnorm": (I32, [VP, VP, VP, I32, I32, C.c_float, VP, VP]),
    "sf_qk_rope": (I32, [VP, VP, I32, I32, I32, VP, VP, C.c_float, I32, C.c_float, VP, VP, VP]),
    "sf_swiglu": (I32, [VP, VP, I64, VP, VP]),
    "sf_add_rmsnorm_select": (I32, [VP, VP, VP, I32, I32, C.c_float, VP, I32, VP, VP]),
    "sf_swiglu_select": (I32, [VP, VP, I32, I32, VP, I32, VP, VP]),
    "sf_to_f16_select": (I32, [VP, I32, I32, VP, I32, VP, VP]),
    "sf_to_f16": (I32, [VP, I64, VP, VP]),
    "sf_residual_add": (I32, [VP, VP, I64, VP]),
    "sf_refine_lag_delta": (I32, [VP, I32, C.POINTER(sf_qweight), VP, I32, I32, VP, VP, VP, VP]),
    "sf_argmax": (I32, [VP, I32, I64, VP, VP]),
}
EXPORTS = tuple(_PROTOS)


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python __graft_entry__.py` "
                    "(there is no CPU fallback)"
                )
            L = C.CDLL(LIB_PATH)
            for name, (res, args) in _PROTOS.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
        return _lib


def reload():
    global _lib
    with _lock:
        _lib = None
    return lib()


def check(status):
    if status != 0:
        L = lib()
        raise SFError(status, f"{L.sf_status_string(status).decode()}: {L.sf_last_error().decode()}")


def _torch():
    import torch

    return torch


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


def _dev_tensor(a, dtype, device):
    torch = _torch()
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=dtype).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


def _f16_bits(a, device):
    """fp16 values (numpy or torch) -> device int16 tensor holding the bit patterns."""
    torch = _torch()
    t = _dev_tensor(a, torch.float16, device)
    return t.view(torch.int16)


# ---- workspace ------------------------------------------------------------------
class Workspace:
    def __init__(self, nbytes):
        h = C.c_void_p()
        check(lib().sf_workspace_create(int(nbytes), C.byref(h)))
        self.handle = h
        self.nbytes = int(nbytes)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.sf_workspace_destroy(self.handle)
            self.handle = None

    def check(self):
        check(lib().sf_workspace_check(self.handle))

    def set_spin_limit(self, polls):
        check(lib().sf_workspace_set_spin_limit(self.handle, int(polls)))


_ws = {}


def check_workspaces():
    """sf_workspace_check on every workspace this module created (raises SFError with
    SF_ESTATE if a device-side wait timed out since the last check)."""
    for w in list(_ws.values()):
        w.check()


def workspace(nbytes, device=None):
    """A per-device workspace at least ``nbytes`` large (grown on demand)."""
    torch = _torch()
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    w = _ws.get(dev.index)
    if w is None or w.nbytes < nbytes:
        torch.cuda.synchronize(dev)
        with torch.cuda.device(dev):
            w = Workspace(max(nbytes, 1 << 20))
        _ws[dev.index] = w
    return w


# ---- nested weights ---------------------------------------------------------------
class QuantWeight:
    """A nested-quantised weight [n_out][k_in] on the device."""

    def __init__(self, resident, sz, refine, n_out, k_in, b, r):
        self.resident, self.sz, self.refine = resident, sz, refine
        self.n_out, self.k_in, self.b, self.r = n_out, k_in, b, r

    @classmethod
    def from_device(cls, W, b, r, stream=None):
        torch = _torch()
        W = W.contiguous().to(torch.float32)
        n, k = W.shape
        dev = W.device
        res = torch.empty((n, k * b // 8), dtype=torch.uint8, device=dev)
        sz = torch.empty((n, k // 128), dtype=torch.int32, device=dev)
        ref = torch.empty((k, n * r // 8), dtype=torch.uint8, device=dev) if r > 0 else None
        check(
            lib().sf_quantize_nested(
                _ptr(W), n, k, sf_qfmt(b, r, 128), SF_REFINE_CHANNEL_MAJOR, _ptr(res), _ptr(sz), _ptr(ref),
                _stream(stream),
            )
        )
        return cls(res, sz, ref, n, k, b, r)

    @classmethod
    def from_host(cls, W, b, r, device="cuda"):
        return cls.from_device(_dev_tensor(W, _torch().float32, device), b, r)

    def desc(self):
        return sf_qweight(self.resident.data_ptr(), self.sz.data_ptr(), self.n_out, self.k_in, sf_qfmt(self.b, self.r, 128))

    @property
    def unit_bytes(self):
        return self.n_out * self.r // 8

    def resident_pool_desc(self, max_lookup=0):
        """A pool holding every refinement unit of this matrix on the device."""
        return sf_pool_desc(self.unit_bytes, self.k_in, self.k_in, None, self.refine.data_ptr(), max_lookup)

    def host_store(self):
        """Pinned host copy of the refinement units [k_in][unit_bytes]."""
        return self.refine.to("cpu").pin_memory()

    def dequantize(self, which, stream=None):
        torch = _torch()
        out = torch.empty((self.n_out, self.k_in), dtype=torch.float32, device=self.resident.device)
        check(
            lib().sf_debug_dequantize(
                _ptr(self.resident), _ptr(self.sz), _ptr(self.refine), self.n_out, self.k_in,
                sf_qfmt(self.b, self.r, 128), SF_REFINE_CHANNEL_MAJOR, which, _ptr(out), _stream(stream),
            )
        )
        return out


def quantize_rows(X, b, r, device="cuda", stream=None):
    """Row-major nested quantisation of X [rows][cols]: (resident, sz, refine) device tensors."""
    torch = _torch()
    X = _dev_tensor(X, torch.float32, device)
    n, k = X.shape
    res = torch.empty((n, k * b // 8), dtype=torch.uint8, device=X.device)
    sz = torch.empty((n, k // 128), dtype=torch.int32, device=X.device)
    ref = torch.empty((n, k * r // 8), dtype=torch.uint8, device=X.device) if r > 0 else None
    check(
        lib().sf_quantize_nested(
            _ptr(X), n, k, sf_qfmt(b, r, 128), SF_REFINE_ROW_MAJOR, _ptr(res), _ptr(sz), _ptr(ref), _stream(stream)
        )
    )
    return res, sz, ref


def dequantize_rows(res, sz, ref, rows, cols, b, r, which, stream=None):
    torch = _torch()
    out = torch.empty((rows, cols), dtype=torch.float32, device=res.device)
    check(
        lib().sf_debug_dequantize(
            _ptr(res), _ptr(sz), _ptr(ref), rows, cols, sf_qfmt(b, r, 128), SF_REFINE_ROW_MAJOR, which,
            _ptr(out), _stream(stream),
        )
    )
    return out


# ---- nested KV cache ---------------------------------------------------------------
class QuantKV:
    """Nested-quantised KV cache [batch][n_kv][t_cap][head_dim] on the device, plus a
    device copy of every token's refinement unit (unit id (b*n_kv + h)*t_cap + t)."""

    def __init__(self, batch, n_kv, t_cap, b, r, device="cuda", head_dim=128):
        torch = _torch()
        self.batch, self.n_kv, self.t_cap, self.b, self.r, self.d = batch, n_kv, t_cap, b, r, head_dim
        self.t_len = 0
        dev = torch.device(device)
        self.k_res = torch.zeros((batch, n_kv, t_cap, head_dim * b // 8), dtype=torch.uint8, device=dev)
        self.v_res = torch.zeros_like(self.k_res)
        self.k_sz = torch.zeros((batch, n_kv, t_cap), dtype=torch.int32, device=dev)
        self.v_sz = torch.zeros_like(self.k_sz)
        self.refine = torch.zeros((batch, n_kv, t_cap, self.unit_bytes), dtype=torch.uint8, device=dev)

    @property
    def unit_bytes(self):
        return 2 * self.d * self.r // 8

    @property
    def n_units(self):
        return self.batch * self.n_kv * self.t_cap

    def desc(self, t_len=None):
        return sf_qkv(
            self.k_res.data_ptr(), self.k_sz.data_ptr(), self.v_res.data_ptr(), self.v_sz.data_ptr(),
            self.batch, self.n_kv, self.d, self.t_len if t_len is None else t_len, self.t_cap,
            sf_qfmt(self.b, self.r, 128),
        )

    def append(self, K_new, V_new, stream=None):
        """Quantise n_tok new tokens (fp32 [batch][n_kv][n_tok][d]) at t_len.."""
        torch = _torch()
        dev = self.k_res.device
        K_new = _dev_tensor(K_new, torch.float32, dev)
        V_new = _dev_tensor(V_new, torch.float32, dev)
        n_tok = K_new.shape[2]
        d = self.desc()
        # refinement units land in place in the device store
        dst = self.refine.data_ptr() + self.t_len * self.unit_bytes
        check(lib().sf_kv_append(_ptr(K_new), _ptr(V_new), n_tok, self.t_len, C.byref(d), C.c_void_p(dst),
                                 self.t_cap, _stream(stream)))
        self.t_len += n_tok
        return self.refine[:, :, self.t_len - n_tok : self.t_len]

    @classmethod
    def from_host(cls, K, V, b, r, device="cuda", t_cap=None):
        batch, n_kv, T, d = K.shape
        kv = cls(batch, n_kv, t_cap or T, b, r, device=device, head_dim=d)
        kv.append(K, V)
        return kv

    def resident_pool_desc(self, max_lookup=0):
        return sf_pool_desc(self.unit_bytes, self.n_units, self.n_units, None, self.refine.data_ptr(), max_lookup)

    def host_store(self):
        return self.refine.reshape(self.n_units, self.unit_bytes).to("cpu").pin_memory()


# ---- refinement cache ---------------------------------------------------------------
class RefineCache:
    def __init__(self, pools, mode=SF_CACHE_DETERMINISTIC, max_fill=0, device=None, keep=()):
        torch = _torch()
        arr = (sf_pool_desc * len(pools))(*pools)
        h = C.c_void_p()
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        with torch.cuda.device(dev):
            check(lib().sf_refine_cache_create(arr, len(pools), mode, max_fill, C.byref(h)))
        self.handle = h
        self.n_pools = len(pools)
        self._keep = list(keep)  # host stores etc. that must outlive the cache

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.sf_refine_cache_destroy(self.handle)
            self.handle = None

    def lookup(self, pool, ids, stream=None):
        torch = _torch()
        ids = ids.to(torch.int32).contiguous()
        out = torch.empty_like(ids)
        check(lib().sf_refine_cache_lookup(self.handle, pool, _ptr(ids), ids.numel(), _ptr(out), _stream(stream)))
        return out

    def fill(self, stream=None, side=None):
        torch = _torch()
        if side is None:
            side = getattr(self, "_side", None)
            if side is None:
                side = self._side = torch.cuda.Stream()
        n = C.c_int64(0)
        check(lib().sf_refine_cache_fill(self.handle, _stream(stream), _stream(side), C.byref(n)))
        return n.value

    def stats(self, pool=-1):
        v = [C.c_int64(0) for _ in range(4)]
        check(lib().sf_refine_cache_stats(self.handle, pool, *[C.byref(x) for x in v]))
        return dict(zip(("lookups", "hits", "installed", "h2d_bytes"), [x.value for x in v]))

    def prefetch(self, pool, ids, stream=None):
        """Fetch lead: the pool's lead slots come to hold the units `ids` (device int32)."""
        torch = _torch()
        ids = ids.to(torch.int32).contiguous()
        check(lib().sf_refine_cache_prefetch(self.handle, pool, _ptr(ids), ids.numel(), _stream(stream)))
        return ids

    def io_stats(self, pool=-1):
        """Reads of the pools with a store file: units, bytes, median / p99 read time
        (us), wall time spent reading (ms)."""
        n, by = C.c_int64(0), C.c_int64(0)
        a, b, w = C.c_double(0), C.c_double(0), C.c_double(0)
        check(lib().sf_refine_cache_io_stats(self.handle, pool, C.byref(n), C.byref(by), C.byref(a), C.byref(b),
                                             C.byref(w)))
        return {"reads": n.value, "bytes": by.value, "p50_us": a.value, "p99_us": b.value, "read_ms": w.value}

    def resident(self, pool, capacity):
        ids = (C.c_int64 * max(1, capacity))()
        n = C.c_int64(0)
        check(lib().sf_refine_cache_resident(self.handle, pool, ids, C.byref(n)))
        return set(ids[i] for i in range(n.value))


def write_store_file(path, store):
    """Writes a store tensor [n_units][unit_bytes] (any device) to `path`, unit u at
    byte u * unit_bytes (plain bytes: the file a store-file pool reads)."""
    arr = store.reshape(store.shape[0], -1).to("cpu").numpy()
    with open(path, "wb") as f:
        f.write(arr.tobytes())
        f.flush()
        os.fsync(f.fileno())


def file_pool_desc(path, unit_bytes, n_units, capacity, max_lookup=0, offset=0):
    """Pool whose units are read from a file (unit u at offset + u * unit_bytes)."""
    d = sf_pool_desc(unit_bytes, n_units, capacity, None, None, max_lookup)
    d.store_file = os.fsencode(path)
    d.store_offset = offset
    return d


def host_pool_desc(host_store, capacity, max_lookup=0, lead_slots=0):
    """Pool over a pinned host store tensor [n_units][unit_bytes] with `capacity` LRU
    slots and `lead_slots` slots for prefetches (fetch lead)."""
    n, ub = host_store.shape
    d = sf_pool_desc(ub, n, capacity, host_store.data_ptr(), None, max_lookup)
    d.lead_slots = lead_slots
    return d


# ---- refined GEMV -------------------------------------------------------------------
def refined_gemv(ops, x, k_sel, cache=None, sel_in=None, stream=None, ys=None, want_hits=True):
    """ops: list of (QuantWeight, pool index or -1); x fp16 [batch][k_in].
    Returns (list of y [batch][n_out] fp32, sel int32 [k_sel], list of hit tensors)."""
    torch = _torch()
    w0 = ops[0][0]
    dev = w0.resident.device
    xb = _f16_bits(x, dev)
    if xb.dim() == 1:
        xb = xb[None]
    batch = xb.shape[0]
    n = len(ops)
    arr = (sf_gemv_op * n)()
    outs, hits = [], []
    for i, (w, pool) in enumerate(ops):
        y = ys[i] if ys is not None else torch.empty((batch, w.n_out), dtype=torch.float32, device=dev)
        h = torch.empty(max(1, k_sel), dtype=torch.int32, device=dev) if want_hits else None
        arr[i] = sf_gemv_op(w.desc(), pool if cache is not None else -1, y.data_ptr(), h.data_ptr() if h is not None else None)
        outs.append(y)
        hits.append(h[:k_sel] if h is not None else None)
    sel = torch.empty(max(1, k_sel), dtype=torch.int32, device=dev)
    sin = _dev_tensor(sel_in, torch.int32, dev) if sel_in is not None else None
    ws = workspace(lib().sf_workspace_bytes_gemv(arr, n, batch, k_sel), dev)
    check(
        lib().sf_refined_gemv(
            arr, n, _ptr(xb), batch, k_sel, _ptr(sin), _ptr(sel), cache.handle if cache else None, ws.handle,
            _stream(stream),
        )
    )
    return outs, sel[:k_sel], hits


# ---- refined attention ----------------------------------------------------------------
SF_ATTN_NESTED, SF_ATTN_FP16_TOKENS, SF_ATTN_DROP_UNSELECTED = 0, 1, 2


def refined_attention(q, kv, scale, k_sel, cache=None, pool=0, sel_in=None, stream=None, out=None, t_len=None,
                      variant=SF_ATTN_NESTED):
    """q fp16 [batch][n_q][d].  Returns (out fp32 [batch][n_q][d], sel [batch][n_kv][k_sel],
    hits [batch][n_kv][k_sel])."""
    torch = _torch()
    dev = kv.k_res.device
    qb = _f16_bits(q, dev)
    batch, n_q, d = qb.shape
    o = out if out is not None else torch.empty((batch, n_q, d), dtype=torch.float32, device=dev)
    ks = max(1, k_sel)
    sel = torch.empty((batch, kv.n_kv, ks), dtype=torch.int32, device=dev)
    hit = torch.empty((batch, kv.n_kv, ks), dtype=torch.int32, device=dev)
    sin = _dev_tensor(sel_in, torch.int32, dev) if sel_in is not None else None
    tl = kv.t_len if t_len is None else t_len
    ws = workspace(lib().sf_workspace_bytes_attn(batch, n_q, kv.n_kv, tl, k_sel), dev)
    d_ = kv.desc(tl)
    check(
        lib().sf_attn_decode_variant(
            _ptr(qb), n_q, C.byref(d_), float(scale), k_sel, _ptr(sin), cache.handle if cache else None, pool,
            _ptr(o), _ptr(sel), _ptr(hit), ws.handle, _stream(stream), variant,
        )
    )
    return o, sel[:, :, :k_sel], hit[:, :, :k_sel]


def refined_attention_append(q, kv, K_new, V_new, scale, k_sel, cache=None, pool=0, stream=None, out=None,
                             out_f16=None):
    """Appends one token (K_new, V_new fp32 [batch][n_kv][d]) at position kv.t_len and
    attends over kv.t_len + 1 tokens in one call (sf_refined_attn_decode_append); the
    token's refinement units land in place in kv.refine; out_f16 (int16 [batch][n_q][d],
    optional) receives the output as fp16 bits.  Returns (out, sel, hits) as
    refined_attention."""
    torch = _torch()
    dev = kv.k_res.device
    qb = _f16_bits(q, dev)
    batch, n_q, d = qb.shape
    K_new = _dev_tensor(K_new, torch.float32, dev).reshape(batch, kv.n_kv, d).contiguous()
    V_new = _dev_tensor(V_new, torch.float32, dev).reshape(batch, kv.n_kv, d).contiguous()
    o = out if out is not None else torch.empty((batch, n_q, d), dtype=torch.float32, device=dev)
    ks = max(1, k_sel)
    sel = torch.empty((batch, kv.n_kv, ks), dtype=torch.int32, device=dev)
    hit = torch.empty((batch, kv.n_kv, ks), dtype=torch.int32, device=dev)
    tl = kv.t_len + 1
    ws = workspace(lib().sf_workspace_bytes_attn(batch, n_q, kv.n_kv, tl, k_sel), dev)
    d_ = kv.desc(tl)
    dst = kv.refine.data_ptr() + kv.t_len * kv.unit_bytes
    check(
        lib().sf_refined_attn_decode_append(
            _ptr(qb), n_q, C.byref(d_), _ptr(K_new), _ptr(V_new), C.c_void_p(dst), kv.t_cap, float(scale), k_sel,
            None, cache.handle if cache else None, pool, _ptr(o), _ptr(out_f16), _ptr(sel), _ptr(hit), ws.handle,
            _stream(stream),
        )
    )
    kv.t_len = tl
    return o, sel[:, :, :k_sel], hit[:, :, :k_sel]


# ---- decode-step glue ------------------------------------------------------------------
def embed(table_f16, ids, out=None, stream=None):
    """table_f16 int16/fp16 [vocab][hidden] (device), ids int32 [batch] -> fp32 [batch][hidden]."""
    torch = _torch()
    vocab, hidden = table_f16.shape
    ids = _dev_tensor(ids, torch.int32, table_f16.device)
    out = out if out is not None else torch.empty((ids.numel(), hidden), dtype=torch.float32, device=table_f16.device)
    check(lib().sf_embed(_ptr(table_f16), vocab, hidden, _ptr(ids), ids.numel(), _ptr(out), _stream(stream)))
    return out


def add_rmsnorm(h, y, w, eps, out=None, stream=None):
    """h fp32 [batch][hidden] (h += y in place if y is given); returns fp16 bits int16 [batch][hidden]."""
    torch = _torch()
    batch, hidden = h.shape
    out = out if out is not None else torch.empty((batch, hidden), dtype=torch.int16, device=h.device)
    check(lib().sf_add_rmsnorm(_ptr(h), _ptr(y), _ptr(w), batch, hidden, float(eps), _ptr(out), _stream(stream)))
    return out


def qk_rope(q, k, n_q, n_kv, q_norm_w, k_norm_w, eps, pos, theta, stream=None):
    """q fp32 [batch][n_q*128], k fp32 [batch][n_kv*128]; returns (q fp16 bits int16
    [batch][n_q][128], rotated k fp32 [batch][n_kv][128])."""
    torch = _torch()
    batch = q.shape[0]
    qh = torch.empty((batch, n_q, 128), dtype=torch.int16, device=q.device)
    ko = torch.empty((batch, n_kv, 128), dtype=torch.float32, device=q.device)
    check(lib().sf_qk_rope(_ptr(q), _ptr(k), batch, n_q, n_kv, _ptr(q_norm_w), _ptr(k_norm_w), float(eps), int(pos),
                           float(theta), _ptr(qh), _ptr(ko), _stream(stream)))
    return qh, ko


def swiglu(gate, up, out=None, stream=None):
    torch = _torch()
    out = out if out is not None else torch.empty(gate.shape, dtype=torch.int16, device=gate.device)
    check(lib().sf_swiglu(_ptr(gate), _ptr(up), gate.numel(), _ptr(out), _stream(stream)))
    return out


def to_f16(x, out=None, stream=None):
    torch = _torch()
    out = out if out is not None else torch.empty(x.shape, dtype=torch.int16, device=x.device)
    check(lib().sf_to_f16(_ptr(x), x.numel(), _ptr(out), _stream(stream)))
    return out


def argmax(logits, out=None, stream=None):
    torch = _torch()
    batch, vocab = logits.shape
    out = out if out is not None else torch.empty(batch, dtype=torch.int32, device=logits.device)
    check(lib().sf_argmax(_ptr(logits), batch, vocab, _ptr(out), _stream(stream)))
    return out


def add_rmsnorm_select(h, y, w, eps, k_sel, out=None, sel=None, stream=None):
    """h fp32 [batch][hidden] (h += y in place if y is given) -> (x fp16 bits int16
    [batch][hidden], the k_sel channels of largest max-over-rows |x|, ascending)."""
    torch = _torch()
    batch, hidden = h.shape
    out = out if out is not None else torch.empty((batch, hidden), dtype=torch.int16, device=h.device)
    sel = sel if sel is not None else torch.empty(max(1, k_sel), dtype=torch.int32, device=h.device)
    check(lib().sf_add_rmsnorm_select(_ptr(h), _ptr(y), _ptr(w), batch, hidden, float(eps), _ptr(out), k_sel, _ptr(sel),
                                      _stream(stream)))
    return out, sel[:k_sel]


def swiglu_select(gate, up, k_sel, out=None, sel=None, stream=None):
    torch = _torch()
    batch, n = gate.shape
    out = out if out is not None else torch.empty((batch, n), dtype=torch.int16, device=gate.device)
    sel = sel if sel is not None else torch.empty(max(1, k_sel), dtype=torch.int32, device=gate.device)
    check(lib().sf_swiglu_select(_ptr(gate), _ptr(up), batch, n, _ptr(out), k_sel, _ptr(sel), _stream(stream)))
    return out, sel[:k_sel]


def to_f16_select(x, k_sel, out=None, sel=None, stream=None):
    torch = _torch()
    batch, n = x.shape
    out = out if out is not None else torch.empty((batch, n), dtype=torch.int16, device=x.device)
    sel = sel if sel is not None else torch.empty(max(1, k_sel), dtype=torch.int32, device=x.device)
    check(lib().sf_to_f16_select(_ptr(x), batch, n, _ptr(out), k_sel, _ptr(sel), _stream(stream)))
    return out, sel[:k_sel]


def residual_add(h, d, stream=None):
    """h += d in place (fp32 device tensors of equal size)."""
    check(lib().sf_residual_add(_ptr(h), _ptr(d), h.numel(), _stream(stream)))
    return h


def refine_lag_delta(cache, pool, w, x, sel, hit, out=None, stream=None):
    """Late contribution of the selected channels that missed (hit < 0) in a GEMV of
    QuantWeight w on fp16 x [batch][k_in]: fp32 [batch][n_out]."""
    torch = _torch()
    dev = w.resident.device
    xb = _f16_bits(x, dev)
    if xb.dim() == 1:
        xb = xb[None]
    batch = xb.shape[0]
    o = out if out is not None else torch.empty((batch, w.n_out), dtype=torch.float32, device=dev)
    d = w.desc()
    check(lib().sf_refine_lag_delta(cache.handle, pool, C.byref(d), _ptr(xb), batch, sel.numel(), _ptr(sel), _ptr(hit),
                                    _ptr(o), _stream(stream)))
    return o


def fp16_fetch_gemv(w, x, k_sel, cache, pool, sel_in=None, stream=None):
    """FP16 fetch (comparison variant) for one QuantWeight: the resident GEMV with the
    channel selection, a lookup of the selection in `pool` (fp16 columns), and the
    fetched columns' correction to their fp16 value.  Returns (y, sel, slots)."""
    (y,), sel, _ = refined_gemv([(w, -1)], x, k_sel, cache=None, sel_in=sel_in, stream=stream, want_hits=False)
    if k_sel == 0:
        return y, sel, sel
    slots = cache.lookup(pool, sel, stream=stream)
    xb = _f16_bits(x, w.resident.device)
    if xb.dim() == 1:
        xb = xb[None]
    d = w.desc()
    check(lib().sf_fp16_fetch_delta(cache.handle, pool, C.byref(d), _ptr(xb), xb.shape[0], k_sel, _ptr(sel),
                                    _ptr(slots), _ptr(y), _stream(stream)))
    return y, sel, slots


def fp16_weight_units(W, device="cuda"):
    """fp16 columns of W [n_out][k_in] as units [k_in][2 * n_out] bytes (unit k =
    fp16(W[:, k]), nearest even), on `device`."""
    torch = _torch()
    Wt = torch.as_tensor(np.asarray(W, dtype=np.float32)).t().contiguous().to(torch.float16)
    return Wt.view(torch.uint8).reshape(Wt.shape[0], -1).to(device)


def fp16_kv_units(K, V, device="cuda"):
    """fp16 K and V of every token-head as units [batch*n_kv*T][512] bytes (K's 128
    values, then V's; unit (b, h, t) at (b * n_kv + h) * T + t)."""
    torch = _torch()
    KV = torch.cat([torch.as_tensor(np.asarray(K, dtype=np.float32)), torch.as_tensor(np.asarray(V, dtype=np.float32))],
                   dim=-1).to(torch.float16)
    return KV.view(torch.uint8).reshape(-1, 4 * KV.shape[-1] // 2).to(device)


def device_pool_desc(units):
    """A resident pool over device units [n_units][unit_bytes] (every unit present)."""
    n, ub = units.shape
    return sf_pool_desc(ub, n, n, None, units.data_ptr(), 0)
