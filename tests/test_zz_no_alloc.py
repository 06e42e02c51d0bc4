"""GPU: sf_refined_gemv_noalloc (no workspace; library-owned scratch array) gives the
same outputs, selection and hits as sf_refined_gemv on the same inputs, on two calls
in a row, the second one smaller, and refuses a call that needs more scratch than
the array holds before launching anything."""
import ctypes as C

import numpy as np
import pytest
import torch

from bit_decode_selective_amd import binding, inputs
from oracle import selection

from gpu_util import assert_close

pytestmark = pytest.mark.gpu


def _ops(ws_list, ys, hits):
    arr = (binding.sf_gemv_op * len(ws_list))()
    for i, (w, y, h) in enumerate(zip(ws_list, ys, hits)):
        arr[i] = binding.sf_gemv_op(w.desc(), i, y.data_ptr(), h.data_ptr())
    return arr


def _both(qws, x, k_sel, cache):
    """(outputs, selection, hits) of the workspace call and of the scratch call."""
    L = binding.lib()
    dev = qws[0].resident.device
    xb = binding._f16_bits(x, dev)
    batch = xb.shape[0]
    res = []
    for noalloc in (False, True):
        ys = [torch.full((batch, w.n_out), float("nan"), dtype=torch.float32, device=dev) for w in qws]
        hits = [torch.full((max(1, k_sel),), -7, dtype=torch.int32, device=dev) for _ in qws]
        sel = torch.full((max(1, k_sel),), -7, dtype=torch.int32, device=dev)
        arr = _ops(qws, ys, hits)
        s = binding._stream()
        if noalloc:
            st = L.sf_refined_gemv_noalloc(arr, len(qws), binding._ptr(xb), batch, k_sel, None, binding._ptr(sel),
                                           cache.handle, s)
        else:
            ws = binding.workspace(L.sf_workspace_bytes_gemv(arr, len(qws), batch, k_sel), dev)
            st = L.sf_refined_gemv(arr, len(qws), binding._ptr(xb), batch, k_sel, None, binding._ptr(sel),
                                   cache.handle, ws.handle, s)
        binding.check(st)
        torch.cuda.synchronize()
        res.append(([y.cpu().numpy() for y in ys], sel.cpu().numpy()[:k_sel], [h.cpu().numpy()[:k_sel] for h in hits]))
    return res


def _mats(cfg, shapes, b=2, r=2):
    out = []
    for i, (n, k) in enumerate(shapes):
        W = inputs.weight(cfg, 0, i, n, k)
        out.append(binding.QuantWeight.from_host(W, b, r))
    return out


@pytest.mark.parametrize("batch", [1, 8])
def test_noalloc_matches_workspace_call(batch):
    big = _mats(95, [(4096, 4096), (1024, 4096), (1024, 4096)])
    small = _mats(96, [(512, 1024)])
    for qws in (big, small):  # two calls in a row, the second with a smaller input
        k_in = qws[0].k_in
        cache = binding.RefineCache([w.resident_pool_desc() for w in qws])
        x = inputs.activation(95, 0, 0, 0, batch, k_in)
        ks = selection.k_select(3, k_in)
        (ya, sa, ha), (yb, sb, hb) = _both(qws, x, ks, cache)
        assert sb.tolist() == sa.tolist() == selection.select_channels(x, ks)
        for a_, b_ in zip(ha, hb):
            assert np.array_equal(a_, b_)
        for a_, b_ in zip(ya, yb):
            assert not np.isnan(b_).any()
            assert_close(b_, a_, what="noalloc vs workspace")


def test_noalloc_refuses_calls_beyond_the_scratch():
    """A batch-16 GEMV with 4 x 14336 rows and every channel refined needs more than
    8 MiB of scratch for its selection, slots and partials: SF_ENOMEM, no launch."""
    L = binding.lib()
    ops = (binding.sf_gemv_op * 4)()
    for i in range(4):
        ops[i] = binding.sf_gemv_op(binding.sf_qweight(C.c_void_p(256), C.c_void_p(256), 14336, 32768,
                                                       binding.sf_qfmt(2, 2, 128)), -1, C.c_void_p(256), None)
    need = L.sf_workspace_bytes_gemv(ops, 4, 16, 32768)
    assert need > (8 << 20)
    st = L.sf_refined_gemv_noalloc(ops, 4, C.c_void_p(256), 16, 32768, None, None, None, None)
    assert st == 3
    assert b"scratch" in L.sf_last_error()
