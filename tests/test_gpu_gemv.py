"""GPU parity: refined GEMV (channel selection bit-exact, outputs within 1e-3 rel /
1e-4 abs of the fp64 oracle), through the C ABI."""
import numpy as np
import pytest
import torch

from bit_decode_selective_amd import binding, inputs
from oracle import gemv as o_gemv
from oracle import nested, selection

from gpu_util import assert_close

pytestmark = pytest.mark.gpu


def _setup(cfg, n_out, k_in, b, r, tensor=0):
    W = inputs.weight(cfg, 0, tensor, n_out, k_in)
    qw = binding.QuantWeight.from_host(W, b, r)
    return W, qw, nested.quantize(W, b, r, 128)


def _run(qws, x, k_sel, sel_in=None, cache="resident"):
    if cache == "resident" and qws[0].r == 0:
        cache = None
    if cache == "resident":
        cache = binding.RefineCache([w.resident_pool_desc() for w in qws])
    ops = [(w, i) for i, w in enumerate(qws)]
    ys, sel, hits = binding.refined_gemv(ops, x, k_sel, cache=cache, sel_in=sel_in)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys], sel.cpu().numpy().tolist(), [h.cpu().numpy() for h in hits]


KINDS = {"split": "1", "staged": "2", "fused": "0"}


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("rpw", ["4", "8"])
@pytest.mark.parametrize("b,r", [(2, 2), (3, 1), (4, 4), (1, 3), (8, 0), (2, 0)])
@pytest.mark.parametrize("batch", [1, 2, 3])
def test_small_shapes(b, r, batch, rpw, kind, monkeypatch):
    """Selection by one workgroup while the others stream (split: x in registers;
    staged: x in LDS) or in every workgroup (fused); 4 or 8 rows per wave; one launch
    for batch 1-2; b = 3 at batch 3 takes the selection launch and two launches,
    the others the batched kernel."""
    monkeypatch.setenv("SF_GEMV_ROWS_PER_WAVE", rpw)
    monkeypatch.setenv("SF_GEMV_SPLIT", KINDS[kind])
    # 200 rows is ragged against every row tile; channel-major refinement units need
    # n_out * r to be a multiple of 32, so the odd-r formats use 224 rows
    n_out = 200 if r in (0, 4) else 224
    k_in = 640  # 5 groups
    W, qw, q = _setup(11, n_out, k_in, b, r)
    x = inputs.activation(11, 0, 0, 0, batch, k_in)
    for k_sel in ([0] if r == 0 else [0, 1, 17, k_in]):
        (y,), sel, (hit,) = _run([qw], x, k_sel)
        want_sel = selection.select_channels(x, k_sel)
        assert sel == want_sel
        if k_sel:
            assert np.all(hit >= 0)
        assert_close(y, o_gemv.refined_gemv(q, x, want_sel), what=f"b{b} r{r} batch{batch} k{k_sel}")


def test_selection_ties_go_to_lower_channel():
    W, qw, q = _setup(12, 64, 256, 2, 2)
    x = np.zeros((1, 256), dtype=np.float16)
    x[0, [3, 50, 51, 200, 7]] = [2.0, -1.0, 1.0, 1.0, -2.0]
    (y,), sel, _ = _run([qw], x, 3)
    assert sel == [3, 7, 50]
    assert_close(y, o_gemv.refined_gemv(q, x, [3, 7, 50]))


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("fill", [0.0, 0.5])
def test_all_equal_inputs_select_lowest_channels(kind, fill, monkeypatch):
    """Every |x| equal (an all-zero input, or one constant): all keys tie, so the
    selection is the lowest k_sel channels; 14336 input channels (the down
    projection's width) at batch 1."""
    monkeypatch.setenv("SF_GEMV_SPLIT", KINDS[kind])
    W, qw, q = _setup(13, 256, 14336, 2, 2)
    x = np.full((1, 14336), fill, dtype=np.float16)
    x[0, 1::2] *= -1  # signs do not change the key
    ks = selection.k_select(3, 14336)
    (y,), sel, _ = _run([qw], x, ks)
    assert sel == list(range(ks))
    assert_close(y, o_gemv.refined_gemv(q, x, sel), what=f"constant |x| = {fill}")


def test_fused_ops_and_external_selection():
    k_in = 1024
    qs = [_setup(13, n, k_in, 2, 2, tensor=i) for i, n in enumerate((256, 64, 64))]
    x = inputs.activation(13, 0, 0, 0, 1, k_in)
    ks = selection.k_select(3, k_in)
    ys, sel, hits = _run([t[1] for t in qs], x, ks)
    want = selection.select_channels(x, ks)
    assert sel == want
    for (W, qw, q), y in zip(qs, ys):
        assert_close(y, o_gemv.refined_gemv(q, x, want))
    ext = sorted(np.random.default_rng(0).choice(k_in, ks, replace=False).tolist())
    ys, sel, _ = _run([t[1] for t in qs], x, ks, sel_in=np.array(ext, dtype=np.int32))
    assert sel == ext
    for (W, qw, q), y in zip(qs, ys):
        assert_close(y, o_gemv.refined_gemv(q, x, ext))


def test_misses_fall_back_to_resident():
    """No cache / an empty pool: every selected channel misses -> b-bit GEMV."""
    W, qw, q = _setup(14, 128, 512, 2, 2)
    x = inputs.activation(14, 0, 0, 0, 1, 512)
    (y,), sel, (hit,) = _run([qw], x, 40, cache=None)
    assert np.all(hit == -1)
    assert_close(y, o_gemv.refined_gemv(q, x, []))
    store = qw.host_store()
    empty = binding.RefineCache([binding.host_pool_desc(store, 0)], keep=[store])
    (y2,), _, (hit2,) = _run([qw], x, 40, cache=empty)
    assert np.all(hit2 == -1)
    assert_close(y2, o_gemv.refined_gemv(q, x, []))


def test_repeated_calls_reuse_workspace():
    W, qw, q = _setup(15, 304, 768, 2, 2)
    cache = binding.RefineCache([qw.resident_pool_desc()])
    for step in range(5):
        x = inputs.activation(15, 0, 0, step, 1, 768)
        ks = [0, 23, 5, 768, 23][step]
        (y,), sel, _ = _run([qw], x, ks, cache=cache)
        want = selection.select_channels(x, ks)
        assert sel == want
        assert_close(y, o_gemv.refined_gemv(q, x, want))


def test_single_layer_4096():
    """4096 x 4096, 2 + 2 bits, x with 1% outlier channels x20, top 5% refined."""
    W, qw, q = _setup(1, 4096, 4096, 2, 2)
    x = inputs.activation(1, 0, 0, 0, 1, 4096)
    ks = selection.k_select(5, 4096)
    (y,), sel, (hit,) = _run([qw], x, ks)
    want = selection.select_channels(x, ks)
    assert sel == want and np.all(hit >= 0)
    assert_close(y, o_gemv.refined_gemv(q, x, want))


@pytest.mark.parametrize("batch", [1, 8])
def test_llama8b_layer_shapes(batch):
    """One decoder layer of Llama-3.1-8B shape at full size: q/k/v fused, o, gate/up
    fused, down; 2 + 2 bits; top 3% channels; batch 1 and 8."""
    shapes = {"qkv": [(4096, 4096), (1024, 4096), (1024, 4096)], "o": [(4096, 4096)],
              "gu": [(14336, 4096), (14336, 4096)], "down": [(4096, 14336)]}
    for gi, (name, mats) in enumerate(shapes.items()):
        k_in = mats[0][1]
        qs = [_setup(2, n, k, 2, 2, tensor=10 * gi + i) for i, (n, k) in enumerate(mats)]
        x = inputs.activation(2, 0, 10 * gi, 0, batch, k_in)
        ks = selection.k_select(3, k_in)
        ys, sel, hits = _run([t[1] for t in qs], x, ks)
        want = selection.select_channels(x, ks)
        assert sel == want, name
        for (W, qw, q), y in zip(qs, ys):
            assert_close(y, o_gemv.refined_gemv(q, x, want), what=name)
        del qs
        torch.cuda.empty_cache()


@pytest.mark.parametrize("rt,slices", [("1", "1"), ("2", "0"), ("4", "5"), ("0", "0")])
@pytest.mark.parametrize("b,r", [(2, 2), (4, 4), (1, 3), (8, 0)])
@pytest.mark.parametrize("batch", [1, 3, 8, 16, 19])
def test_batched_mfma(b, r, batch, rt, slices, monkeypatch):
    """The batched (MFMA) kernel: 16-row tiles, 1/2/4 tiles per wave, one or several
    channel slices summed by the last workgroup, batch rows beyond 16 in a second
    launch; ragged rows; no, one, a few and all channels refined."""
    monkeypatch.setenv("SF_GEMV_MFMA", "1")
    monkeypatch.setenv("SF_GEMV_MFMA_RT", rt)
    monkeypatch.setenv("SF_GEMV_MFMA_SLICES", slices)
    n_out = 200 if r in (0, 4) else 224
    k_in = 640
    W, qw, q = _setup(16, n_out, k_in, b, r)
    x = inputs.activation(16, 0, 0, 0, batch, k_in)
    for k_sel in ([0] if r == 0 else [0, 1, 17, k_in]):
        (y,), sel, (hit,) = _run([qw], x, k_sel)
        want_sel = selection.select_channels(x, k_sel)
        assert sel == want_sel
        assert_close(y, o_gemv.refined_gemv(q, x, want_sel), what=f"b{b} r{r} batch{batch} k{k_sel}")


@pytest.mark.parametrize("slices", ["0", "1", "4"])
def test_batched_mfma_fused_ragged_ops(slices, monkeypatch):
    """Three fused matrices with ragged row counts, 20 groups (more than one slice
    must hold them by default), an external selection and a pool with misses."""
    monkeypatch.setenv("SF_GEMV_MFMA_SLICES", slices)
    k_in = 2560
    qs = [_setup(17, n, k_in, 2, 2, tensor=i) for i, n in enumerate((336, 64, 96))]
    x = inputs.activation(17, 0, 0, 0, 8, k_in)
    ks = selection.k_select(3, k_in)
    ys, sel, hits = _run([t[1] for t in qs], x, ks)
    want = selection.select_channels(x, ks)
    assert sel == want
    for (W, qw, q), y in zip(qs, ys):
        assert_close(y, o_gemv.refined_gemv(q, x, want))
    # empty pools: every selected channel misses and keeps its resident value
    stores = [t[1].host_store() for t in qs]
    cache = binding.RefineCache([binding.host_pool_desc(s, 0) for s in stores], keep=stores)
    ext = sorted(np.random.default_rng(1).choice(k_in, ks, replace=False).tolist())
    ys, sel, hits = _run([t[1] for t in qs], x, ks, sel_in=np.array(ext, dtype=np.int32), cache=cache)
    assert sel == ext
    for (W, qw, q), y, h in zip(qs, ys, hits):
        assert np.all(h == -1)
        assert_close(y, o_gemv.refined_gemv(q, x, []))


def test_batched_mfma_wide_input_takes_the_selection_launch():
    """k_in = 32768 at batch 4: the selector's LDS would not fit the batched launch,
    so the channels come from the selection launch before it (984 of 32768)."""
    W, qw, q = _setup(19, 256, 32768, 2, 2)
    x = inputs.activation(19, 0, 0, 0, 4, 32768)
    ks = selection.k_select(3, 32768)
    (y,), sel, _ = _run([qw], x, ks)
    want = selection.select_channels(x, ks)
    assert sel == want
    assert_close(y, o_gemv.refined_gemv(q, x, want))


def test_batched_mfma_repeated_calls():
    """Slice counters return to zero after every call: alternate shapes and batch
    sizes on one workspace."""
    a = _setup(18, 512, 4096, 2, 2, tensor=0)
    bq = _setup(18, 4096, 1024, 2, 2, tensor=1)
    cache_a = binding.RefineCache([a[1].resident_pool_desc()])
    cache_b = binding.RefineCache([bq[1].resident_pool_desc()])
    for step in range(6):
        W, qw, q = a if step % 2 == 0 else bq
        batch = (8, 5, 16, 8, 3, 12)[step]
        x = inputs.activation(18, 0, step, 0, batch, qw.k_in)
        ks = selection.k_select(3, qw.k_in)
        (y,), sel, _ = _run([qw], x, ks, cache=cache_a if step % 2 == 0 else cache_b)
        want = selection.select_channels(x, ks)
        assert sel == want
        assert_close(y, o_gemv.refined_gemv(q, x, want), what=f"step {step}")


LLAMA_GROUPS = {"qkv": [(4096, 4096), (1024, 4096), (1024, 4096)], "o": [(4096, 4096)],
                "gu": [(14336, 4096), (14336, 4096)], "down": [(4096, 14336)]}


@pytest.mark.parametrize("batch", [1, 3])
def test_llama8b_layer_3plus1(batch):
    """The 128K workload's weights: 3-bit resident + 1 refinement bit (3-bit codes
    straddle words), every Llama-3.1-8B GEMV shape at full size, top 3% channels.
    Batch 3 runs the selection launch, a two-row and a one-row launch; the two-row
    launch of gate/up does not fit the device at once and falls back, which must
    not change the one-row launch's selecting workgroup."""
    for gi, (name, mats) in enumerate(LLAMA_GROUPS.items()):
        k_in = mats[0][1]
        qs = [_setup(6, n, k, 3, 1, tensor=10 * gi + i) for i, (n, k) in enumerate(mats)]
        x = inputs.activation(6, 0, 10 * gi, 0, batch, k_in)
        ks = selection.k_select(3, k_in)
        ys, sel, hits = _run([t[1] for t in qs], x, ks)
        want = selection.select_channels(x, ks)
        assert sel == want, name
        for (W, qw, q), y, h in zip(qs, ys, hits):
            assert np.all(h >= 0)
            assert_close(y, o_gemv.refined_gemv(q, x, want), what=f"3+1 {name} batch {batch}")
        del qs
        torch.cuda.empty_cache()


@pytest.mark.parametrize("batch", [1, 8])
def test_qwen3_ffn_shapes(batch):
    """Qwen3-8B FFN at full size: gate/up 4096 -> 12288 (fused) and down 12288 -> 4096,
    2 + 2 bits, top 3% channels (369 of 12288), batch 1 and 8."""
    for gi, (name, mats) in enumerate({"gu": [(12288, 4096), (12288, 4096)], "down": [(4096, 12288)]}.items()):
        k_in = mats[0][1]
        qs = [_setup(7, n, k, 2, 2, tensor=10 * gi + i) for i, (n, k) in enumerate(mats)]
        x = inputs.activation(7, 0, 10 * gi, 0, batch, k_in)
        ks = selection.k_select(3, k_in)
        ys, sel, hits = _run([t[1] for t in qs], x, ks)
        want = selection.select_channels(x, ks)
        assert sel == want, name
        for (W, qw, q), y in zip(qs, ys):
            assert_close(y, o_gemv.refined_gemv(q, x, want), what=f"qwen3 {name} batch {batch}")
        del qs
        torch.cuda.empty_cache()


@pytest.mark.parametrize("batch", [1, 8])
def test_qwen3_lm_head(batch):
    """The Qwen3-8B lm_head, 4096 -> 151936, 2 + 2 bits, top 3% channels, batch 1 and 8.
    The selection is compared in full; the outputs on 1024 sampled rows plus the
    first and last rows (each output row depends only on its own weight row)."""
    n_out, k_in = 151936, 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(8151936)
    W = inputs.torch_weight(g, n_out, k_in)
    qw = binding.QuantWeight.from_device(W, 2, 2)
    rows = np.unique(np.concatenate([[0, n_out - 1], np.random.default_rng(3).choice(n_out, 1024, replace=False)]))
    W_rows = W[torch.as_tensor(rows, device="cuda")].cpu().numpy()
    del W
    x = inputs.activation(8, 0, inputs.LM_HEAD, 0, batch, k_in)
    ks = selection.k_select(3, k_in)
    (y,), sel, (hit,) = _run([qw], x, ks)
    want = selection.select_channels(x, ks)
    assert sel == want
    assert np.all(hit >= 0)
    q_rows = nested.quantize(W_rows, 2, 2, 128)
    assert_close(y[:, rows], o_gemv.refined_gemv(q_rows, x, want), what=f"lm_head batch {batch}")
    del qw
    torch.cuda.empty_cache()


def test_forced_wait_timeout_is_reported_and_cleared():
    """The host makes the split kernel's bounded waits give up at once (spin limit of
    one poll): every kernel still ends, each output row is either refined or at its
    resident value, sf_workspace_check reports SF_ESTATE and clears the hand-off
    words, and the next call is exact again."""
    W, qw, q = _setup(19, 4096, 4096, 2, 2)
    x = inputs.activation(19, 0, 0, 0, 1, 4096)
    ks = selection.k_select(3, 4096)
    want = selection.select_channels(x, ks)
    y_ref = o_gemv.refined_gemv(q, x, want)
    y_res = o_gemv.refined_gemv(q, x, [])
    cache = binding.RefineCache([qw.resident_pool_desc()])
    ops = [(qw, 0)]
    arr = (binding.sf_gemv_op * 1)(binding.sf_gemv_op(qw.desc(), 0, None, None))
    ws = binding.workspace(binding.lib().sf_workspace_bytes_gemv(arr, 1, 1, ks))
    ws.set_spin_limit(1)
    try:
        (y,), sel, _ = binding.refined_gemv(ops, x, ks, cache=cache)
        torch.cuda.synchronize()
        with pytest.raises(binding.SFError) as err:
            ws.check()
        assert err.value.status == 5
    finally:
        ws.set_spin_limit(0)
    y = y.cpu().numpy()[0]
    tol = 1e-4 + 1e-3 * np.abs(y_ref[0])
    refined = np.abs(y - y_ref[0]) <= tol
    resident = np.abs(y - y_res[0]) <= 1e-4 + 1e-3 * np.abs(y_res[0])
    assert np.all(refined | resident)
    (y2,), sel2, _ = _run([qw], x, ks, cache=cache)
    assert sel2 == want
    assert_close(y2, y_ref)
    ws.check()
