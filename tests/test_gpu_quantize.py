"""GPU parity: nested quantisation (packed codes, scale/zero, dequantised values) and
KV append, bit-exact against the oracle (through the C ABI)."""
import numpy as np
import pytest

from bit_decode_selective_amd import binding, inputs
from oracle import attention as o_attn
from oracle import nested

pytestmark = pytest.mark.gpu


def _split_sz(sz):
    w = sz.cpu().numpy().astype(np.uint32)
    return (w & 0xFFFF).astype(np.uint16), (w >> 16).astype(np.uint16)


def _check_weight(W, b, r):
    qw = binding.QuantWeight.from_host(W, b, r)
    q = nested.quantize(W, b, r, 128)
    p = nested.pack_weight(q)
    assert np.array_equal(qw.resident.cpu().numpy(), p["resident"]), "resident bytes"
    s_bits, z_bits = _split_sz(qw.sz)
    assert np.array_equal(s_bits, q["scale"].view(np.uint16)), "scale bits"
    assert np.array_equal(z_bits, q["zero"].view(np.uint16)), "zero bits"
    if r > 0:
        assert np.array_equal(qw.refine.cpu().numpy(), p["refine"]), "channel-major refinement"
    res = qw.dequantize(0).cpu().numpy()
    assert np.array_equal(res, nested.to_f32(nested.dequant_resident(q))), "resident values"
    if r > 0:
        full = qw.dequantize(1).cpu().numpy()
        assert np.array_equal(full, nested.to_f32(nested.dequant_full(q))), "full values"
    # row-major refinement layout
    res_b, sz_b, ref_b = binding.quantize_rows(W, b, r)
    rr, rl = nested.pack_rows(q)
    assert np.array_equal(res_b.cpu().numpy(), rr)
    if r > 0:
        assert np.array_equal(ref_b.cpu().numpy(), rl)
        full2 = binding.dequantize_rows(res_b, sz_b, ref_b, W.shape[0], W.shape[1], b, r, 1).cpu().numpy()
        assert np.array_equal(full2, nested.to_f32(nested.dequant_full(q)))


def test_worked_example_embedded(golden):
    ex = golden["nested_2bit"]
    W = np.zeros((32, 128), dtype=np.float32)
    W[0, :4] = ex["x"]  # padding zeros lie inside [min, max]: same z and s
    qw = binding.QuantWeight.from_host(W, 2, 2)
    s_bits, z_bits = _split_sz(qw.sz)
    assert np.float16(s_bits[0, 0:1].view(np.float16)[0]) == ex["scale"]
    assert np.float16(z_bits[0, 0:1].view(np.float16)[0]) == ex["zero"]
    assert qw.resident.cpu().numpy()[0, 0] == ex["resident_bytes"][0]
    full = qw.dequantize(1).cpu().numpy()[0, :4]
    res = qw.dequantize(0).cpu().numpy()[0, :4]
    assert full.tolist() == ex["full_value"]
    assert res.tolist() == ex["resident_value"]
    _check_weight(W, 2, 2)


def test_worked_example_3bit_embedded(golden):
    ex = golden["nested_3bit_straddle"]
    W = np.zeros((32, 128), dtype=np.float32)
    W[0, :8] = np.array(ex["x_over_0.0625"], dtype=np.float32) * np.float32(0.0625)
    qw = binding.QuantWeight.from_host(W, 3, 1)
    assert qw.resident.cpu().numpy()[0, :3].tolist() == ex["resident_bytes"]
    _check_weight(W, 3, 1)


@pytest.mark.parametrize("b,r", [(2, 2), (3, 1), (2, 1), (1, 3), (4, 4), (8, 0), (5, 2), (2, 0)])
def test_random_formats(b, r):
    W = inputs.weight(90, b, r, 96, 384)
    W[3, :128] *= 40.0  # outlier group
    W[5, 128:256] = 0.125  # constant group
    W[7, 256:] = -0.0
    _check_weight(W, b, r)


def test_full_size_single_layer_weight():
    """4096 x 4096 weight, N(0, 0.02), 2 + 2 bits."""
    W = inputs.weight(1, 0, inputs.Q_PROJ, 4096, 4096)
    _check_weight(W, 2, 2)


@pytest.mark.parametrize("b,r", [(2, 2), (4, 4), (1, 1)])
def test_kv_append_matches_oracle(b, r):
    K, V = inputs.kv(91, b, 2, 3, 70, 128)
    kv = binding.QuantKV(2, 3, 80, b, r)
    kv.append(K[:, :, :33], V[:, :, :33])
    kv.append(K[:, :, 33:], V[:, :, 33:])  # second append lands at t = 33
    qk = o_attn.quantize_kv(K, b, r)
    qv = o_attn.quantize_kv(V, b, r)
    rk, lk = nested.pack_rows(qk)
    rv, lv = nested.pack_rows(qv)
    got_k = kv.k_res.cpu().numpy()[:, :, :70].reshape(-1, 16 * b)
    got_v = kv.v_res.cpu().numpy()[:, :, :70].reshape(-1, 16 * b)
    assert np.array_equal(got_k, rk) and np.array_equal(got_v, rv)
    s_bits, z_bits = _split_sz(kv.k_sz[:, :, :70].reshape(-1, 1))
    assert np.array_equal(s_bits, qk["scale"].view(np.uint16))
    assert np.array_equal(z_bits, qk["zero"].view(np.uint16))
    unit = kv.refine.cpu().numpy()[:, :, :70].reshape(-1, 32 * r)
    assert np.array_equal(unit[:, : 16 * r], lk) and np.array_equal(unit[:, 16 * r :], lv)
    # positions beyond t_len untouched
    assert not kv.k_res[:, :, 70:].any()
