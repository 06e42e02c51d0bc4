"""The C ABI library loads on the CPU and exports every function the header declares
(no compute calls: there is no GPU here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "strataflux.h")
LIB = os.path.join(ROOT, "bit_decode_selective_amd", "libstrataflux.so")


@pytest.fixture(scope="module")
def built():
    if not os.path.exists(LIB):
        import __graft_entry__

        __graft_entry__.build()
    assert os.path.exists(LIB)
    return LIB


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sf_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for required in (
        "sf_quantize_nested",
        "sf_refined_gemv",
        "sf_refined_attn_decode",
        "sf_refine_cache_lookup",
        "sf_refine_cache_fill",
        "sf_kv_append",
    ):
        assert required in names


def test_library_exports_every_declared_symbol(built):
    out = subprocess.run(["nm", "-D", "--defined-only", built], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s(sf_[a-z0-9_]+)$", out, flags=re.M))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing


def test_binding_prototypes_cover_header(built):
    from bit_decode_selective_amd import binding

    assert set(_declared()) == set(binding.EXPORTS)


def test_host_only_calls(built):
    lib = ctypes.CDLL(built)
    lib.sf_abi_version.restype = ctypes.c_int32
    assert lib.sf_abi_version() == 1
    lib.sf_status_string.restype = ctypes.c_char_p
    lib.sf_status_string.argtypes = [ctypes.c_int32]
    assert lib.sf_status_string(0) == b"ok"
    assert lib.sf_status_string(1) == b"invalid argument"
    # size queries are host arithmetic
    from bit_decode_selective_amd.binding import sf_gemv_op, sf_qfmt, sf_qweight

    lib.sf_workspace_bytes_gemv.restype = ctypes.c_size_t
    lib.sf_workspace_bytes_gemv.argtypes = [ctypes.POINTER(sf_gemv_op), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    ops = (sf_gemv_op * 3)()
    for i, n_out in enumerate((4096, 1024, 1024)):
        ops[i] = sf_gemv_op(sf_qweight(None, None, n_out, 4096, sf_qfmt(2, 2, 128)), i, None, None)
    # selection and per-op slots of the GEMV live in the workspace
    one = lib.sf_workspace_bytes_gemv(ops, 3, 1, 123)
    assert one >= 123 * 4 * (1 + 3)
    # batch 8 adds the partial outputs of the channel slices: at most
    # [32 slices][8 rows][6144 rows padded to 256] fp32
    eight = lib.sf_workspace_bytes_gemv(ops, 3, 8, 123)
    assert one <= eight <= one + 32 * 8 * 6144 * 4 + 4096
    lib.sf_workspace_bytes_attn.restype = ctypes.c_size_t
    lib.sf_workspace_bytes_attn.argtypes = [ctypes.c_int32] * 5
    assert lib.sf_workspace_bytes_attn(1, 32, 8, 32768, 656) >= 32 * 32768 * 4


def test_argument_errors_without_gpu(built):
    """Argument checks run before any HIP call and report SF_EINVAL / SF_EUNSUPPORTED."""
    from bit_decode_selective_amd import binding

    L = binding.lib()
    st = L.sf_quantize_nested(None, 4, 128, binding.sf_qfmt(2, 2, 128), 0, None, None, None, None)
    assert st == 1
    assert b"null tensor" in L.sf_last_error()
    st = L.sf_quantize_nested(ctypes.c_void_p(8), 4, 128, binding.sf_qfmt(2, 2, 64), 0,
                              ctypes.c_void_p(8), ctypes.c_void_p(8), None, None)
    assert st == 2
    st = L.sf_refined_gemv(None, 0, None, 1, 0, None, None, None, None, None)
    assert st == 1
