"""CPU tests of libtq.so: exported symbols, host-only setup tables against the
oracle, and argument validation (no compute call needs a GPU here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

T = pytest.importorskip("online_vector_quantization_amd")


def _lib():
    if not os.path.exists(T.LIB_PATH):
        pytest.fail("libtq.so is not built (run python -m online_vector_quantization_amd.build)")
    return T.load_library()


def test_library_exports_every_declared_symbol():
    lib = _lib()
    header = open(os.path.join(ROOT, "include", "tq.h")).read()
    declared = set(re.findall(r"^(?:const char \*|tq_status )(tq_\w+)\(", header, flags=re.M))
    assert declared == set(T.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("d", [2, 3, 4, 16, 128])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_host_codebook_matches_oracle(d, bits):
    cb = T.Codebook(d, bits, 32 if d <= 64 else 128, 7, 8, device=-1)
    e32, e64 = cb.export(), cb.export(f64=True)
    c, t, _ = O.lloyd_max(d, bits)
    np.testing.assert_array_equal(e32["centroids"], c.astype(np.float32))
    np.testing.assert_array_equal(e32["thresholds"], t.astype(np.float32))
    np.testing.assert_allclose(e64["centroids"], c, atol=1e-12)
    # the library's codebook is a Lloyd-Max fixed point of the oracle's law too
    edges = np.concatenate(([-1.0], e64["thresholds"], [1.0]))
    cond = np.diff(O.coord_partial_mean(edges, d)) / np.diff(O.coord_cdf(edges, d))
    np.testing.assert_allclose(cond, e64["centroids"], atol=1e-12)


@pytest.mark.parametrize("d,seed", [(4, 0), (16, 3), (128, 0), (128, 12345)])
def test_host_rotation_and_qjl_match_oracle(d, seed):
    m = 32 if d < 128 else 128
    cb = T.Codebook(d, 2, m, seed, seed + 1, device=-1)
    e64, e32 = cb.export(f64=True), cb.export()
    Pi = O.haar_rotation(d, seed)
    np.testing.assert_allclose(e64["rotation"], Pi, atol=1e-12)
    assert np.abs(e64["rotation"] @ e64["rotation"].T - np.eye(d)).max() < 1e-12
    S = O.qjl_matrix(m, d, seed + 1)
    np.testing.assert_allclose(e64["qjl"], S, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(e32["rotation"], Pi.astype(np.float32), atol=1e-7)
    np.testing.assert_allclose(e32["qjl"], S.astype(np.float32), rtol=1e-6)


def test_host_build_is_reproducible():
    a = T.Codebook(128, 3, 128, 0, 1, device=-1).export()
    b = T.Codebook(128, 3, 128, 0, 1, device=-1).export()
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_record_words():
    for bits in (1, 2, 3, 4):
        cb = T.Codebook(128, bits, 128, 0, 1, device=-1)
        assert cb.code_words == 4 * bits and cb.sign_words == 4
    assert T.Codebook(128, 3, 0, 0, 1, device=-1).sign_words == 0


@pytest.mark.parametrize("args,status", [
    ((1, 2, 0), T.api.TQ_ERR_INVALID_ARG),       # head_dim < 2
    ((128, 0, 0), T.api.TQ_ERR_INVALID_ARG),     # bits 0
    ((128, 5, 0), T.api.TQ_ERR_INVALID_ARG),     # bits 5
    ((128, 2, 48), T.api.TQ_ERR_INVALID_ARG),    # m not a multiple of 32
    ((128, 2, -32), T.api.TQ_ERR_INVALID_ARG),
])
def test_build_rejects_bad_arguments(args, status):
    lib = _lib()
    h = ctypes.c_void_p()
    s = lib.tq_codebook_build(args[0], args[1], args[2], 0, 1, -1, ctypes.byref(h))
    assert s == status and not h.value
    assert len(lib.tq_last_error()) > 0


def test_gpu_only_shapes_rejected_before_any_device_call():
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.tq_codebook_build(64, 2, 0, 0, 1, 0, ctypes.byref(h)) == T.api.TQ_ERR_UNSUPPORTED
    assert lib.tq_codebook_build(128, 2, 64, 0, 1, 0, ctypes.byref(h)) == T.api.TQ_ERR_UNSUPPORTED
    assert lib.tq_codebook_build(128, 2, 0, 0, 1, -2, ctypes.byref(h)) == T.api.TQ_ERR_INVALID_ARG
    assert lib.tq_codebook_build(128, 2, 0, 0, 1, 0, None) == T.api.TQ_ERR_INVALID_ARG


def test_host_only_handle_refuses_encode_and_decode():
    lib = _lib()
    cb = T.Codebook(128, 2, 128, 0, 1, device=-1)
    buf = (ctypes.c_uint8 * 4096)()
    s = lib.tq_encode_kv(cb.handle, buf, 1, 1, 128, None, 1, buf, buf, buf, buf, None, None, None)
    assert s == T.api.TQ_ERR_INVALID_ARG
    assert b"host-only" in lib.tq_last_error()
    cache = T.api.TqCache(ctypes.addressof(buf), None, ctypes.addressof(buf), None, 1)
    s = lib.tq_decode_attention(cb.handle, cb.handle, buf, 1, ctypes.byref(cache), ctypes.byref(cache), buf,
                                1, 1, 1, 0.0, buf, 0, None, buf, 4096, None)
    assert s == T.api.TQ_ERR_INVALID_ARG
    s = lib.tq_attention_logits(cb.handle, buf, 1, ctypes.byref(cache), buf, 1, 1, 1, 0.0, buf, buf, 4096, None)
    assert s == T.api.TQ_ERR_INVALID_ARG
    assert b"GPU device" in lib.tq_last_error()
    s = lib.tq_attention_logits(cb.handle, buf, 1, ctypes.byref(cache), buf, 1, 1, 1, 0.0, None, buf, 4096, None)
    assert s == T.api.TQ_ERR_INVALID_ARG
    assert b"logits is NULL" in lib.tq_last_error()


def test_encode_zero_rows_is_a_noop_and_bad_dtype_rejected():
    lib = _lib()
    cb = T.Codebook(128, 2, 0, 0, 1, device=-1)
    # host-only handles are rejected first; check the status table and workspace sizing instead
    assert lib.tq_status_string(0) == b"TQ_OK"
    assert lib.tq_status_string(-4) == b"TQ_ERR_DEVICE"
    assert lib.tq_status_string(7) == b"TQ_UNKNOWN_STATUS"
    del cb


def test_workspace_sizing():
    n1 = T.decode_workspace_bytes(1, 32, 8, 32768)
    n2 = T.decode_workspace_bytes(16, 32, 8, 8200)
    assert n1 > 0 and n2 > 0 and n1 % 256 == 0
    with pytest.raises(T.TQError):
        T.decode_workspace_bytes(1, 30, 8, 100)      # not a multiple
    with pytest.raises(T.TQError):
        T.decode_workspace_bytes(0, 32, 8, 100)
    with pytest.raises(T.TQError):
        T.decode_workspace_bytes(1, 32, 8, 0)


def test_chunk_workspace_sizing():
    # one query per head: the decode plan; 16+ query rows per kv head: the
    # matrix-core plan, which also holds (q~, s) of every query row
    assert T.chunk_workspace_bytes(1, 32, 8, 1, 32768) == T.decode_workspace_bytes(1, 32, 8, 32768)
    assert T.chunk_workspace_bytes(2, 32, 8, 3, 1000) == T.decode_workspace_bytes(6, 32, 8, 1000)
    big = T.chunk_workspace_bytes(1, 32, 8, 16, 32768)
    assert big % 256 == 0 and big >= 1 * 32 * 16 * 256 * 4
    assert T.api.chunk_uses_mfma(4, 4) and not T.api.chunk_uses_mfma(4, 3)
    with pytest.raises(T.TQError):
        T.chunk_workspace_bytes(1, 32, 8, 0, 100)
    with pytest.raises(T.TQError):
        T.chunk_workspace_bytes(1, 30, 8, 4, 100)


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_split_codebook_tables_match_oracle(bits):
    cb = T.Codebook(128, bits, 128, 0, 1, device=-1, wide_coords=64)
    assert cb.split_info() == (64, bits + 1)
    assert cb.code_words == (128 * bits + 64) // 32 and cb.sign_words == 4
    book = O.build_split_book(128, bits, 64)
    wide, narrow = cb.export_wide(), cb.export()
    np.testing.assert_array_equal(wide["centroids"], book["wide"][0])
    np.testing.assert_array_equal(wide["thresholds"], book["wide"][1])
    np.testing.assert_array_equal(narrow["centroids"], book["narrow"][0])
    np.testing.assert_array_equal(narrow["thresholds"], book["narrow"][1])
    # the same seeds give the same Pi and S as a uniform codebook
    u = T.Codebook(128, bits, 128, 0, 1, device=-1).export()
    np.testing.assert_array_equal(narrow["rotation"], u["rotation"])
    np.testing.assert_array_equal(narrow["qjl"], u["qjl"])


def test_split_codebook_validation():
    lib = _lib()
    h = ctypes.c_void_p()
    INV, UNS = T.api.TQ_ERR_INVALID_ARG, T.api.TQ_ERR_UNSUPPORTED
    assert lib.tq_codebook_build_split(128, 4, 64, 0, 0, 1, -1, ctypes.byref(h)) == INV   # b' + 1 = 5
    assert lib.tq_codebook_build_split(128, 2, 129, 0, 0, 1, -1, ctypes.byref(h)) == INV  # past d
    assert lib.tq_codebook_build_split(128, 2, -1, 0, 0, 1, -1, ctypes.byref(h)) == INV
    assert lib.tq_codebook_build_split(128, 2, 32, 0, 0, 1, 0, ctypes.byref(h)) == UNS   # GPU: 0 or 64 only
    assert not h.value
    # host-only: any count; a uniform handle has no wide tables
    cb = T.Codebook(16, 2, 0, 0, 1, device=-1, wide_coords=5)
    assert cb.split_info() == (5, 3) and cb.code_words == (16 * 2 + 5 + 31) // 32
    assert T.Codebook(128, 2, 0, 0, 1, device=-1).split_info() == (0, 0)
    with pytest.raises(T.TQError):
        T.Codebook(128, 2, 0, 0, 1, device=-1).export_wide()
