"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Bars: codes, sign bits and packing bit-exact when the
oracle quantizes the GPU's rotated fp32 values (and signs the GPU's fp32
projections); rotated values, projections, norms and scores within 1e-4
relative; decode output within 2e-3 max-abs (fp32 output mode), the bf16
output equal to the RNE rounding of the fp32 one."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from online_vector_quantization_amd import synth  # noqa: E402

import gpu_helpers as H  # noqa: E402
import online_vector_quantization_amd as T  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch sees no GPU")
    T.load_library()


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ encode

def test_encode_tiny_config_fp32_keys():
    wl = synth.tiny()
    x = wl.k.reshape(-1, 128)
    _log(f"encode tiny fp32 n={x.shape[0]}")
    cb = H.gpu_book(2, 128)
    got = H.encode_gpu(cb, H.to_device(x, "f32"))
    flips = H.check_encode(x, got, 2, 128)
    # Codes/signs are checked bit-exactly on the GPU's own fp32 values above; against the
    # oracle's float64 values only decisions within rounding of a threshold (or of p = 0)
    # may differ: a handful in 10^6.
    _log(f"near-boundary flips vs float64 oracle: {flips} of {x.shape[0] * 256}")
    assert flips <= 1e-4 * x.shape[0] * 256


@pytest.mark.parametrize("bits,m", [(1, 128), (2, 128), (3, 128), (1, 0), (2, 0), (3, 0), (4, 0)])
def test_encode_bf16_all_bit_widths(bits, m):
    n = 4133   # several tiles and a ragged tail
    rng = np.random.default_rng(100 + bits + m)
    x = synth.bf16_bits(synth.kv_block(rng, 1, 1, n, synth.outlier_channels(rng, 1, 4))[0, 0])
    _log(f"encode bf16 bits={bits} m={m} n={n}")
    cb = H.gpu_book(bits, m)
    got = H.encode_gpu(cb, H.to_device(x, "bf16"))
    H.check_encode(H.host_values(x, "bf16"), got, bits, m)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 33, 100])
def test_encode_small_and_ragged(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((n, 128)).astype(np.float32)
    _log(f"encode ragged n={n}")
    cb = H.gpu_book(3, 128)
    got = H.encode_gpu(cb, H.to_device(x, "f32"))
    H.check_encode(x, got, 3, 128)


def test_encode_row_stride_and_heavy_tails():
    rng = np.random.default_rng(7)
    n = 1000
    base = synth.kv_block(rng, 1, 1, n, student_t_rate=0.05, lognormal_sigma=0.5)[0, 0]
    wide = np.zeros((n, 192), dtype=np.float32)
    wide[:, :128] = base
    xb = synth.bf16_bits(wide)
    dev = H.to_device(xb, "bf16")[:, :128]        # row stride 192 elements
    assert dev.stride(0) == 192
    cb = H.gpu_book(3, 128)
    got = H.encode_gpu(cb, dev)
    H.check_encode(H.host_values(xb[:, :128], "bf16"), got, 3, 128)


def test_encode_zero_nan_inf_vectors():
    x = np.random.default_rng(3).standard_normal((40, 128)).astype(np.float32)
    x[0] = 0.0
    x[1, 5] = np.nan
    x[2, 7] = np.inf
    x[3] = -0.0
    _log("encode special vectors")
    cb = H.gpu_book(2, 128)
    got = H.encode_gpu(cb, H.to_device(x, "f32"))
    # zero vectors: nu = 0, y = 0 -> middle threshold (0) sends every code up
    for r in (0, 3):
        assert got["norms"][r] == 0.0 and np.all(got["y"][r] == 0.0)
        assert np.all(got["codes"][r] == np.uint32(0xAAAAAAAA))     # code 2 in every 2-bit slot
    # NaN / Inf: norm and rotated values become NaN, codes and signs are 0
    for r in (1, 2):
        assert np.isnan(got["y"][r]).all() and np.all(got["codes"][r] == 0) and np.all(got["signs"][r] == 0)
    assert np.isnan(got["norms"][1]) and np.isinf(got["norms"][2])
    H.check_encode(x[4:], {k: v[4:] for k, v in got.items()}, 2, 128)


@pytest.mark.parametrize("scale_exp,dt", [(-55, "bf16"), (40, "bf16"), (-58, "f32"), (50, "f32")])
def test_encode_tiny_and_huge_norms(scale_exp, dt):
    # vectors scaled by 2^-55 or 2^-58 (the squared norm, about 2^-103 or
    # 2^-109, lies below the range where the hardware square root is taken
    # directly) and by 2^40 or 2^50; the oracle sees the same stored inputs
    x = np.random.default_rng(11 + abs(scale_exp)).standard_normal((100, 128)).astype(np.float32)
    xs = np.ldexp(x, scale_exp).astype(np.float32)
    _log(f"encode {dt} norms near 2^{scale_exp + 3.5}")
    cb = H.gpu_book(3, 128)
    if dt == "bf16":
        xb = synth.bf16_bits(xs)
        got = H.encode_gpu(cb, H.to_device(xb, "bf16"))
        H.check_encode(H.host_values(xb, "bf16"), got, 3, 128)
    else:
        got = H.encode_gpu(cb, H.to_device(xs, "f32"))
        H.check_encode(xs, got, 3, 128)


@pytest.mark.parametrize("bits,m,dt", [(1, 128, "bf16"), (2, 128, "bf16"), (3, 128, "bf16"), (3, 128, "f32"),
                                        (4, 0, "bf16")])
def test_encode_debug_instantiation_equals_hot_path(bits, m, dt):
    # The launch with debug outputs (y and p kept) is a separate kernel
    # instantiation; its codes, signs and norms must be the hot path's bit for
    # bit over many vectors, including the sign bits whose p lies within
    # rounding of zero (the residual is formed the same way in both).
    n = 1 << 18
    x = torch.randn(n, 128, generator=torch.Generator(device=H.DEV).manual_seed(77 + bits + m), device=H.DEV)
    x = x.to(torch.bfloat16) if dt == "bf16" else x.contiguous()
    cb = H.gpu_book(bits, m)
    _log(f"encode {n} {dt} vectors, bits={bits} m={m}: hot path against the debug instantiation")
    hot = H.encode_gpu(cb, x, debug=False)
    dbg = H.encode_gpu(cb, x, debug=True)
    np.testing.assert_array_equal(hot["codes"], dbg["codes"])
    np.testing.assert_array_equal(hot["norms"].view(np.uint32), dbg["norms"].view(np.uint32))
    if m:
        np.testing.assert_array_equal(hot["signs"], dbg["signs"])
        np.testing.assert_array_equal(hot["res_norms"].view(np.uint32), dbg["res_norms"].view(np.uint32))


def test_encode_dst_row_scatter_skips_out_of_range():
    n, rows = 300, 512
    rng = np.random.default_rng(9)
    x = rng.standard_normal((n, 128)).astype(np.float32)
    dst = rng.permutation(rows)[:n].astype(np.int64)
    dst[5] = -1
    dst[17] = rows           # outside the cache: skipped
    cb = H.gpu_book(2, 128)
    codes = torch.full((rows, cb.code_words), -1, dtype=torch.int32, device=H.DEV)
    norms = torch.full((rows,), -7.0, device=H.DEV)
    signs = torch.full((rows, 4), -1, dtype=torch.int32, device=H.DEV)
    res = torch.full((rows,), -7.0, device=H.DEV)
    dbg = torch.empty(n, 128, device=H.DEV)
    dbgp = torch.empty(n, 128, device=H.DEV)
    T.encode_kv(cb, H.to_device(x, "f32"), codes, norms, signs, res, torch.from_numpy(dst).to(H.DEV), dbg, dbgp)
    torch.cuda.synchronize()
    got = {"codes": H.u32(codes), "norms": norms.cpu().numpy(), "signs": H.u32(signs),
           "res_norms": res.cpu().numpy(), "y": dbg.cpu().numpy(), "p": dbgp.cpu().numpy()}
    keep = np.ones(n, bool)
    keep[[5, 17]] = False
    sub = {"codes": got["codes"], "norms": got["norms"], "signs": got["signs"], "res_norms": got["res_norms"],
           "y": got["y"][keep], "p": got["p"][keep]}
    H.check_encode(x[keep], sub, 2, 128, rows=dst[keep])
    untouched = np.setdiff1d(np.arange(rows), dst[keep])
    assert np.all(got["norms"][untouched] == -7.0) and np.all(got["codes"][untouched] == 0xFFFFFFFF)


def test_encode_is_deterministic_and_idempotent():
    rng = np.random.default_rng(11)
    x = H.to_device(synth.bf16_bits(rng.standard_normal((2000, 128)).astype(np.float32)), "bf16")
    cb = H.gpu_book(3, 128)
    a = H.encode_gpu(cb, x)
    b = H.encode_gpu(cb, x)
    for k in a:
        np.testing.assert_array_equal(a[k].view(np.uint32), b[k].view(np.uint32))


# ------------------------------------------------------------------ decode

def _decode_case(B, Hq, Hkv, t_cap, T_fill, seq_len, kbits, vbits, m, seed, outliers=0, lognormal=None):
    rng = np.random.default_rng(seed)
    oc_k = synth.outlier_channels(rng, Hkv, outliers) if outliers else None
    oc_v = synth.outlier_channels(rng, Hkv, outliers) if outliers else None
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, T_fill, oc_k, lognormal_sigma=lognormal))
    v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, T_fill, oc_v, lognormal_sigma=lognormal))
    q = synth.bf16_bits(rng.standard_normal((B, Hq, 128)).astype(np.float32))
    kcb, vcb = H.gpu_book(kbits, m), H.gpu_book(vbits, 0)
    kc, vc = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, t_cap, T_fill)
    _log(f"decode B={B} Hq={Hq} Hkv={Hkv} t_cap={t_cap} seq={seq_len} kbits={kbits} vbits={vbits} m={m}")
    sl = [min(max(s, 0), t_cap) for s in seq_len]
    return H.check_decode(kcb, vcb, H.to_device(q, "bf16"), kc, vc, seq_len, kbits, vbits, m) if sl == seq_len else \
        (kcb, vcb, H.to_device(q, "bf16"), kc, vc)


def test_decode_tiny_config():
    wl = synth.tiny()
    kcb, vcb = H.gpu_book(2, 128), H.gpu_book(2, 0)
    k = H.to_device(wl.k.reshape(-1, 128), "f32")
    v = H.to_device(wl.k.reshape(-1, 128), "f32")     # the tiny config has keys only; values reuse them
    kc, vc = H.build_cache(kcb, vcb, k.reshape(1, 1, 4096, 128), v.reshape(1, 1, 4096, 128), 1, 1, 4096, 4096)
    _log("decode tiny")
    H.check_decode(kcb, vcb, H.to_device(wl.q, "f32"), kc, vc, [4096], 2, 2, 128)


@pytest.mark.parametrize("kbits,vbits,m,g", [(2, 3, 128, 4), (2, 2, 128, 8), (1, 1, 128, 4), (3, 4, 128, 4),
                                             (2, 3, 0, 4), (3, 2, 128, 1), (1, 4, 128, 2), (2, 1, 128, 8),
                                             # MSE-only keys (no QJL) at every width
                                             (1, 2, 0, 8), (3, 3, 0, 2), (4, 4, 0, 4), (2, 2, 0, 1),
                                             # 3-bit keys through the code-pair table (g = 2, 4)
                                             (3, 1, 128, 2), (3, 2, 0, 4)])
def test_decode_bit_widths_and_gqa(kbits, vbits, m, g):
    _decode_case(2, 4 * g, 4, 1300, 1300, [1300, 777], kbits, vbits, m, seed=kbits * 10 + vbits + g, outliers=4)


def test_decode_ragged_lengths_and_empty():
    _decode_case(5, 8, 2, 1031, 1031, [0, 1, 255, 257, 1031], 2, 3, 128, seed=5, lognormal=0.5)


def test_decode_llama8b_shape_short():
    _decode_case(1, 32, 8, 4096, 4096, [4096], 2, 3, 128, seed=21, outliers=4)


def test_decode_seq_len_clamped_to_capacity():
    kcb, vcb, q, kc, vc = _decode_case(2, 8, 2, 300, 300, [400, -3], 2, 2, 128, seed=3)
    sl = torch.tensor([400, -3], dtype=torch.int32, device=H.DEV)
    a = T.decode_attention(kcb, vcb, q, kc, vc, sl)
    b = T.decode_attention(kcb, vcb, q, kc, vc, torch.tensor([300, 0], dtype=torch.int32, device=H.DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
    assert np.all(a[1].cpu().numpy() == 0.0)


def test_decode_single_chunk_rows_write_output_in_kernel():
    # Caches of <= 256 tokens are one token chunk per row: the main kernel writes the
    # output itself (no merge launch). Oracle parity, and agreement with the same tokens
    # in a longer cache that splits into several chunks and merges them.
    B, Hkv, g, T_fill = 3, 2, 4, 200
    rng = np.random.default_rng(44)
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, T_fill, synth.outlier_channels(rng, Hkv, 4)))
    v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, T_fill))
    q = H.to_device(synth.bf16_bits(rng.standard_normal((B, Hkv * g, 128)).astype(np.float32)), "bf16")
    kcb, vcb = H.gpu_book(2, 128), H.gpu_book(3, 0)
    seq = [200, 57, 0]
    _log(f"decode single chunk: B={B} Hkv={Hkv} g={g} t_cap={T_fill} seq={seq}")
    kc, vc = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, T_fill, T_fill)
    H.check_decode(kcb, vcb, q, kc, vc, seq, 2, 3, 128)
    kl, vl = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, 1200, T_fill)
    sl = torch.tensor(seq, dtype=torch.int32, device=H.DEV)
    one = T.decode_attention(kcb, vcb, q, kc, vc, sl)
    many = T.decode_attention(kcb, vcb, q, kl, vl, sl)
    torch.cuda.synchronize()
    np.testing.assert_allclose(one.cpu().numpy(), many.cpu().numpy(), rtol=1e-5, atol=1e-6)
