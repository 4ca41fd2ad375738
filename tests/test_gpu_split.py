"""Split bit widths on the GPU (rotated coordinates 0..63 on the (b'+1)-bit
codebook, 64..127 on the b'-bit one): encode, single-query decode, attention
logits and the decode-loop step against the oracle's split functions, at
small ragged sizes and at the Llama-3-8B-shaped layer; unsupported reads are
refused.  Bars as in the uniform tests: codes, signs and packing bit-exact on
the GPU's own fp32 rotated values and projections; scores within 1e-4
relative; outputs within 2e-3 max-abs; logits bit-equal to the decode's own."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from online_vector_quantization_amd import synth  # noqa: E402

import gpu_helpers as H  # noqa: E402
import online_vector_quantization_amd as T  # noqa: E402

WIDE = 64


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch sees no GPU")
    T.load_library()


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("bits,m,dtype", [(1, 128, "bf16"), (2, 128, "bf16"), (3, 128, "bf16"), (2, 128, "f32"),
                                          (1, 0, "bf16"), (2, 0, "bf16"), (3, 0, "f32")])
def test_split_encode(bits, m, dtype):
    n = 2085   # several tiles and a ragged tail
    rng = np.random.default_rng(300 + 10 * bits + m)
    x = synth.kv_block(rng, 1, 1, n, synth.outlier_channels(rng, 1, 4))[0, 0]
    x = synth.bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)
    _log(f"split encode bits={bits} m={m} dtype={dtype} n={n}")
    cb = H.gpu_book(bits, m, WIDE)
    assert cb.code_words == (128 * bits + WIDE) // 32
    got = H.encode_gpu(cb, H.to_device(x, dtype))
    flips = H.check_encode(H.host_values(x, dtype), got, bits, m, wide=WIDE)
    assert flips <= 1e-3 * n * 256
    # without debug outputs: the same records
    plain = H.encode_gpu(cb, H.to_device(x, dtype), debug=False)
    np.testing.assert_array_equal(plain["codes"], got["codes"])
    if m:
        np.testing.assert_array_equal(plain["signs"], got["signs"])


@pytest.mark.parametrize("kbits,vbits,m,g", [(2, 3, 128, 4), (1, 2, 128, 8), (3, 1, 128, 2), (2, 2, 0, 1),
                                             (3, 3, 0, 4)])
def test_split_decode_parity(kbits, vbits, m, g):
    B, Hkv, t_cap = 3, 2, 1300
    lens = [1300, 1, 777]
    rng = np.random.default_rng(400 + 10 * kbits + vbits + g)
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap, synth.outlier_channels(rng, Hkv, 4)))
    v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap, lognormal_sigma=0.5))
    q = H.to_device(synth.bf16_bits(rng.standard_normal((B, Hkv * g, 128)).astype(np.float32)), "bf16")
    _log(f"split decode kbits={kbits} vbits={vbits} m={m} g={g} lens={lens}")
    kcb, vcb = H.gpu_book(kbits, m, WIDE), H.gpu_book(vbits, 0, WIDE)
    kc, vc = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, t_cap, t_cap)
    err = H.check_decode(kcb, vcb, q, kc, vc, lens, kbits, vbits, m, wide=WIDE)
    _log(f"  max-abs error {err:.2e}")
    # logits: the decode's own l_t, bit for bit, and the oracle's
    sl = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    got = T.attention_logits(kcb, q, kc, sl, logits=torch.full((B, Hkv * g, t_cap), float("nan"), device=H.DEV))
    dbg = torch.full((B, Hkv * g, t_cap), float("nan"), device=H.DEV)
    T.decode_attention(kcb, vcb, q, kc, vc, sl, dbg_scores=dbg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), dbg.cpu().numpy().view(np.uint32))
    ref = H.oracle_logits(q.float().cpu().numpy().astype(np.float64), H.cache_to_host(kc), lens,
                          H.oracle_book(kbits, m, wide=WIDE), g)
    H.check_logits(got.cpu().numpy(), ref, lens)


def test_split_append_decode_steps():
    """Decode-loop steps with split codebooks equal encode-then-decode of the
    grown cache, bit for bit, and the oracle."""
    B, Hkv, g, t_cap, S, steps = 2, 2, 4, 520, 509, 3
    rng = np.random.default_rng(450)
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, S))
    v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, S))
    kcb, vcb = H.gpu_book(2, 128, WIDE), H.gpu_book(3, 0, WIDE)
    kc, vc = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, t_cap, S)
    kc2, vc2 = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, t_cap, S)
    sl = torch.tensor([S, S - 100], dtype=torch.int32, device=H.DEV)
    for step in range(steps):
        kn = H.to_device(synth.bf16_bits(rng.standard_normal((B, Hkv, 128)).astype(np.float32)), "bf16")
        vn = H.to_device(synth.bf16_bits(rng.standard_normal((B, Hkv, 128)).astype(np.float32)), "bf16")
        q = H.to_device(synth.bf16_bits(rng.standard_normal((B, Hkv * g, 128)).astype(np.float32)), "bf16")
        _log(f"split append step {step}")
        before = sl.cpu().numpy().copy()
        out = T.append_decode(kcb, vcb, kn, vn, q, kc, vc, sl)
        # reference: encode the new rows at seq_len, then decode seq_len + 1
        rows = torch.tensor([(b * Hkv + h) * t_cap + int(before[b]) for b in range(B) for h in range(Hkv)],
                            dtype=torch.int64, device=H.DEV)
        T.encode_into_cache(kcb, kn.reshape(-1, 128), kc2, dst_row=rows)
        T.encode_into_cache(vcb, vn.reshape(-1, 128), vc2, dst_row=rows)
        ref = T.decode_attention(kcb, vcb, q, kc2, vc2, torch.tensor(before + 1, dtype=torch.int32, device=H.DEV))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(sl.cpu().numpy(), before + 1)
        np.testing.assert_array_equal(H.u32(kc.codes), H.u32(kc2.codes))
        np.testing.assert_array_equal(H.u32(vc.codes), H.u32(vc2.codes))
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))
    H.check_decode(kcb, vcb, q, kc, vc, list(sl.cpu().numpy()), 2, 3, 128, wide=WIDE)


def test_split_unsupported_reads_are_refused():
    B, Hkv, g = 1, 2, 4
    kcb, vcb = H.gpu_book(2, 128, WIDE), H.gpu_book(3, 0, WIDE)
    vu = H.gpu_book(3, 0)
    q = torch.zeros(B, Hkv * g, 128, dtype=torch.bfloat16, device=H.DEV)
    sl = torch.tensor([8], dtype=torch.int32, device=H.DEV)
    kc, vc = T.CompressedCache.allocate(kcb, B, Hkv, 16), T.CompressedCache.allocate(vcb, B, Hkv, 16)
    vcu = T.CompressedCache.allocate(vu, B, Hkv, 16)
    with pytest.raises(T.TQError) as e:       # keys split, values uniform
        T.decode_attention(kcb, vu, q, kc, vcu, sl)
    assert e.value.status == T.api.TQ_ERR_UNSUPPORTED
    kc3, vc3 = T.CompressedCache.allocate(kcb, B, Hkv, 15), T.CompressedCache.allocate(vcb, B, Hkv, 15)
    with pytest.raises(T.TQError) as e:       # t_cap not a multiple of 4
        T.decode_attention(kcb, vcb, q, kc3, vc3, sl)
    assert e.value.status == T.api.TQ_ERR_UNSUPPORTED
    qc = torch.zeros(B, Hkv * g, 4, 128, dtype=torch.bfloat16, device=H.DEV)
    with pytest.raises(T.TQError) as e:       # a chunk of several queries
        T.chunk_attention(kcb, vcb, qc, kc, vc, sl)
    assert e.value.status == T.api.TQ_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_split_llama8b_layer_full():
    """The Llama-3-8B-shaped layer at 3.5 bits per key coordinate (2.5-bit
    codes + 1-bit QJL) and 3.5-bit values: every record and the full decode."""
    wl = synth.llama8b()
    _log(f"{wl.name} split widths: encode all rows, then decode")
    kcb, vcb = H.gpu_book(2, 128, WIDE), H.gpu_book(3, 0, WIDE)
    for cb, arr, bits, m in ((kcb, wl.k, 2, 128), (vcb, wl.v, 3, 0)):
        x = arr.reshape(-1, 128)
        got = H.encode_gpu(cb, H.to_device(x, "bf16"))
        flips = H.check_encode(H.host_values(x, "bf16"), got, bits, m, wide=WIDE)
        _log(f"  bits={bits}+{WIDE} wide m={m}: near-boundary flips vs float64 oracle {flips}")
    kc = T.CompressedCache.allocate(kcb, 1, 8, wl.seq_len)
    vc = T.CompressedCache.allocate(vcb, 1, 8, wl.seq_len)
    T.encode_into_cache(kcb, H.to_device(wl.k.reshape(-1, 128), "bf16"), kc)
    T.encode_into_cache(vcb, H.to_device(wl.v.reshape(-1, 128), "bf16"), vc)
    err = H.check_decode(kcb, vcb, H.to_device(wl.q, "bf16"), kc, vc, [wl.seq_len], 2, 3, 128, wide=WIDE)
    _log(f"  decode max-abs error {err:.2e}")


def test_split_edge_cases():
    """Split widths at the smallest row (t_cap = 4), empty and full sequences,
    g = 8, fp32 queries, bf16 output (the RNE rounding of the fp32 output), and
    the allocation-free entry point (bit-equal to the workspace one)."""
    rng = np.random.default_rng(460)
    for (B, Hkv, g, t_cap, lens, qdt) in ((2, 1, 8, 4, [4, 0], "f32"), (3, 2, 2, 8, [0, 8, 3], "bf16")):
        k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap))
        v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap))
        qf = rng.standard_normal((B, Hkv * g, 128)).astype(np.float32)
        q = H.to_device(qf if qdt == "f32" else synth.bf16_bits(qf), qdt)
        _log(f"split edge B={B} Hkv={Hkv} g={g} t_cap={t_cap} lens={lens} q={qdt}")
        kcb, vcb = H.gpu_book(1, 128, WIDE), H.gpu_book(2, 0, WIDE)
        kc, vc = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, t_cap, t_cap)
        H.check_decode(kcb, vcb, q, kc, vc, lens, 1, 2, 128, wide=WIDE)
        sl = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
        a = T.decode_attention(kcb, vcb, q, kc, vc, sl)
        s = T.decode_attention_static(kcb, vcb, q, kc, vc, sl)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(a.cpu().numpy().view(np.uint32), s.cpu().numpy().view(np.uint32))
        for b, L in enumerate(lens):
            if L == 0:
                assert np.all(a[b].cpu().numpy() == 0.0)
