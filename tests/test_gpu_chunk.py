"""tq_chunk_attention: a chunk of n_new queries per (b, q head), query j at
position seq_len - n_new + j attending causally over the compressed cache.

* Oracle parity (chunk_attention) at g = 1, 2, 4, 8, n_new = 1 .. 24, keys
  with and without QJL, bf16 and fp32 queries, over ragged sequences, one
  shorter than the chunk (its first queries see nothing and give zeros); both
  the decode-kernel path (< 16 query rows per kv head) and the matrix-core
  path, including its padded row blocks (g = 1, 16 rows).
* Query j equals tq_decode_attention of that query alone with
  seq_len - n_new + j + 1 tokens: bit for bit for n_new = 1 (same launch
  plan); within 1e-5 relative and absolute while fewer than 16 query rows per
  kv head run through the decode kernel (longer token chunks add the partial
  sums in another order); within the 2e-3 output bar on the matrix-core path,
  whose bf16 hi/lo score operands carry about 1e-5 relative error into the
  logits (observed 3e-5 .. 6e-5 at these sizes, 5.6e-4 at the full 8B layer,
  whose outlier channels make large logits).
* Full size: 8 queries per head (32 rows per kv head: the matrix-core path)
  over the Llama-3-8B-shaped layer (32768 tokens): every query against the
  single-query decode, two against the oracle; and the batched workload's
  shape (16 x 8 x 8192, ragged lengths, 4 queries per head): every query
  against the single-query decode, two sequences against the oracle.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
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


def _per_query_decode(kcb, vcb, q, kc, vc, lens):
    """Each query of the chunk through tq_decode_attention alone."""
    B, Hq, n_new, d = q.shape
    outs = []
    for j in range(n_new):
        sl = torch.tensor([ln - n_new + j + 1 for ln in lens], dtype=torch.int32, device=H.DEV)
        outs.append(T.decode_attention(kcb, vcb, q[:, :, j].contiguous(), kc, vc, sl))
    return torch.stack(outs, dim=2)


@pytest.mark.parametrize("kbits,m,vbits,g,n_new,qdt", [(2, 128, 3, 4, 5, "bf16"), (1, 128, 2, 8, 16, "bf16"),
                                                       (3, 128, 4, 1, 1, "bf16"), (2, 0, 2, 4, 16, "bf16"),
                                                       (4, 0, 3, 8, 5, "bf16"), (2, 128, 3, 1, 16, "f32"),
                                                       (3, 128, 2, 2, 24, "f32"), (4, 128, 4, 2, 3, "f32"),
                                                       (3, 128, 2, 4, 3, "bf16"), (3, 0, 3, 2, 5, "f32")])
def test_chunk_parity(kbits, m, vbits, g, n_new, qdt):
    B, Hkv, t_cap = 3, 2, 1100
    lens = [1100, 3, 640]
    Hq = Hkv * g
    rng = np.random.default_rng(1000 + 10 * kbits + g + n_new)
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap, lognormal_sigma=0.5))
    v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap, lognormal_sigma=0.5))
    qf = rng.standard_normal((B, Hq, n_new, 128)).astype(np.float32)
    q = H.to_device(synth.bf16_bits(qf), "bf16") if qdt == "bf16" else H.to_device(qf, "f32")
    kcb, vcb = H.gpu_book(kbits, m), H.gpu_book(vbits, 0)
    kc, vc = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, t_cap, t_cap)
    sl = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    _log(f"chunk kbits={kbits} m={m} vbits={vbits} g={g} n_new={n_new} q={qdt} lens={lens}")
    got = T.chunk_attention(kcb, vcb, q, kc, vc, sl)
    per = _per_query_decode(kcb, vcb, q, kc, vc, lens)
    torch.cuda.synchronize()
    g_np = got.cpu().numpy()
    p_np = per.cpu().numpy()
    _log(f"  vs single-query decode: max-abs {np.abs(g_np - p_np).max():.2e} (max |o| {np.abs(p_np).max():.2e})")
    if n_new == 1:
        np.testing.assert_array_equal(g_np.view(np.uint32), p_np.view(np.uint32))
    elif not T.api.chunk_uses_mfma(g, n_new):
        np.testing.assert_allclose(g_np, p_np, rtol=1e-5, atol=1e-5)
    else:   # both sides within the 2e-3 output bar of the oracle; observed 3e-5 .. 6e-5 here
        np.testing.assert_allclose(g_np, p_np, rtol=0, atol=2e-3)
    ref = O.chunk_attention(q.float().cpu().numpy().astype(np.float64), H.cache_to_host(kc), H.cache_to_host(vc),
                            lens, H.oracle_book(kbits, m), H.oracle_book(vbits, 0))
    err = np.abs(g_np - ref).max()
    _log(f"  vs oracle: max-abs {err:.2e}")
    assert err <= 2e-3, f"max-abs error {err:.3e}"
    # the short sequence: queries 0 .. n_new - 4 see no token
    empty = max(0, n_new - 3)
    assert np.all(g_np[1, :, :empty] == 0.0)


@pytest.mark.parametrize("exp2,qdt", [(60, "bf16"), (-60, "bf16"), (40, "f32"), (-40, "f32")])
def test_chunk_query_magnitude_extremes(exp2, qdt):
    """The matrix-core tiles scale each query row by a power of two into fp16
    range before the query rotation: queries 2^+-60 (bf16) and 2^+-40 (fp32)
    give finite outputs within the oracle's bar (near one-hot softmax for the
    large ones, near uniform for the small ones)."""
    B, Hkv, g, n_new, t = 1, 2, 4, 16, 700
    Hq = Hkv * g
    rng = np.random.default_rng(5151 + abs(exp2) + (qdt == "f32"))
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t))
    v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t))
    qf = (rng.standard_normal((B, Hq, n_new, 128)) * 2.0 ** exp2).astype(np.float32)
    q = H.to_device(synth.bf16_bits(qf), "bf16") if qdt == "bf16" else H.to_device(qf, "f32")
    kcb, vcb = H.gpu_book(2, 128), H.gpu_book(3, 0)
    assert T.api.chunk_uses_mfma(g, n_new)
    kc, vc = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, t, t)
    lens = [t]
    sl = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    _log(f"chunk with queries of magnitude 2^{exp2} ({qdt})")
    got = T.chunk_attention(kcb, vcb, q, kc, vc, sl)
    torch.cuda.synchronize()
    g_np = got.cpu().numpy()
    assert np.all(np.isfinite(g_np)), "non-finite outputs"
    ref = O.chunk_attention(q.float().cpu().numpy().astype(np.float64), H.cache_to_host(kc), H.cache_to_host(vc),
                            lens, H.oracle_book(2, 128), H.oracle_book(3, 0))
    err = np.abs(g_np - ref).max()
    _log(f"  vs oracle: max-abs {err:.2e}")
    assert err <= 2e-3, f"max-abs error {err:.3e}"


def test_chunk_bf16_output_and_determinism():
    B, Hkv, g, n_new, t_cap = 2, 2, 4, 7, 900
    rng = np.random.default_rng(5)
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap))
    v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap))
    q = H.to_device(synth.bf16_bits(rng.standard_normal((B, Hkv * g, n_new, 128)).astype(np.float32)), "bf16")
    kcb, vcb = H.gpu_book(2, 128), H.gpu_book(3, 0)
    kc, vc = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, t_cap, t_cap)
    sl = torch.tensor([900, 450], dtype=torch.int32, device=H.DEV)
    o32 = T.chunk_attention(kcb, vcb, q, kc, vc, sl)
    o32b = T.chunk_attention(kcb, vcb, q, kc, vc, sl)
    o16 = T.chunk_attention(kcb, vcb, q, kc, vc, sl, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    a = o32.cpu().numpy()
    np.testing.assert_array_equal(a.view(np.uint32), o32b.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(o16.float().cpu().numpy(), H.rne_bf16(a))


def test_chunk_llama8b_full():
    wl = synth.llama8b()
    S, n_new = wl.seq_len, 8
    _log(f"{wl.name}: {n_new} causal queries per head over {S} tokens")
    kcb, vcb = H.gpu_book(2, 128), H.gpu_book(3, 0)
    kc = T.CompressedCache.allocate(kcb, 1, 8, S)
    vc = T.CompressedCache.allocate(vcb, 1, 8, S)
    T.encode_into_cache(kcb, H.to_device(wl.k.reshape(-1, 128), "bf16"), kc)
    T.encode_into_cache(vcb, H.to_device(wl.v.reshape(-1, 128), "bf16"), vc)
    rng = np.random.default_rng(8)
    q = H.to_device(synth.bf16_bits(rng.standard_normal((1, 32, n_new, 128)).astype(np.float32)), "bf16")
    sl = torch.tensor([S], dtype=torch.int32, device=H.DEV)
    got = T.chunk_attention(kcb, vcb, q, kc, vc, sl)
    per = _per_query_decode(kcb, vcb, q, kc, vc, [S])
    torch.cuda.synchronize()
    g_np = got.cpu().numpy()
    _log(f"  vs single-query decode: max-abs {np.abs(g_np - per.cpu().numpy()).max():.2e}")
    np.testing.assert_allclose(g_np, per.cpu().numpy(), rtol=0, atol=2e-3)
    q_host = q.float().cpu().numpy().astype(np.float64)
    kh, vh = H.cache_to_host(kc), H.cache_to_host(vc)
    for j in (0, n_new - 1):
        ref = O.decode_attention(q_host[:, :, j], kh, vh, [S - n_new + j + 1], H.oracle_book(2, 128),
                                 H.oracle_book(3, 0))
        err = np.abs(g_np[:, :, j] - ref).max()
        _log(f"  query {j}: max-abs error {err:.2e}")
        assert err <= 2e-3


def test_chunk_batched_full():
    """The batched workload's shape (16 sequences x 8 kv heads x 8192 tokens,
    32 q heads) with 4 new queries per head: 16 rows per kv head, the
    matrix-core path, ragged lengths."""
    wl = synth.batched(2)
    B, Hkv, S = wl.batch, wl.n_kv_heads, wl.seq_len
    n_new = 4
    _log(f"{wl.name}: {n_new} causal queries per head, ragged lengths")
    kcb, vcb = H.gpu_book(1, 128), H.gpu_book(2, 0)
    kc, vc = H.build_cache(kcb, vcb, H.to_device(wl.k, "bf16"), H.to_device(wl.v, "bf16"), B, Hkv, S, S)
    rng = np.random.default_rng(12)
    q = H.to_device(synth.bf16_bits(rng.standard_normal((B, 32, n_new, 128)).astype(np.float32)), "bf16")
    lens = [S - 301 * b for b in range(B)]
    sl = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    got = T.chunk_attention(kcb, vcb, q, kc, vc, sl)
    per = _per_query_decode(kcb, vcb, q, kc, vc, lens)
    torch.cuda.synchronize()
    g_np = got.cpu().numpy()
    diff = np.abs(g_np - per.cpu().numpy()).max()
    _log(f"  vs single-query decode: max-abs {diff:.2e}")
    assert diff <= 2e-3
    # two sequences against the oracle
    kh, vh = H.cache_to_host(kc), H.cache_to_host(vc)
    q_host = q.float().cpu().numpy().astype(np.float64)
    for b in (0, B - 1):
        sub = lambda c: {k: (None if v is None else v[b:b + 1]) for k, v in c.items()}
        ref = O.chunk_attention(q_host[b:b + 1], sub(kh), sub(vh), [lens[b]], H.oracle_book(1, 128),
                                H.oracle_book(2, 0))
        err = np.abs(g_np[b:b + 1] - ref).max()
        _log(f"  sequence {b}: max-abs error vs oracle {err:.2e}")
        assert err <= 2e-3


def test_chunk_decode_kernel_wide_batch():
    # 40 sequences x 16 kv heads x 7 queries (g = 1: the decode kernel, 4,480
    # query rows in the grid's y and z) over ragged windows.  Oracle parity at
    # the 2e-3 bar.
    B, Hkv, g, n_new, t_cap = 40, 16, 1, 7, 80
    rng = np.random.default_rng(91)
    lens = [int(x) for x in rng.integers(n_new, t_cap + 1, size=B)]
    lens[0] = 3   # its first queries see nothing
    Hq = Hkv * g
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap, lognormal_sigma=0.5))
    v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap, lognormal_sigma=0.5))
    q = H.to_device(synth.bf16_bits(rng.standard_normal((B, Hq, n_new, 128)).astype(np.float32)), "bf16")
    kcb, vcb = H.gpu_book(2, 128), H.gpu_book(3, 0)
    kc, vc = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, t_cap, t_cap)
    sl = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    _log(f"chunk two-launch merge: B={B} Hkv={Hkv} n_new={n_new} t_cap={t_cap}")
    got = T.chunk_attention(kcb, vcb, q, kc, vc, sl)
    torch.cuda.synchronize()
    g_np = got.cpu().numpy()
    ref = O.chunk_attention(q.float().cpu().numpy().astype(np.float64), H.cache_to_host(kc), H.cache_to_host(vc),
                            lens, H.oracle_book(2, 128), H.oracle_book(3, 0))
    err = np.abs(g_np - ref).max()
    _log(f"  vs oracle: max-abs {err:.2e}")
    assert err <= 2e-3, f"max-abs error {err:.3e}"
    assert np.all(g_np[0, :, :n_new - 3] == 0.0)


@pytest.mark.parametrize("qdt", ["bf16", "f32"])
def test_chunk_mfma_query_4byte_aligned(qdt):
    """The matrix-core path reads the queries in its own prologue; the call
    promises only 4-byte alignment of q, so a query tensor starting 4 bytes
    past a 16-byte boundary must give the same result, bit for bit, as an
    aligned copy of it."""
    B, Hkv, g, n_new, t_cap = 2, 2, 4, 8, 600
    rng = np.random.default_rng(77)
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap))
    v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap))
    qf = rng.standard_normal((B, Hkv * g, n_new, 128)).astype(np.float32)
    q = H.to_device(synth.bf16_bits(qf), "bf16") if qdt == "bf16" else H.to_device(qf, "f32")
    assert T.api.chunk_uses_mfma(g, n_new)
    kcb, vcb = H.gpu_book(2, 128), H.gpu_book(3, 0)
    kc, vc = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, t_cap, t_cap)
    sl = torch.tensor([600, 333], dtype=torch.int32, device=H.DEV)
    shift = 4 // q.element_size()
    buf = torch.empty(q.numel() + shift, dtype=q.dtype, device=H.DEV)
    q_off = buf[shift:].view(q.shape)
    q_off.copy_(q)
    assert q_off.data_ptr() % 16 == 4
    _log(f"chunk, query at a 4-byte offset: q={qdt}")
    a = T.chunk_attention(kcb, vcb, q, kc, vc, sl)
    b = T.chunk_attention(kcb, vcb, q_off, kc, vc, sl)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))
