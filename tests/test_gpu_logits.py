"""tq_attention_logits: the scaled logits of every cached key, without the
softmax and the value sum.

* Oracle parity (decode_scores per (b, q head)) at every key width, with and
  without the QJL sign bits, at g = 1, 2, 4, 8, over caches of several
  work-group chunks with ragged, empty and full sequences; entries past
  seq_len are not written.
* Bit-equal to the l_t that tq_decode_attention reports for the same inputs.
* Full sizes: the Llama-3-8B-shaped layer (32768 tokens, 32 q heads) and the
  batched workload (16 x 8 x 8192, b = 2), every logit checked.
"""
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


def _nan_logits(B, Hq, t_cap):
    return torch.full((B, Hq, t_cap), float("nan"), dtype=torch.float32, device=H.DEV)


@pytest.mark.parametrize("kbits,m,g", [(1, 128, 4), (2, 128, 8), (3, 128, 2), (4, 128, 1),
                                       (1, 0, 2), (2, 0, 4), (3, 0, 8), (4, 0, 1), (3, 128, 4), (3, 0, 4)])
def test_logits_parity(kbits, m, g):
    B, Hkv, t_cap = 4, 2, 1300
    lens = [1300, 0, 777, 5]
    Hq = Hkv * g
    rng = np.random.default_rng(100 * kbits + 10 * g + (m > 0))
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap, lognormal_sigma=0.5))
    v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap, lognormal_sigma=0.5))
    q = H.to_device(synth.bf16_bits(rng.standard_normal((B, Hq, 128)).astype(np.float32)), "bf16")
    kcb, vcb = H.gpu_book(kbits, m), H.gpu_book(2, 0)
    kc, vc = H.build_cache(kcb, vcb, H.to_device(k, "bf16"), H.to_device(v, "bf16"), B, Hkv, t_cap, t_cap)
    sl = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    _log(f"logits kbits={kbits} m={m} g={g} lens={lens}")
    got = T.attention_logits(kcb, q, kc, sl, logits=_nan_logits(B, Hq, t_cap))
    dbg = _nan_logits(B, Hq, t_cap)
    T.decode_attention(kcb, vcb, q, kc, vc, sl, dbg_scores=dbg)
    torch.cuda.synchronize()
    g_np = got.cpu().numpy()
    # the decode's own logits, bit for bit (NaN sentinels included)
    np.testing.assert_array_equal(g_np.view(np.uint32), dbg.cpu().numpy().view(np.uint32))
    ref = H.oracle_logits(q.float().cpu().numpy().astype(np.float64), H.cache_to_host(kc), lens,
                          H.oracle_book(kbits, m), g)
    H.check_logits(g_np, ref, lens)


def test_logits_scale_and_seq_clamp():
    """softmax_scale scales every logit; seq_len beyond t_cap is clamped and
    a negative one reads as empty; fp32 queries."""
    B, Hkv, g, t_cap = 3, 1, 4, 700
    rng = np.random.default_rng(9)
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap))
    q = H.to_device(synth.bf16_bits(rng.standard_normal((B, Hkv * g, 128)).astype(np.float32)), "bf16")
    kcb = H.gpu_book(2, 128)
    kc = T.CompressedCache.allocate(kcb, B, Hkv, t_cap)
    T.encode_into_cache(kcb, H.to_device(k.reshape(-1, 128), "bf16"), kc)
    sl = torch.tensor([10_000, -3, 333], dtype=torch.int32, device=H.DEV)
    got = T.attention_logits(kcb, q, kc, sl, logits=_nan_logits(B, Hkv * g, t_cap), softmax_scale=0.5)
    # an fp32 query (values not representable in bf16)
    q32 = torch.from_numpy(rng.standard_normal((B, Hkv * g, 128)).astype(np.float32)).to(H.DEV)
    got32 = T.attention_logits(kcb, q32, kc, sl, logits=_nan_logits(B, Hkv * g, t_cap))
    torch.cuda.synchronize()
    seq_c = [t_cap, 0, 333]
    ref = H.oracle_logits(q.float().cpu().numpy().astype(np.float64), H.cache_to_host(kc), seq_c,
                          H.oracle_book(2, 128), g, scale=0.5)
    H.check_logits(got.cpu().numpy(), ref, seq_c)
    ref32 = H.oracle_logits(q32.cpu().numpy().astype(np.float64), H.cache_to_host(kc), seq_c, H.oracle_book(2, 128), g)
    H.check_logits(got32.cpu().numpy(), ref32, seq_c)


def test_logits_llama8b_full():
    wl = synth.llama8b()
    S = wl.seq_len
    _log(f"{wl.name}: logits of all {S} tokens x 32 q heads")
    kcb = H.gpu_book(2, 128)
    kc = T.CompressedCache.allocate(kcb, 1, 8, S)
    T.encode_into_cache(kcb, H.to_device(wl.k.reshape(-1, 128), "bf16"), kc)
    q = H.to_device(wl.q, "bf16")
    sl = torch.tensor([S], dtype=torch.int32, device=H.DEV)
    ws = T.alloc_workspace(1, 32, 8, S, H.DEV)
    got = T.attention_logits(kcb, q, kc, sl, logits=_nan_logits(1, 32, S), workspace=ws)
    torch.cuda.synchronize()
    ref = H.oracle_logits(q.float().cpu().numpy().astype(np.float64), H.cache_to_host(kc), [S],
                          H.oracle_book(2, 128), 4)
    worst = H.check_logits(got.cpu().numpy(), ref, [S])
    _log(f"  worst relative error {worst:.2e}")


def test_logits_batched_full():
    wl = synth.batched(2)
    B, Hkv, S = wl.batch, wl.n_kv_heads, wl.seq_len
    _log(f"{wl.name}: logits of {B} x {Hkv} x {S} keys, 32 q heads")
    kcb = H.gpu_book(1, 128)
    kc = T.CompressedCache.allocate(kcb, B, Hkv, S)
    T.encode_into_cache(kcb, H.to_device(wl.k.reshape(-1, 128), "bf16"), kc)
    q = H.to_device(wl.q, "bf16")
    lens = [S - 37 * b for b in range(B)]
    sl = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    got = T.attention_logits(kcb, q, kc, sl, logits=_nan_logits(B, 32, S))
    torch.cuda.synchronize()
    ref = H.oracle_logits(q.float().cpu().numpy().astype(np.float64), H.cache_to_host(kc), lens,
                          H.oracle_book(1, 128), 4)
    worst = H.check_logits(got.cpu().numpy(), ref, lens)
    _log(f"  worst relative error {worst:.2e}")


@pytest.mark.parametrize("kbits,g,qdt", [(2, 8, "bf16"), (3, 8, "f32"), (3, 4, "bf16"), (4, 8, "bf16"), (2, 4, "f32")])
def test_logits_precision_margin(kbits, g, qdt):
    """The query products keep fp32-level precision on both decode kernels
    (the matrix cores at g = 8 and at g = 4 with 3-bit codes, the vector ALU at
    g = 4 with 2-bit codes): worst relative logit error at most 2e-6, fifty
    times inside the 1e-4 bar.  Observed 3e-7 .. 5e-7; products with 16-bit
    (bf16 hi/lo) operands give 4.5e-6 .. 1e-5 here."""
    B, Hkv, t = 2, 2, 1536
    Hq = Hkv * g
    rng = np.random.default_rng(7 + kbits + g)
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t, lognormal_sigma=0.5))
    qf = rng.standard_normal((B, Hq, 128)).astype(np.float32) * 3
    q = H.to_device(synth.bf16_bits(qf), "bf16") if qdt == "bf16" else H.to_device(qf, "f32")
    kcb = H.gpu_book(kbits, 128)
    kc = T.CompressedCache.allocate(kcb, B, Hkv, t)
    T.encode_into_cache(kcb, H.to_device(k.reshape(-1, 128), "bf16"), kc)
    lens = [t, t - 100]
    sl = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    _log(f"logits precision kbits={kbits} g={g} q={qdt}")
    got = T.attention_logits(kcb, q, kc, sl, logits=_nan_logits(B, Hq, t))
    torch.cuda.synchronize()
    ref = H.oracle_logits(q.float().cpu().numpy().astype(np.float64), H.cache_to_host(kc), lens,
                          H.oracle_book(kbits, 128), g)
    worst = H.check_logits(got.cpu().numpy(), ref, lens)
    _log(f"  worst relative error {worst:.2e}")
    assert worst <= 2e-6, f"relative logit error {worst:.3e}"


@pytest.mark.parametrize("exp2,qdt", [(-60, "bf16"), (60, "bf16"), (-40, "f32"), (40, "f32")])
def test_logits_query_magnitude_extremes(exp2, qdt):
    """The matrix-core decode scales each head's query by a power of two into
    fp16 range before its products: queries 2^+-60 (bf16) and 2^+-40 (fp32)
    give the oracle's logits to the same relative bar, with no overflow or
    flush to zero (g = 8, 2-bit codes + QJL)."""
    B, Hkv, g, t = 1, 2, 8, 700
    Hq = Hkv * g
    rng = np.random.default_rng(4242 + exp2)
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t))
    qf = (rng.standard_normal((B, Hq, 128)) * 2.0 ** exp2).astype(np.float32)
    q = H.to_device(synth.bf16_bits(qf), "bf16") if qdt == "bf16" else H.to_device(qf, "f32")
    kcb = H.gpu_book(2, 128)
    kc = T.CompressedCache.allocate(kcb, B, Hkv, t)
    T.encode_into_cache(kcb, H.to_device(k.reshape(-1, 128), "bf16"), kc)
    lens = [t]
    sl = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    _log(f"logits with queries of magnitude 2^{exp2} ({qdt})")
    got = T.attention_logits(kcb, q, kc, sl, logits=_nan_logits(B, Hq, t))
    torch.cuda.synchronize()
    g_np = got.cpu().numpy()
    assert np.all(np.isfinite(g_np)), "non-finite logits"
    ref = H.oracle_logits(q.float().cpu().numpy().astype(np.float64), H.cache_to_host(kc), lens,
                          H.oracle_book(2, 128), g)
    worst = H.check_logits(g_np, ref, lens)
    _log(f"  worst relative error {worst:.2e}")
