"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same entry points, same work-group plans).

* Llama-3-8B-shaped layer (1 x 8 KV heads x 32768 tokens, 32 q heads): every
  encoded key and value row and the full decode are checked.
* Batched decode (16 x 8 x 8192 tokens, b = 2 and b = 4): 8 steps that each
  append one token per (sequence, head); sampled encode rows, every step's
  output and one step's scores are checked.
* Llama-3-70B-shaped long context (131072 tokens, 64 q heads): sampled encode
  rows and the full decode.
* Bulk encode (16,777,216 K and V vectors, keys b = 4, values 4-bit), then 64
  queries over the first 262144-token x 8-head cache: sampled rows of the full
  run (re-encoded with debug outputs, which must reproduce the same codes) and
  the full decode.
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


def _check_rows(cb, x_dev, rows_cache, cache, bits, m, sample):
    """Re-encode sampled input rows with debug outputs: the codes must equal
    the full run's, and the sampled encode must pass the oracle parity."""
    sub = x_dev[torch.from_numpy(sample).to(H.DEV)].contiguous()
    got = H.encode_gpu(cb, sub)
    full_codes = cache.codes.reshape(-1, cb.code_words)[torch.from_numpy(rows_cache).to(H.DEV)]
    np.testing.assert_array_equal(H.u32(full_codes), got["codes"])
    np.testing.assert_array_equal(cache.norms.reshape(-1)[torch.from_numpy(rows_cache).to(H.DEV)].cpu().numpy(),
                                  got["norms"])
    if m:
        full_signs = cache.signs.reshape(-1, cb.sign_words)[torch.from_numpy(rows_cache).to(H.DEV)]
        np.testing.assert_array_equal(H.u32(full_signs), got["signs"])
    x_host = sub.float().cpu().numpy()
    return H.check_encode(x_host, got, bits, m)


def test_llama8b_layer_full():
    wl = synth.llama8b()
    _log(f"{wl.name}: encode all {wl.k.size // 128} K and V rows, then decode")
    kcb, vcb = H.gpu_book(2, 128), H.gpu_book(3, 0)
    for cb, arr, bits, m in ((kcb, wl.k, 2, 128), (vcb, wl.v, 3, 0)):
        x = arr.reshape(-1, 128)
        got = H.encode_gpu(cb, H.to_device(x, "bf16"))
        flips = H.check_encode(H.host_values(x, "bf16"), got, bits, m)
        _log(f"  bits={bits} m={m}: near-boundary flips vs float64 oracle {flips}")
    kc = T.CompressedCache.allocate(kcb, 1, 8, wl.seq_len)
    vc = T.CompressedCache.allocate(vcb, 1, 8, wl.seq_len)
    T.encode_into_cache(kcb, H.to_device(wl.k.reshape(-1, 128), "bf16"), kc)
    T.encode_into_cache(vcb, H.to_device(wl.v.reshape(-1, 128), "bf16"), vc)
    err = H.check_decode(kcb, vcb, H.to_device(wl.q, "bf16"), kc, vc, [wl.seq_len], 2, 3, 128)
    _log(f"  decode max-abs error {err:.2e}")


@pytest.mark.parametrize("bits", [2, 4])
def test_batched_decode_with_appends(bits):
    wl = synth.batched(bits)
    B, Hkv, S = wl.batch, wl.n_kv_heads, wl.seq_len
    steps = 8
    t_cap = S + steps
    _log(f"{wl.name}: encode {B * Hkv * S} rows into t_cap={t_cap}, then {steps} append+decode steps")
    kcb, vcb = H.gpu_book(bits - 1, 128), H.gpu_book(bits, 0)
    k_dev = H.to_device(wl.k, "bf16")
    v_dev = H.to_device(wl.v, "bf16")
    kc, vc = H.build_cache(kcb, vcb, k_dev, v_dev, B, Hkv, t_cap, S)
    rng = np.random.default_rng(bits)
    sample = rng.choice(B * Hkv * S, size=4096, replace=False)
    b_i, rem = np.divmod(sample, Hkv * S)
    h_i, t_i = np.divmod(rem, S)
    rows = (b_i * Hkv + h_i) * t_cap + t_i
    _check_rows(kcb, k_dev.reshape(-1, 128), rows, kc, bits - 1, 128, sample)
    _check_rows(vcb, v_dev.reshape(-1, 128), rows, vc, bits, 0, sample)
    ws = T.alloc_workspace(B, wl.n_q_heads, Hkv, t_cap, H.DEV)
    for s in range(steps):
        ka, va, qa = synth.appended_tokens(s)
        dst = torch.tensor([(b * Hkv + h) * t_cap + S + s for b in range(B) for h in range(Hkv)],
                           dtype=torch.int64, device=H.DEV)
        T.encode_into_cache(kcb, H.to_device(ka.reshape(-1, 128), "bf16"), kc, dst_row=dst)
        T.encode_into_cache(vcb, H.to_device(va.reshape(-1, 128), "bf16"), vc, dst_row=dst)
        seq = [S + s + 1] * B
        q_dev = H.to_device(qa, "bf16")
        if s in (0, steps - 1):
            err = H.check_decode(kcb, vcb, q_dev, kc, vc, seq, bits - 1, bits, 128)
            _log(f"  step {s}: decode max-abs error {err:.2e}")
        else:
            T.decode_attention(kcb, vcb, q_dev, kc, vc, torch.tensor(seq, dtype=torch.int32, device=H.DEV),
                               workspace=ws)
    torch.cuda.synchronize()


def test_llama70b_long_context():
    wl = synth.llama70b()
    S = wl.seq_len
    _log(f"{wl.name}: encode {8 * S} K and V rows, then decode with 64 q heads")
    kcb, vcb = H.gpu_book(2, 128), H.gpu_book(2, 0)
    k_dev = H.to_device(wl.k.reshape(-1, 128), "bf16")
    v_dev = H.to_device(wl.v.reshape(-1, 128), "bf16")
    kc = T.CompressedCache.allocate(kcb, 1, 8, S)
    vc = T.CompressedCache.allocate(vcb, 1, 8, S)
    T.encode_into_cache(kcb, k_dev, kc)
    T.encode_into_cache(vcb, v_dev, vc)
    sample = np.random.default_rng(70).choice(8 * S, size=8192, replace=False)
    _check_rows(kcb, k_dev, sample, kc, 2, 128, sample)
    _check_rows(vcb, v_dev, sample, vc, 2, 0, sample)
    del k_dev, v_dev
    err = H.check_decode(kcb, vcb, H.to_device(wl.q, "bf16"), kc, vc, [S], 2, 2, 128)
    _log(f"  decode max-abs error {err:.2e}")


def test_bulk_encode_and_wide_decode():
    n = 16_777_216
    _log(f"bulk: generating {n} K and V rows on the GPU")
    k_dev, v_dev, q = synth.bulk_device(n, H.DEV)
    kcb, vcb = H.gpu_book(3, 128), H.gpu_book(4, 0)
    kc = T.CompressedCache.allocate(kcb, 1, 1, n)
    vc = T.CompressedCache.allocate(vcb, 1, 1, n)
    T.encode_into_cache(kcb, k_dev, kc)
    T.encode_into_cache(vcb, v_dev, vc)
    torch.cuda.synchronize()
    _log("  full encode done; checking sampled rows")
    sample = np.random.default_rng(5).choice(n, size=16384, replace=False)
    _check_rows(kcb, k_dev, sample, kc, 3, 128, sample)
    _check_rows(vcb, v_dev, sample, vc, 4, 0, sample)
    del k_dev, v_dev
    # decode: 64 q heads over the first 2,097,152 rows viewed as [1, 8, 262144]
    T_len = 262144
    kview = T.CompressedCache(kc.codes.reshape(-1, kcb.code_words)[: 8 * T_len].reshape(1, 8, T_len, -1),
                              kc.norms.reshape(-1)[: 8 * T_len].reshape(1, 8, T_len),
                              kc.signs.reshape(-1, kcb.sign_words)[: 8 * T_len].reshape(1, 8, T_len, -1),
                              kc.res_norms.reshape(-1)[: 8 * T_len].reshape(1, 8, T_len))
    vview = T.CompressedCache(vc.codes.reshape(-1, vcb.code_words)[: 8 * T_len].reshape(1, 8, T_len, -1),
                              vc.norms.reshape(-1)[: 8 * T_len].reshape(1, 8, T_len))
    _log("  decode over 262144 tokens x 8 kv heads, 64 q heads")
    err = H.check_decode(kcb, vcb, q, kview, vview, [T_len], 3, 4, 128)
    _log(f"  decode max-abs error {err:.2e}")
