"""The allocation-free decode entry point (tq_decode_attention_static) against
tq_decode_attention, through the C ABI: two calls in a row, the second on a
smaller input, each bitwise equal to the workspace entry point's output and
within the oracle's bar.  Sizes past the static scratch are rejected."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import online_vector_quantization_amd as T  # noqa: E402
from online_vector_quantization_amd import synth  # noqa: E402

from gpu_helpers import DEV, build_cache, check_decode, gpu_book, to_device  # noqa: E402


def _case(seed, B, Hq, Hkv, t_cap, seq_len):
    rng = np.random.default_rng(seed)
    k = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap, synth.outlier_channels(rng, Hkv, 4)))
    v = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap))
    q = synth.bf16_bits(rng.standard_normal((B, Hq, 128)).astype(np.float32))
    return to_device(k, "bf16"), to_device(v, "bf16"), to_device(q, "bf16"), seq_len


def test_static_entry_point_equals_workspace_entry_point_twice():
    kcb, vcb = gpu_book(2, 128), gpu_book(3, 0)
    cases = [(_case(31, 2, 16, 4, 3000, [3000, 1777]), 2, 16, 4, 3000),
             (_case(32, 1, 8, 2, 700, [513]), 1, 8, 2, 700)]      # second call: a smaller input
    for (k, v, q, seq), B, Hq, Hkv, t_cap in cases:
        print(f"[no-alloc] B={B} Hq={Hq} Hkv={Hkv} t_cap={t_cap} seq={seq}", flush=True)
        kc, vc = build_cache(kcb, vcb, k, v, B, Hkv, t_cap, t_cap)
        sl = torch.tensor(seq, dtype=torch.int32, device=DEV)
        ref = T.decode_attention(kcb, vcb, q, kc, vc, sl, out_dtype=torch.float32)
        sc_ref = torch.full((B, Hq, t_cap), float("nan"), device=DEV)
        sc = torch.full((B, Hq, t_cap), float("nan"), device=DEV)
        T.decode_attention(kcb, vcb, q, kc, vc, sl, out_dtype=torch.float32, dbg_scores=sc_ref)
        got = T.decode_attention_static(kcb, vcb, q, kc, vc, sl, out_dtype=torch.float32, dbg_scores=sc)
        got16 = T.decode_attention_static(kcb, vcb, q, kc, vc, sl, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))
        np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), sc_ref.cpu().numpy().view(np.uint32))
        ref16 = T.decode_attention(kcb, vcb, q, kc, vc, sl, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got16.view(torch.int16).cpu().numpy(), ref16.view(torch.int16).cpu().numpy())
        # and the shared result meets the oracle's bar
        check_decode(kcb, vcb, q, kc, vc, seq, 2, 3, 128)


def test_static_entry_point_rejects_sizes_past_its_scratch():
    kcb, vcb = gpu_book(2, 128), gpu_book(3, 0)
    B, Hq, Hkv, t_cap = 4096, 32, 8, 16
    assert T.decode_workspace_bytes(B, Hq, Hkv, t_cap) > (16 << 20)
    kc = T.CompressedCache.allocate(kcb, B, Hkv, t_cap)
    vc = T.CompressedCache.allocate(vcb, B, Hkv, t_cap)
    q = torch.zeros(B, Hq, 128, dtype=torch.bfloat16, device=DEV)
    sl = torch.full((B,), t_cap, dtype=torch.int32, device=DEV)
    with pytest.raises(T.TQError) as ei:
        T.decode_attention_static(kcb, vcb, q, kc, vc, sl)
    assert ei.value.status == -1 and "scratch" in str(ei.value)
