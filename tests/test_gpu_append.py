"""tq_append_decode: one decode-loop step (append the new K and V, attend over
the grown cache, advance seq_len on the device) in a single call.  bf16 new
rows take the combined key + value encode launch; fp32 rows two launches.

* Equal, bit for bit, to the separate path (tq_encode_kv of the new rows into
  rows seq_len[b], then tq_decode_attention with seq_len + 1), step after step,
  including an empty sequence and one that fills up (a full sequence is
  neither written nor advanced and attends over its t_cap tokens).
* The final caches and output pass the oracle parity.
* A captured graph of one step, replayed with new inputs, gives the eager
  results of every step.
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


def _clone(c: T.CompressedCache) -> T.CompressedCache:
    return T.CompressedCache(c.codes.clone(), c.norms.clone(), None if c.signs is None else c.signs.clone(),
                             None if c.res_norms is None else c.res_norms.clone())


def _same_cache(a: T.CompressedCache, b: T.CompressedCache):
    for x, y in ((a.codes, b.codes), (a.norms, b.norms), (a.signs, b.signs), (a.res_norms, b.res_norms)):
        if x is None:
            assert y is None
            continue
        np.testing.assert_array_equal(x.cpu().numpy().view(np.uint32), y.cpu().numpy().view(np.uint32))


def _setup(B, Hkv, g, t_cap, lens, kbits, vbits, m, seed):
    rng = np.random.default_rng(seed)
    k0 = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap, lognormal_sigma=0.5))
    v0 = synth.bf16_bits(synth.kv_block(rng, B, Hkv, t_cap, lognormal_sigma=0.5))
    kcb, vcb = H.gpu_book(kbits, m), H.gpu_book(vbits, 0)
    kc = T.CompressedCache.allocate(kcb, B, Hkv, t_cap)
    vc = T.CompressedCache.allocate(vcb, B, Hkv, t_cap)
    # prefill: sequence b holds lens[b] tokens
    rows = [(b * Hkv + h) * t_cap + t for b in range(B) for h in range(Hkv) for t in range(lens[b])]
    src = [(b * Hkv + h) * t_cap + t for b in range(B) for h in range(Hkv) for t in range(lens[b])]
    if rows:
        dst = torch.tensor(rows, dtype=torch.int64, device=H.DEV)
        idx = torch.tensor(src, dtype=torch.int64, device=H.DEV)
        T.encode_into_cache(kcb, H.to_device(k0.reshape(-1, 128), "bf16")[idx].contiguous(), kc, dst_row=dst)
        T.encode_into_cache(vcb, H.to_device(v0.reshape(-1, 128), "bf16")[idx].contiguous(), vc, dst_row=dst)
    return rng, kcb, vcb, kc, vc


def _step_inputs(rng, B, Hkv, Hq, kv_dtype="bf16"):
    k = synth.kv_block(rng, B, Hkv, 1, lognormal_sigma=0.5)[:, :, 0]
    v = synth.kv_block(rng, B, Hkv, 1, lognormal_sigma=0.5)[:, :, 0]
    q = synth.bf16_bits(rng.standard_normal((B, Hq, 128)).astype(np.float32))
    if kv_dtype == "bf16":
        return H.to_device(synth.bf16_bits(k), "bf16"), H.to_device(synth.bf16_bits(v), "bf16"), H.to_device(q, "bf16")
    return H.to_device(k, "f32"), H.to_device(v, "f32"), H.to_device(q, "bf16")


@pytest.mark.parametrize("kbits,vbits,m,g,kv_dtype", [(2, 3, 128, 4, "bf16"), (1, 2, 128, 8, "bf16"),
                                                      (3, 3, 0, 2, "bf16"), (4, 1, 128, 1, "f32")])
def test_append_decode_equals_separate_path(kbits, vbits, m, g, kv_dtype):
    B, Hkv, t_cap = 4, 2, 300
    lens = [250, 0, 297, 300]            # mixed, empty, filling up, already full
    Hq = Hkv * g
    rng, kcb, vcb, kc_a, vc_a = _setup(B, Hkv, g, t_cap, lens, kbits, vbits, m, seed=kbits * 7 + g)
    kc_b, vc_b = _clone(kc_a), _clone(vc_a)
    seq_a = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    seq_b = list(lens)
    ws_a = T.alloc_workspace(B, Hq, Hkv, t_cap, H.DEV)
    steps = 5
    _log(f"append_decode kbits={kbits} vbits={vbits} m={m} g={g} kv={kv_dtype} lens={lens} steps={steps}")
    for s in range(steps):
        kn, vn, q = _step_inputs(rng, B, Hkv, Hq, kv_dtype)
        out_a = T.append_decode(kcb, vcb, kn, vn, q, kc_a, vc_a, seq_a, workspace=ws_a)
        # separate path
        app = [b for b in range(B) if 0 <= seq_b[b] < t_cap]
        if app:
            rows = torch.tensor([(b * Hkv + h) * t_cap + seq_b[b] for b in app for h in range(Hkv)],
                                dtype=torch.int64, device=H.DEV)
            sel = torch.tensor([b * Hkv + h for b in app for h in range(Hkv)], dtype=torch.int64, device=H.DEV)
            T.encode_into_cache(kcb, kn.reshape(-1, 128)[sel].contiguous(), kc_b, dst_row=rows)
            T.encode_into_cache(vcb, vn.reshape(-1, 128)[sel].contiguous(), vc_b, dst_row=rows)
        attend = [min(s_ + 1, t_cap) for s_ in seq_b]
        out_b = T.decode_attention(kcb, vcb, q, kc_b, vc_b, torch.tensor(attend, dtype=torch.int32, device=H.DEV))
        seq_b = [s_ + 1 if 0 <= s_ < t_cap else s_ for s_ in seq_b]
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_a.cpu().numpy().view(np.uint32), out_b.cpu().numpy().view(np.uint32))
        assert seq_a.cpu().tolist() == seq_b
    _same_cache(kc_a, kc_b)
    _same_cache(vc_a, vc_b)
    assert seq_b == [255, 5, 300, 300]
    # the final state against the oracle
    H.check_decode(kcb, vcb, q, kc_a, vc_a, seq_b, kbits, vbits, m)


def test_append_decode_graph_replay():
    B, Hkv, g, t_cap = 16, 8, 4, 8200
    Hq = Hkv * g
    lens = [8192] * B
    rng, kcb, vcb, kc_e, vc_e = _setup(B, Hkv, g, t_cap, lens, 2, 3, 128, seed=77)
    kc_g, vc_g = _clone(kc_e), _clone(vc_e)
    seq_e = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    seq_g = seq_e.clone()
    ws_e = T.alloc_workspace(B, Hq, Hkv, t_cap, H.DEV)
    ws_g = T.alloc_workspace(B, Hq, Hkv, t_cap, H.DEV)
    kn_s, vn_s, q_s = (torch.empty(B, Hkv, 128, dtype=torch.bfloat16, device=H.DEV),
                       torch.empty(B, Hkv, 128, dtype=torch.bfloat16, device=H.DEV),
                       torch.empty(B, Hq, 128, dtype=torch.bfloat16, device=H.DEV))
    out_s = torch.empty(B, Hq, 128, dtype=torch.float32, device=H.DEV)
    inputs = [_step_inputs(rng, B, Hkv, Hq) for _ in range(8)]
    # capture one step (the first eager call also warms the library up)
    kn_s.copy_(inputs[0][0]); vn_s.copy_(inputs[0][1]); q_s.copy_(inputs[0][2])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            T.append_decode(kcb, vcb, kn_s, vn_s, q_s, kc_g, vc_g, seq_g, out=out_s, workspace=ws_g,
                            stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture did not run the step: state unchanged
    assert seq_g.cpu().tolist() == lens
    _log("append_decode graph: 8 replays against eager steps")
    for s in range(8):
        kn, vn, q = inputs[s]
        kn_s.copy_(kn); vn_s.copy_(vn); q_s.copy_(q)
        graph.replay()
        out_e = T.append_decode(kcb, vcb, kn, vn, q, kc_e, vc_e, seq_e, workspace=ws_e)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_s.cpu().numpy().view(np.uint32), out_e.cpu().numpy().view(np.uint32))
        assert seq_g.cpu().tolist() == [8193 + s] * B
    _same_cache(kc_g, kc_e)
    _same_cache(vc_g, vc_e)


def test_append_decode_wide_batch():
    # 460 sequences x 8 kv heads (3,680 rows, one token chunk each) with
    # ragged, empty and full sequences.  Same bar: bit for bit the separate
    # path, step after step, and the oracle at the end.
    B, Hkv, g, t_cap = 460, 8, 1, 24
    rng0 = np.random.default_rng(77)
    lens = [int(x) for x in rng0.integers(0, t_cap + 1, size=B)]
    lens[0], lens[1], lens[2] = 0, t_cap, t_cap - 1
    Hq = Hkv * g
    rng, kcb, vcb, kc_a, vc_a = _setup(B, Hkv, g, t_cap, lens, 2, 3, 128, seed=78)
    kc_b, vc_b = _clone(kc_a), _clone(vc_a)
    seq_a = torch.tensor(lens, dtype=torch.int32, device=H.DEV)
    seq_b = list(lens)
    ws_a = T.alloc_workspace(B, Hq, Hkv, t_cap, H.DEV)
    _log(f"append_decode wide: B={B} Hkv={Hkv} g={g} t_cap={t_cap}")
    for s in range(3):
        kn, vn, q = _step_inputs(rng, B, Hkv, Hq)
        out_a = T.append_decode(kcb, vcb, kn, vn, q, kc_a, vc_a, seq_a, workspace=ws_a)
        app = [b for b in range(B) if 0 <= seq_b[b] < t_cap]
        rows = torch.tensor([(b * Hkv + h) * t_cap + seq_b[b] for b in app for h in range(Hkv)],
                            dtype=torch.int64, device=H.DEV)
        sel = torch.tensor([b * Hkv + h for b in app for h in range(Hkv)], dtype=torch.int64, device=H.DEV)
        T.encode_into_cache(kcb, kn.reshape(-1, 128)[sel].contiguous(), kc_b, dst_row=rows)
        T.encode_into_cache(vcb, vn.reshape(-1, 128)[sel].contiguous(), vc_b, dst_row=rows)
        attend = [min(s_ + 1, t_cap) for s_ in seq_b]
        out_b = T.decode_attention(kcb, vcb, q, kc_b, vc_b, torch.tensor(attend, dtype=torch.int32, device=H.DEV))
        seq_b = [s_ + 1 if 0 <= s_ < t_cap else s_ for s_ in seq_b]
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_a.cpu().numpy().view(np.uint32), out_b.cpu().numpy().view(np.uint32))
        assert seq_a.cpu().tolist() == seq_b
    _same_cache(kc_a, kc_b)
    _same_cache(vc_a, vc_b)
    H.check_decode(kcb, vcb, q, kc_a, vc_a, seq_b, 2, 3, 128)
