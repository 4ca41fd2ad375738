"""Inner-product bias of MSE-only keys against the (b-1)-bit + QJL form,
measured through the library (the decode's logits).

[admirer.cn memory-wall article, section 2]: an MSE-optimal quantizer is
biased for inner products, which is why stage two adds the 1-bit QJL sketch
of the residual.  For a Lloyd-Max quantizer the centroid condition gives the
bias exactly: E<q, k_hat> = (1 - D) <q, k>, with D the codebook's distortion;
the QJL form is unbiased (over S; pooled over many queries for one seeded S).

Workload: 8 KV heads x 4096 iid N(0,1) bf16 keys, 64 N(0,1) q heads (g = 8).
The regression slope of the estimated on the exact logits is pooled over all
(query, key) pairs; its standard error comes from the spread of the 64
per-query slopes.
"""
import math
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


def _logits(kcb, vcb, k, q, Hkv, Tn):
    kc = T.CompressedCache.allocate(kcb, 1, Hkv, Tn)
    vc = T.CompressedCache.allocate(vcb, 1, Hkv, Tn)
    kd = H.to_device(k.reshape(-1, 128), "bf16")
    T.encode_into_cache(kcb, kd, kc)
    T.encode_into_cache(vcb, kd, vc)
    Hq = q.shape[1]
    scores = torch.zeros(1, Hq, Tn, dtype=torch.float32, device=H.DEV)
    T.decode_attention(kcb, vcb, H.to_device(q, "bf16"), kc, vc, torch.tensor([Tn], dtype=torch.int32, device=H.DEV),
                       dbg_scores=scores)
    torch.cuda.synchronize()
    return scores.cpu().numpy()[0].astype(np.float64) * math.sqrt(128.0)   # <q, k> estimates


def _slopes(est, exact):
    per_q = (est * exact).sum(1) / (exact * exact).sum(1)
    pooled = (est * exact).sum() / (exact * exact).sum()
    return pooled, per_q.std() / math.sqrt(per_q.size)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_inner_product_bias_mse_only_vs_qjl(b):
    Hkv, g, Tn = 8, 8, 4096
    rng = np.random.default_rng(40 + b)
    k = synth.bf16_bits(rng.standard_normal((1, Hkv, Tn, 128), dtype=np.float32))
    q = synth.bf16_bits(rng.standard_normal((1, Hkv * g, 128), dtype=np.float32))
    kf = synth.bf16_to_f32(k).astype(np.float64)[0]
    qf = synth.bf16_to_f32(q).astype(np.float64)[0]
    exact = np.stack([kf[h // g] @ qf[h] for h in range(Hkv * g)])          # [Hq, Tn]
    vcb = H.gpu_book(2, 0)
    est_mse = _logits(H.gpu_book(b, 0), vcb, k, q, Hkv, Tn)
    est_qjl = _logits(H.gpu_book(b - 1, 128), vcb, k, q, Hkv, Tn)
    c, t = O.build_codebook(128, b)
    D = O.codebook_distortion(128, c.astype(np.float64), t.astype(np.float64))
    s_mse, se_mse = _slopes(est_mse, exact)
    s_qjl, se_qjl = _slopes(est_qjl, exact)
    rmse_mse = np.sqrt(np.mean((est_mse - exact) ** 2))
    rmse_qjl = np.sqrt(np.mean((est_qjl - exact) ** 2))
    print(f"b={b}: MSE-only slope {s_mse:.4f} +- {se_mse:.4f} (1-D = {1 - D:.4f}), rmse {rmse_mse:.3f}; "
          f"{b - 1}+1 QJL slope {s_qjl:.4f} +- {se_qjl:.4f}, rmse {rmse_qjl:.3f}", file=sys.stderr, flush=True)
    # MSE-only: shrinks inner products by exactly 1 - D
    assert abs(s_mse - (1.0 - D)) < 4.0 * se_mse + 1e-3
    assert 1.0 - s_mse > 5.0 * se_mse
    # (b-1) + 1 QJL: unbiased
    assert abs(s_qjl - 1.0) < 4.0 * se_qjl + 1e-3


def test_tiny_config_report_matches_oracle():
    # The tiny workload through the library (fp32 keys, b = 3: 2-bit codes + QJL; the values
    # reuse the keys at 2 bits): its quality report equals the oracle's, whose unbiasedness and
    # closed-form RMSE tests/test_tiny_report.py pins.
    from test_tiny_report import oracle_tiny, tiny_report
    wl = synth.tiny()
    kcb, vcb = H.gpu_book(2, 128), H.gpu_book(2, 0)
    k = H.to_device(wl.k.reshape(-1, 128), "f32")
    kc, vc = H.build_cache(kcb, vcb, k.reshape(1, 1, 4096, 128), k.reshape(1, 1, 4096, 128), 1, 1, 4096, 4096)
    scores = torch.zeros(1, 1, 4096, dtype=torch.float32, device=H.DEV)
    T.decode_attention(kcb, vcb, H.to_device(wl.q, "f32"), kc, vc,
                       torch.tensor([4096], dtype=torch.int32, device=H.DEV), dbg_scores=scores)
    torch.cuda.synchronize()
    est = scores.cpu().numpy()[0, 0].astype(np.float64) * math.sqrt(128.0)
    exact, est_o, _, _, _, _, _ = oracle_tiny()
    got, ref = tiny_report(est, exact), tiny_report(est_o, exact)
    print("tiny report (GPU):   ", {k_: round(v, 5) for k_, v in got.items()}, file=sys.stderr, flush=True)
    print("tiny report (oracle):", {k_: round(v, 5) for k_, v in ref.items()}, file=sys.stderr, flush=True)
    assert abs(got["bias"]) <= 3 * got["bias_se"]
    assert abs(got["rmse"] / ref["rmse"] - 1) < 1e-3
    assert abs(got["corr"] - ref["corr"]) < 1e-4
    assert abs(got["softmax_tv"] - ref["softmax_tv"]) < 1e-3
    assert abs(got["softmax_max_abs"] - ref["softmax_max_abs"]) < 1e-4
