"""The tiny workload's quality report on the oracle (CPU).

4096 iid N(0,1) fp32 keys of dim 128 (seed 0), keys b = 3 (2-bit Lloyd-Max
codes + 1-bit QJL, m = 128), one N(0,1) query: the exact q.k against the
estimate nu (<q~, c[idx]> + sqrt(pi/2)/m gamma <S q~, 2z - 1>), and softmax of
both over the keys at scale 1/sqrt(d).

[admirer.cn memory-wall article, section 2, stage two] and [intelliparadigm
"3-bit" article, section 2.2]: the estimate is unbiased, and its variance
over S is gamma^2 nu^2 / m (pi/2 |q~|^2 - <q~, r/gamma>^2) per key.  Pins:

* bias: the mean error over the 4096 keys is within 3 standard errors of 0
  (the codebook is symmetric, so the error is odd in the key and its mean
  over isotropic keys is 0 for any fixed S);
* RMSE: within 10% of the closed form's root-mean variance over the keys;
* the MSE-only part alone (no QJL term) is biased toward 0 by the factor
  1 - D (D: the codebook's distortion), within 3 standard errors over the keys.

The report itself (bias, RMSE, correlation, softmax max-abs and total
variation) is printed; the GPU run of the same workload must reproduce it
(tests/test_gpu_quality.py).
"""
import math

import numpy as np

import oracle as O
from online_vector_quantization_amd import synth


def tiny_report(est, exact, d=128):
    """bias, RMSE, correlation of est against exact, and softmax(./sqrt(d)) max-abs and TV."""
    err = est - exact
    p, ph = O.softmax(exact / math.sqrt(d)), O.softmax(est / math.sqrt(d))
    return {"bias": float(err.mean()), "bias_se": float(err.std() / math.sqrt(err.size)),
            "rmse": float(math.sqrt(np.mean(err * err))), "corr": float(np.corrcoef(est, exact)[0, 1]),
            "softmax_max_abs": float(np.abs(p - ph).max()), "softmax_tv": float(0.5 * np.abs(p - ph).sum())}


def oracle_tiny():
    wl = synth.tiny()
    k = wl.k.reshape(-1, 128).astype(np.float64)
    q = wl.q.reshape(128).astype(np.float64)
    c, th = O.build_codebook(128, 2)
    Pi, S = O.haar_rotation(128, 0), O.qjl_matrix(128, 128, 1)
    enc = O.encode(k, Pi, c, th, S)
    est = O.decode_scores(q, Pi, c, S, enc["idx"], enc["nu"], enc["gamma"], enc["z"], 1.0)
    mse_only = O.decode_scores(q, Pi, c, S, enc["idx"], enc["nu"], None, None, 1.0)
    return k @ q, est, mse_only, enc, Pi @ q, c, th


def test_tiny_report_unbiased_and_closed_form_rmse():
    exact, est, mse_only, enc, q_rot, c, th = oracle_tiny()
    rep = tiny_report(est, exact)
    print("tiny report (oracle):", {k: round(v, 5) for k, v in rep.items()})
    assert abs(rep["bias"]) <= 3 * rep["bias_se"], rep
    # closed-form variance of the QJL estimate per key, times nu^2 (the score is nu <q~, k_hat>)
    gamma, nu, r = enc["gamma"], enc["nu"], enc["r"]
    with np.errstate(invalid="ignore", divide="ignore"):
        rhat = np.where(gamma[:, None] > 0, r / gamma[:, None], 0.0)
    var = gamma ** 2 * nu ** 2 / 128 * (math.pi / 2 * q_rot @ q_rot - (rhat @ q_rot) ** 2)
    pred = math.sqrt(var.mean())
    assert abs(rep["rmse"] / pred - 1) < 0.10, (rep["rmse"], pred)
    # the MSE-only estimate shrinks toward 0 by 1 - D (a property of the codebook alone, so the
    # spread over the keys sets its error).  The QJL form's slope is not pinned here: all keys share
    # one S, so it carries that one draw of S (the GPU bias test pools 64 queries instead).
    D = O.codebook_distortion(128, c, th)
    slope_mse = float(mse_only @ exact / (exact @ exact))
    resid = mse_only - (1 - D) * exact
    se = 3 * math.sqrt(np.mean(resid * resid)) / math.sqrt(exact @ exact)
    assert abs(slope_mse - (1 - D)) < se, (slope_mse, 1 - D, se)
