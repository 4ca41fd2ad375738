"""Pins for the CPU oracle: closed forms, textbook limits, brute force, the
pages' bounds and statistical properties.  Each test is chosen so that a
plausible mistake in the oracle (a dropped term, a wrong sign, a transposed
operand, an off-by-one cell) fails it.  No GPU needed."""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

import oracle as O


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- generator

def test_splitmix64_known_answers(golden_dir):
    g = _load(golden_dir, "splitmix64_seed0.json")
    got = [int(v) for v in O.splitmix64(g["seed"], len(g["outputs_hex"]))]
    assert got == [int(h, 16) for h in g["outputs_hex"]]


def test_splitmix64_stream_offsets():
    # Output i of seed s equals output 0 of seed s + i * golden gamma (counter form).
    gamma = 0x9E3779B97F4A7C15
    a = O.splitmix64(12345, 40)
    for i in (0, 7, 39):
        b = O.splitmix64((12345 + i * gamma) % (1 << 64), 1)
        assert int(a[i]) == int(b[0])


def test_gaussian_stream_is_standard_normal():
    x = O.gaussian_stream(7, 200_000)
    assert abs(x.mean()) < 4.5 / math.sqrt(x.size)
    assert abs(x.var() - 1.0) < 4.5 * math.sqrt(2.0 / x.size)
    assert stats.kstest(x, "norm").pvalue > 1e-3
    # Box-Muller pairs are uncorrelated.
    assert abs(np.corrcoef(x[0::2], x[1::2])[0, 1]) < 4.5 / math.sqrt(x.size / 2)


def test_gaussian_stream_prefix_and_seed_dependence():
    a = O.gaussian_stream(3, 101)
    b = O.gaussian_stream(3, 64)
    np.testing.assert_array_equal(a[:64], b)
    assert not np.allclose(O.gaussian_stream(4, 64), b)


# ---------------------------------------------------------------- coordinate law

@pytest.mark.parametrize("d", [3, 4, 16, 128])
def test_density_normalized_with_variance_one_over_d(d):
    tot, _ = integrate.quad(lambda t: float(O.coord_pdf(t, d)), -1, 1, limit=200)
    var, _ = integrate.quad(lambda t: t * t * float(O.coord_pdf(t, d)), -1, 1, limit=200)
    assert abs(tot - 1.0) < 1e-10
    assert abs(var - 1.0 / d) < 1e-10


@pytest.mark.parametrize("d", [4, 128])
def test_cdf_and_partial_mean_match_quadrature(d):
    for t in (-0.5, -0.1, 0.0, 0.03, 0.2, 0.9):
        cdf, _ = integrate.quad(lambda s: float(O.coord_pdf(s, d)), -1, t, limit=200, epsabs=1e-14)
        pm, _ = integrate.quad(lambda s: s * float(O.coord_pdf(s, d)), -1, t, limit=200, epsabs=1e-14)
        assert abs(float(O.coord_cdf(t, d)) - cdf) < 1e-11
        assert abs(float(O.coord_partial_mean(t, d)) - pm) < 1e-11


def test_density_is_coordinate_law_of_random_unit_vectors():
    # Monte-Carlo: a coordinate of a uniform point on S^{d-1} has CDF coord_cdf.
    rng = np.random.default_rng(0)
    d = 8
    g = rng.standard_normal((100_000, d))
    y = g[:, 0] / np.linalg.norm(g, axis=1)
    assert stats.kstest(y, lambda t: O.coord_cdf(t, d)).pvalue > 1e-3


# ---------------------------------------------------------------- codebook

@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_d3_is_uniform_quantizer(bits):
    # f_3 is uniform on [-1,1]: the optimum is the uniform quantizer and
    # D = 4^-b exactly, i.e. it sits on the page's lower bound.
    c, t, _ = O.lloyd_max(3, bits)
    L = 1 << bits
    np.testing.assert_allclose(c, -1.0 + (2.0 * np.arange(L) + 1.0) / L, atol=1e-12)
    np.testing.assert_allclose(t, -1.0 + 2.0 * np.arange(1, L) / L, atol=1e-12)
    assert abs(O.codebook_distortion(3, c, t) - 4.0 ** -bits) < 1e-12


@pytest.mark.parametrize("d", [4, 16, 128])
def test_codebook_one_bit_closed_form(d):
    # One bit: c = +-E|Y| = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)).
    c, t, _ = O.lloyd_max(d, 1)
    expect = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    np.testing.assert_allclose(c, [-expect, expect], rtol=1e-12)
    assert t[0] == 0.0
    if d == 4:
        assert abs(expect - 4.0 / (3.0 * math.pi)) < 1e-15


@pytest.mark.parametrize("d,bits", [(4, 2), (4, 3), (128, 2), (128, 3), (128, 4)])
def test_codebook_fixed_point_by_quadrature(d, bits):
    # Lloyd-Max conditions checked with an independent route (adaptive
    # quadrature of the density): centroid = conditional mean of its cell,
    # threshold = midpoint of neighbouring centroids.
    c, t, _ = O.lloyd_max(d, bits)
    edges = np.concatenate(([-1.0], t, [1.0]))
    for i in range(len(c)):
        a, b = edges[i], edges[i + 1]
        mass, _ = integrate.quad(lambda s: float(O.coord_pdf(s, d)), a, b, epsabs=1e-15, epsrel=1e-13, limit=200)
        mom, _ = integrate.quad(lambda s: s * float(O.coord_pdf(s, d)), a, b, epsabs=1e-15, epsrel=1e-13, limit=200)
        assert abs(mom / mass - c[i]) < 1e-10
    np.testing.assert_allclose(t, 0.5 * (c[1:] + c[:-1]), atol=0)
    assert np.all(np.diff(c) > 0)
    np.testing.assert_allclose(c, -c[::-1], atol=1e-14)


def test_codebook_distortion_inside_page_bounds(golden_dir):
    g = _load(golden_dir, "page_bounds.json")
    for bits in (1, 2, 3, 4):
        c, t, _ = O.lloyd_max(128, bits)
        D = O.codebook_distortion(128, c, t)
        assert 4.0 ** -bits <= D <= g["mse_upper_factor"] * 4.0 ** -bits
        if bits == 1:
            assert abs(D * 4.0 - g["ratio_to_lower_bound_at_b1"]) < g["ratio_at_b1_tolerance"]


def test_codebook_distortion_matches_monte_carlo():
    # Independent route for D: quantize many sampled coordinates.
    rng = np.random.default_rng(1)
    d = 128
    g = rng.standard_normal((4000, d))
    y = (g / np.linalg.norm(g, axis=1, keepdims=True)).ravel()
    for bits in (2, 3):
        c, t, _ = O.lloyd_max(d, bits)
        err = d * np.mean((y - c[O.quantize(y, t)]) ** 2)
        D = O.codebook_distortion(d, c, t)
        assert abs(err - D) < 0.02 * D


def test_codebook_gaussian_limit(golden_dir):
    g = _load(golden_dir, "gaussian_lloyd_max.json")
    d = g["dimension_used"]
    for bits, levels in g["positive_levels"].items():
        c, _, _ = O.lloyd_max(d, int(bits))
        got = c[len(c) // 2:] * math.sqrt(d)
        np.testing.assert_allclose(got, levels, atol=g["abs_tolerance"])


def test_build_codebook_rounds_float64_tables():
    c32, t32 = O.build_codebook(128, 3)
    c, t, _ = O.lloyd_max(128, 3)
    assert c32.dtype == np.float32 and t32.dtype == np.float32
    np.testing.assert_array_equal(c32, c.astype(np.float32))
    np.testing.assert_array_equal(t32, t.astype(np.float32))


# ---------------------------------------------------------------- rotation

def test_rotation_orthogonal_and_preserves_inner_products():
    Pi = O.haar_rotation(128, 0)
    assert np.abs(Pi.T @ Pi - np.eye(128)).max() < 1e-12
    assert abs(abs(np.linalg.det(Pi)) - 1.0) < 1e-10
    # fp32 copy: inner products preserved to 1e-5 relative (the explainer's
    # claim that the rotation leaves Q K^T unchanged).
    P32 = Pi.astype(np.float32)
    rng = np.random.default_rng(2)
    a = rng.standard_normal((256, 128)).astype(np.float32)
    b = rng.standard_normal((256, 128)).astype(np.float32)
    ra = (a @ P32.T).astype(np.float64)
    rb = (b @ P32.T).astype(np.float64)
    ip = np.sum(a.astype(np.float64) * b, axis=1)
    ipr = np.sum(ra * rb, axis=1)
    scale = np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1)
    assert np.max(np.abs(ipr - ip) / scale) < 1e-5


def test_rotation_reproducible_from_seed():
    np.testing.assert_array_equal(O.haar_rotation(16, 5), O.haar_rotation(16, 5))
    assert not np.allclose(O.haar_rotation(16, 5), O.haar_rotation(16, 6))
    # The rotation is Q of the seed's Gaussian matrix with R's diagonal made positive.
    G = O.gaussian_matrix(5, 16, 16)
    Pi = O.haar_rotation(16, 5)
    R = Pi.T @ G
    assert np.abs(np.tril(R, -1)).max() < 1e-12
    assert np.all(np.diag(R) > 0)


def test_rotation_is_haar_d4():
    # First column of a Haar orthogonal matrix is uniform on S^3, so its first
    # coordinate has density (2/pi) sqrt(1-t^2) with CDF 1/2 + (t sqrt(1-t^2) + asin t)/pi.
    n = 3000
    vals = np.array([O.haar_rotation(4, s)[0, 0] for s in range(n)])
    cdf = lambda t: 0.5 + (t * np.sqrt(1 - t * t) + np.arcsin(t)) / np.pi
    assert stats.kstest(vals, cdf).pvalue > 1e-3
    dets = np.array([np.linalg.det(O.haar_rotation(4, s)) for s in range(n)])
    frac = np.mean(dets > 0)
    assert abs(frac - 0.5) < 4.0 * math.sqrt(0.25 / n)


def test_qjl_matrix_is_seeded_gaussian():
    S = O.qjl_matrix(128, 128, 1)
    np.testing.assert_array_equal(S.ravel(), O.gaussian_stream(1, 128 * 128))
    assert S.shape == (128, 128)


# ---------------------------------------------------------------- quantizer

@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_quantize_equals_bruteforce_nearest_codeword_d4(bits):
    # d = 4: search all L^4 product codewords for the nearest one; it must equal
    # the per-coordinate threshold lookup.
    c, t, _ = O.lloyd_max(4, bits)
    L = len(c)
    grid = np.array(np.meshgrid(*[np.arange(L)] * 4, indexing="ij")).reshape(4, -1).T
    words = c[grid]
    rng = np.random.default_rng(bits)
    g = rng.standard_normal((300, 4))
    y = g / np.linalg.norm(g, axis=1, keepdims=True)
    best = np.argmin(((y[:, None, :] - words[None, :, :]) ** 2).sum(-1), axis=1)
    np.testing.assert_array_equal(grid[best], O.quantize(y, t))


def test_quantize_ties_nan_signed_zero():
    t = np.array([-0.5, 0.0, 0.5], dtype=np.float32)
    y = np.array([-0.5, 0.0, -0.0, 0.5, np.nan, -1.0, 1.0, np.nextafter(np.float32(0.5), np.float32(0))],
                 dtype=np.float32)
    np.testing.assert_array_equal(O.quantize(y, t), [1, 2, 2, 3, 0, 0, 3, 2])


# ---------------------------------------------------------------- packing

def test_pack_literal_patterns():
    # 1 bit, alternating 1,0: 0x55555555 per word.
    v = np.tile([1, 0], 64)[None, :]
    np.testing.assert_array_equal(O.pack_bits(v, 1), [[0x55555555] * 4])
    # 2 bits, all 3: all ones.
    np.testing.assert_array_equal(O.pack_bits(np.full((1, 128), 3), 2), [[0xFFFFFFFF] * 8])
    # 3 bits: code 0 = 7 -> word0 = 7; code 10 = 7 straddles words 0 and 1.
    v = np.zeros((1, 128), dtype=np.int64)
    v[0, 0] = 7
    v[0, 10] = 7
    w = O.pack_bits(v, 3)
    assert w.shape == (1, 12)
    assert w[0, 0] == 0xC0000007 and w[0, 1] == 0x1 and np.all(w[0, 2:] == 0)
    # 4 bits: code j = j % 16 -> word k = 0xFEDCBA98 / 0x76543210 alternating.
    v = (np.arange(128) % 16)[None, :]
    w = O.pack_bits(v, 4)
    np.testing.assert_array_equal(w[0, :2], [0x76543210, 0xFEDCBA98])


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_pack_matches_big_integer_stream(bits):
    rng = np.random.default_rng(10 + bits)
    v = rng.integers(0, 1 << bits, size=(5, 128))
    w = O.pack_bits(v, bits)
    for r in range(5):
        stream = 0
        for j in range(128):
            stream |= int(v[r, j]) << (j * bits)
        expect = [(stream >> (32 * k)) & 0xFFFFFFFF for k in range(128 * bits // 32)]
        assert [int(x) for x in w[r]] == expect
    np.testing.assert_array_equal(O.unpack_bits(w, 128, bits), v)


# ---------------------------------------------------------------- encode

def test_encode_mse_matches_analytic_distortion():
    d = 128
    Pi = O.haar_rotation(d, 0)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20000, d))
    for bits in (1, 2, 3):
        c, t = O.build_codebook(d, bits)
        e = O.encode(x, Pi, c, t)
        u = x / e["nu"][:, None]
        uhat = c.astype(np.float64)[e["idx"]] @ Pi        # Pi^T c, row form
        err = np.sum((u - uhat) ** 2, axis=1)
        D = O.codebook_distortion(d, c.astype(np.float64), t.astype(np.float64))
        assert abs(err.mean() - D) < 4.0 * err.std() / math.sqrt(err.size)


def test_encode_zero_vector_and_scale_invariance():
    d = 16
    Pi = O.haar_rotation(d, 1)
    c, t = O.build_codebook(d, 2)
    S = O.qjl_matrix(32, d, 2)
    x = np.zeros((2, d))
    x[1] = np.linspace(-1, 1, d)
    e = O.encode(x, Pi, c, t, S)
    assert e["nu"][0] == 0.0 and np.all(e["y"][0] == 0.0)
    assert np.all(e["idx"][0] == 2)          # y = 0 sits on the middle threshold -> upper cell
    e2 = O.encode(7.0 * x, Pi, c, t, S)
    np.testing.assert_array_equal(e2["idx"], e["idx"])
    np.testing.assert_allclose(e2["nu"], 7.0 * e["nu"])
    np.testing.assert_allclose(e2["gamma"], e["gamma"], rtol=1e-12)


def test_encode_keys_residual_and_signs():
    d, m = 32, 64
    Pi = O.haar_rotation(d, 4)
    c, t = O.build_codebook(d, 2)
    S = O.qjl_matrix(m, d, 5)
    x = np.random.default_rng(4).standard_normal((50, d))
    e = O.encode(x, Pi, c, t, S)
    # y is the rotated unit vector: norm one, and Pi^T y recovers x / nu.
    np.testing.assert_allclose(np.linalg.norm(e["y"], axis=1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(e["y"] @ Pi, x / e["nu"][:, None], atol=1e-12)
    np.testing.assert_allclose(e["r"] + c.astype(np.float64)[e["idx"]], e["y"], atol=1e-15)
    np.testing.assert_array_equal(e["z"], (e["r"] @ S.T) > 0)
    # residual is the quantization error: no larger than half the widest cell
    assert np.all(np.abs(e["r"]) <= np.max(np.diff(np.concatenate(([-1], t, [1])))))


def test_residual_from_rotated_hand_worked_d4():
    # d = 4, one bit: the centroids are -+4/(3 pi) (closed form, pinned above) and
    # the threshold is 0.  y = (0.5, -0.1, 0.3, -0.7) quantizes to (1, 0, 1, 0),
    # so r = (0.5 - c, -0.1 + c, 0.3 - c, -0.7 + c) with c = 0.42441318157838756
    # (values written out by hand below) and gamma = sqrt(sum r_j^2).
    c = np.array([-4.0 / (3.0 * math.pi), 4.0 / (3.0 * math.pi)])
    y = np.array([[0.5, -0.1, 0.3, -0.7]])
    idx = O.quantize(y, np.array([0.0]))
    np.testing.assert_array_equal(idx, [[1, 0, 1, 0]])
    r, gamma = O.residual_from_rotated(y, idx, c)
    np.testing.assert_allclose(r, [[0.07558681842161241, 0.3244131815783876, -0.1244131815783876,
                                    -0.27558681842161237]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(gamma, [0.44987110791772045], rtol=1e-15)


def test_residual_from_rotated_mean_square_is_distortion():
    # Over uniform unit vectors (Gaussian draws normalized; a rotation leaves
    # that law unchanged), E[gamma^2] = E||y - c[idx]||^2 is the codebook's
    # distortion D, which is pinned to quadrature and to closed forms above.
    # The function also equals encode()'s own residual on the same rows.
    d = 128
    rng = np.random.default_rng(21)
    g = rng.standard_normal((20000, d))
    y = g / np.linalg.norm(g, axis=1, keepdims=True)
    for bits in (1, 2, 3):
        c, t = O.build_codebook(d, bits)
        idx = O.quantize(y, t)
        r, gamma = O.residual_from_rotated(y, idx, c)
        D = O.codebook_distortion(d, c.astype(np.float64), t.astype(np.float64))
        g2 = gamma * gamma
        assert abs(g2.mean() - D) < 3.0 * g2.std() / math.sqrt(g2.size)
        e = O.encode(y[:200], np.eye(d), c, t, O.qjl_matrix(32, d, 3))
        r2, gamma2 = O.residual_from_rotated(e["y"], e["idx"], c)
        np.testing.assert_allclose(r2, e["r"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(gamma2, e["gamma"], rtol=1e-14)


# ---------------------------------------------------------------- QJL estimator

def test_qjl_unbiased_1e5_trials():
    # Mean error of the 1-bit estimate over 10^5 seeded draws of S lies within
    # 3 standard errors of zero (the pages: QJL's inner-product estimate is unbiased).
    rng = np.random.default_rng(11)
    d, m, trials = 128, 16, 100_000
    q = rng.standard_normal(d)
    r = rng.standard_normal(d) * 0.05
    gamma = np.linalg.norm(r)
    true = float(q @ r)
    errs = []
    for chunk in range(10):
        g = np.random.default_rng(1000 + chunk)
        for _ in range(10_000 // 1000):
            S = g.standard_normal((1000, m, d))
            z = np.einsum("tmd,d->tm", S, r) > 0
            sq = np.einsum("tmd,d->tm", S, q)
            est = math.sqrt(math.pi / 2) / m * gamma * np.sum(sq * np.where(z, 1.0, -1.0), axis=1)
            # same numbers through the oracle's estimator for a few trials
            if len(errs) == 0:
                for k in range(3):
                    assert abs(O.qjl_estimate(q, S[k], z[k], gamma) - est[k]) < 1e-12
            errs.append(est - true)
    errs = np.concatenate(errs)
    assert errs.size == trials
    se = errs.std() / math.sqrt(trials)
    assert abs(errs.mean()) < 3.0 * se
    # closed-form variance: gamma^2/m * (pi/2 |q|^2 - <q, r/gamma>^2)
    var = gamma ** 2 / m * (math.pi / 2 * (q @ q) - (q @ r / gamma) ** 2)
    assert abs(errs.var() / var - 1.0) < 0.02


def test_qjl_estimate_flipped_signs_is_biased():
    # The sign convention matters: using 2z-1 with z = [p > 0] is unbiased; the
    # opposite convention estimates -<q,r>.
    rng = np.random.default_rng(12)
    d, m = 64, 4096
    q = rng.standard_normal(d)
    r = rng.standard_normal(d)
    S = rng.standard_normal((m, d))
    z = (S @ r) > 0
    est = O.qjl_estimate(q, S, z, np.linalg.norm(r))
    assert abs(est - q @ r) < 0.15 * np.linalg.norm(q) * np.linalg.norm(r)
    assert abs(O.qjl_estimate(q, S, ~z, np.linalg.norm(r)) + q @ r) < 0.15 * np.linalg.norm(q) * np.linalg.norm(r)


def test_one_bit_mse_inner_product_bias(golden_dir):
    # The page: a 1-bit MSE-optimal quantizer shrinks inner products by 2/pi.
    # For the sphere law the slope is d * c^2 (c = E|Y|), tending to 2/pi.
    g = _load(golden_dir, "page_bounds.json")
    c, _, _ = O.lloyd_max(4096, 1)
    assert abs(4096 * c[1] ** 2 - g["one_bit_inner_product_bias"]) < 1e-3
    d = 128
    Pi = O.haar_rotation(d, 0)
    c32, t32 = O.build_codebook(d, 1)
    rng = np.random.default_rng(13)
    k = rng.standard_normal((20000, d))
    q = rng.standard_normal(d)
    e = O.encode(k, Pi, c32, t32)
    khat = (c32.astype(np.float64)[e["idx"]] @ Pi) * e["nu"][:, None]
    slope = np.polyfit(k @ q, khat @ q, 1)[0]
    assert abs(slope - d * float(c32[1]) ** 2) < 0.01
    assert abs(slope - g["one_bit_inner_product_bias"]) < 0.02


def test_mse_inner_product_slope_is_one_minus_distortion():
    # Centroid condition: E[y Q(y)] = E[Q(y)^2], so for a rotation-invariant
    # key law E<q, k_hat> = (1 - D) <q, k> exactly, at every width (the 1-bit
    # case is the 2/pi shrinkage above); the slope over 20000 keys must match.
    d = 128
    Pi = O.haar_rotation(d, 0)
    rng = np.random.default_rng(13)
    k = rng.standard_normal((20000, d))
    q = rng.standard_normal(d)
    exact = k @ q
    for bits in (1, 2, 3, 4):
        c, t = O.build_codebook(d, bits)
        D = O.codebook_distortion(d, c.astype(np.float64), t.astype(np.float64))
        e = O.encode(k, Pi, c, t)
        est = ((c.astype(np.float64)[e["idx"]] @ Pi) * e["nu"][:, None]) @ q
        slope = (est @ exact) / (exact @ exact)
        se = math.sqrt((est - slope * exact).var() / (exact @ exact))
        assert abs(slope - (1.0 - D)) < 4.0 * se


# ---------------------------------------------------------------- decode

def _lossless_cache(rng, B, Hkv, T, d, kbits, vbits, Pi):
    """K, V whose rotated directions are exact centroid vectors (lossless codes)."""
    ck, _ = O.build_codebook(d, kbits)
    cv, _ = O.build_codebook(d, vbits)
    k_idx = rng.integers(0, 1 << kbits, size=(B, Hkv, T, d))
    v_idx = rng.integers(0, 1 << vbits, size=(B, Hkv, T, d))
    k_nu = rng.uniform(0.5, 3.0, size=(B, Hkv, T))
    v_nu = rng.uniform(0.5, 3.0, size=(B, Hkv, T))
    K = (ck.astype(np.float64)[k_idx] @ Pi) * k_nu[..., None]
    V = (cv.astype(np.float64)[v_idx] @ Pi) * v_nu[..., None]
    kc = {"codes": O.pack_bits(k_idx.reshape(-1, d), kbits).reshape(B, Hkv, T, -1),
          "signs": None, "norms": k_nu, "res_norms": None}
    vc = {"codes": O.pack_bits(v_idx.reshape(-1, d), vbits).reshape(B, Hkv, T, -1), "norms": v_nu}
    return K, V, kc, vc, ck, cv


def test_decode_reduces_to_textbook_attention():
    # With lossless codes and no QJL term the decode must equal plain softmax
    # attention on the (dequantized) keys/values, including GQA and ragged lengths.
    rng = np.random.default_rng(14)
    B, Hq, Hkv, T, d = 2, 4, 2, 37, 16
    Pi = O.haar_rotation(d, 9)
    K, V, kc, vc, ck, cv = _lossless_cache(rng, B, Hkv, T, d, 2, 3, Pi)
    q = rng.standard_normal((B, Hq, d))
    seq_len = [T, 11]
    kb = {"bits": 2, "centroids": ck, "Pi": Pi, "S": None}
    vb = {"bits": 3, "centroids": cv, "Pi": Pi}
    out, sc = O.decode_attention(q, kc, vc, seq_len, kb, vb, return_scores=True)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            T_b = seq_len[b]
            ref = O.exact_attention(q[b, h], K[b, h // g, :T_b], V[b, h // g, :T_b])
            np.testing.assert_allclose(out[b, h], ref, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(sc[b, h, :T_b], K[b, h // g, :T_b] @ q[b, h] / math.sqrt(d), rtol=1e-10, atol=1e-12)
            assert np.all(np.isnan(sc[b, h, T_b:]))
    # an explicit scale is honoured
    out2 = O.decode_attention(q, kc, vc, seq_len, kb, vb, scale=0.3)
    ref2 = O.exact_attention(q[0, 0], K[0, 0], V[0, 0], scale=0.3)
    np.testing.assert_allclose(out2[0, 0], ref2, rtol=1e-11)


def test_decode_scores_unbiased_over_qjl_draws():
    # End to end through encode and decode_scores: averaged over draws of S,
    # the estimated logit equals the exact logit scale * <q, k>.
    rng = np.random.default_rng(15)
    d, m, n_draws = 16, 16, 4000
    Pi = O.haar_rotation(d, 3)
    c, t = O.build_codebook(d, 2)
    k = rng.standard_normal((3, d))
    q = rng.standard_normal(d)
    exact = (k @ q) / math.sqrt(d)
    ests = []
    for s in range(n_draws):
        S = rng.standard_normal((m, d))
        e = O.encode(k, Pi, c, t, S)
        ests.append(O.decode_scores(q, Pi, c, S, e["idx"], e["nu"], e["gamma"], e["z"], 1 / math.sqrt(d)))
    ests = np.array(ests)
    se = ests.std(axis=0) / math.sqrt(n_draws)
    assert np.all(np.abs(ests.mean(axis=0) - exact) < 3.5 * se + 1e-12)
    # without the QJL term the codebook-only logit is biased for b' = 2
    mse_only = O.decode_scores(q, Pi, c, None, e["idx"], e["nu"], None, None, 1 / math.sqrt(d))
    assert np.any(np.abs(mse_only - exact) > 5 * se)


def test_decode_empty_sequence_gives_zero():
    rng = np.random.default_rng(16)
    d = 8
    Pi = O.haar_rotation(d, 0)
    K, V, kc, vc, ck, cv = _lossless_cache(rng, 1, 1, 4, d, 1, 1, Pi)
    kb = {"bits": 1, "centroids": ck, "Pi": Pi, "S": None}
    vb = {"bits": 1, "centroids": cv, "Pi": Pi}
    out = O.decode_attention(rng.standard_normal((1, 2, d)), kc, vc, [0], kb, vb)
    assert np.all(out == 0.0)


def test_chunk_attention_is_causal_masked_attention():
    # Lossless codes, no QJL term: the chunk's output must equal textbook
    # attention of the n_new queries with the standard causal mask (query j at
    # position seq_len - n_new + j sees keys at positions <= its own), written
    # here as one masked score matrix per (b, head), including a sequence
    # shorter than the chunk (its first queries see nothing: zero output).
    rng = np.random.default_rng(17)
    B, Hq, Hkv, T, d, n_new = 3, 4, 2, 23, 16, 5
    Pi = O.haar_rotation(d, 4)
    K, V, kc, vc, ck, cv = _lossless_cache(rng, B, Hkv, T, d, 2, 2, Pi)
    q = rng.standard_normal((B, Hq, n_new, d))
    seq_len = [T, 12, 3]
    kb = {"bits": 2, "centroids": ck, "Pi": Pi, "S": None}
    vb = {"bits": 2, "centroids": cv, "Pi": Pi}
    out = O.chunk_attention(q, kc, vc, seq_len, kb, vb)
    g = Hq // Hkv
    for b in range(B):
        pos = seq_len[b] - n_new + np.arange(n_new)           # query positions
        for h in range(Hq):
            s = q[b, h] @ K[b, h // g].T / math.sqrt(d)       # [n_new, T]
            mask = np.arange(T)[None, :] <= pos[:, None]
            s = np.where(mask, s, -np.inf)
            for j in range(n_new):
                if not mask[j].any():
                    assert np.all(out[b, h, j] == 0.0)
                    continue
                w = np.exp(s[j] - s[j].max())
                np.testing.assert_allclose(out[b, h, j], (w / w.sum()) @ V[b, h // g], rtol=1e-11, atol=1e-12)
    # the last query of the chunk is the single-query decode over seq_len
    dec = O.decode_attention(q[:, :, -1], kc, vc, seq_len, kb, vb)
    np.testing.assert_allclose(out[:, :, -1], dec, rtol=0, atol=0)
