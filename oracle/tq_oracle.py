"""TurboQuant CPU oracle: plain, slow, float64 numpy.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library (no common helpers, tables or constants): everything here is written
from the method's description, step by step, so a reader can check it against
the pages by eye.

Pages cited (short tags used in every docstring below):

* [memory-wall §2]   admirer.cn article on TurboQuant and the memory wall,
                     section 2 "What does TurboQuant actually do", with its
                     "stage one" (random rotation + MSE-optimal scalar
                     quantization) and "stage two" (QJL residual correction)
                     parts, and the distortion-bound paragraph and figure
                     caption that close the section.
* [memory-wall §1]   same article, section 1 (KV cache and the memory wall:
                     decode is memory-bound).
* [explainer §2]     cc-newplayer explainer "Google TurboQuant KV-cache
                     compression explained", technical breakdown item 2
                     (rotation pre-conditioning and its core-formula box).
* [explainer §4]     same page, item 4 (the flow graph: Q is not compressed,
                     K and V are rotated, quantized, cached, and attention
                     runs with dequantization).
* [3-bit §2.1.2]     intelliparadigm article "TurboQuant: a 3-bit lossless
                     compression scheme", §2.1.2 QJL residual correction
                     (projection, `> 0` binarization, unbiased estimator).
* [3-bit §2.1.1]     same article, §2.1.1 step 1 (Haar random rotation).
* [3-bit §2.2]       same article, §2.2 Theorem 2 (unbiasedness, variance).

Readings taken where the pages are silent or garbled are listed per function.
Pinned against: closed forms, textbook limits, brute force and the pages'
bounds (tests/test_oracle_pins.py).  Every function below has at least one pin.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import betainc, gammaln

# --------------------------------------------------------------------------
# 1. Coordinate law of a rotated unit vector  [memory-wall §2, stage one]
# --------------------------------------------------------------------------


def coord_norm_const(d: int) -> float:
    """Normalizing constant of f_d(t) = C_d (1-t^2)^((d-3)/2) on [-1, 1].

    C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)).  The page states that each
    coordinate of a randomly rotated unit vector follows a Beta law (normal in
    high dimension); this is that law written on [-1, 1].
    """
    return math.exp(gammaln(d / 2.0) - 0.5 * math.log(math.pi) - gammaln((d - 1) / 2.0))


def coord_pdf(t, d: int):
    """Density f_d(t) of one coordinate of a uniform point on S^{d-1}."""
    t = np.asarray(t, dtype=np.float64)
    k = (d - 3) / 2.0
    return coord_norm_const(d) * np.power(np.clip(1.0 - t * t, 0.0, None), k)


def coord_cdf(t, d: int):
    """P(Y <= t) for Y ~ f_d: the regularized incomplete beta I_{(1+t)/2}(a, a), a=(d-1)/2."""
    t = np.clip(np.asarray(t, dtype=np.float64), -1.0, 1.0)
    a = (d - 1) / 2.0
    return betainc(a, a, (1.0 + t) / 2.0)


def coord_partial_mean(t, d: int):
    """Integral of s f_d(s) ds from -1 to t.

    Closed form: d/dt (1-t^2)^(k+1) = -2(k+1) t (1-t^2)^k with k=(d-3)/2, so the
    integral equals -C_d (1-t^2)^(k+1) / (2(k+1)).
    """
    t = np.clip(np.asarray(t, dtype=np.float64), -1.0, 1.0)
    k1 = (d - 1) / 2.0
    return -coord_norm_const(d) * np.power(1.0 - t * t, k1) / (2.0 * k1)


# --------------------------------------------------------------------------
# 2. Lloyd-Max codebook  [memory-wall §2, stage one]
# --------------------------------------------------------------------------


def lloyd_max(d: int, bits: int, tol: float = 1e-15, max_iter: int = 200000):
    """Lloyd-Max scalar quantizer for f_d with L = 2**bits levels.

    The page calls it a one-dimensional continuous k-means on the known
    coordinate law, solved once per bit width and stored.  Steps (Lloyd's
    iteration): thresholds are midpoints of neighbouring centroids; each
    centroid is the conditional mean of its cell.  Reading: start from a
    symmetric equal-spaced guess, stop when no centroid moves by `tol`
    (1e-15: the iteration contracts slowly at 4 bits, so a looser stop would
    leave ~1e-12 of error, enough to move an fp32 rounding).  The
    law is even, so the optimum is symmetric; each step is symmetrized
    (c <- (c - reversed c)/2) so that rounding cannot tilt it and the middle
    threshold is exactly 0.

    Returns (centroids[L], thresholds[L-1], iterations) in float64.
    """
    L = 1 << bits
    sigma = 1.0 / math.sqrt(d)
    c = np.linspace(-1.0, 1.0, L) * min(0.9, 2.0 * sigma)
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        mass = np.diff(coord_cdf(edges, d))
        moment = np.diff(coord_partial_mean(edges, d))
        c_new = moment / mass
        c_new = 0.5 * (c_new - c_new[::-1])
        step = np.max(np.abs(c_new - c))
        c = c_new
        if step < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, it


def codebook_distortion(d: int, centroids, thresholds) -> float:
    """D = E||u - u_hat||^2 for a unit vector u, per the quantizer (c, t).

    Per coordinate the MSE is E[Y^2] - 2 sum c_i E[Y; cell i] + sum c_i^2 P_i,
    and E[Y^2] = 1/d because the d squared coordinates of a unit vector sum to
    one; D is d times the per-coordinate MSE.  This is the quantity the page's
    distortion bounds (lower 4^-b, upper sqrt(3) pi / 2 * 4^-b) speak of.
    """
    c = np.asarray(centroids, dtype=np.float64)
    edges = np.concatenate(([-1.0], np.asarray(thresholds, dtype=np.float64), [1.0]))
    mass = np.diff(coord_cdf(edges, d))
    moment = np.diff(coord_partial_mean(edges, d))
    per_coord = 1.0 / d - 2.0 * np.sum(c * moment) + np.sum(c * c * mass)
    return d * per_coord


def build_codebook(d: int, bits: int):
    """Stored codebook: fp32 centroids and fp32 midpoints (rounded from float64)."""
    c, t, _ = lloyd_max(d, bits)
    return c.astype(np.float32), t.astype(np.float32)


# --------------------------------------------------------------------------
# 3. Seeded Gaussian draws (the pages name no generator)
# --------------------------------------------------------------------------
# Reading: SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) as a counter stream:
# output i of seed s is mix(s + (i+1) * 0x9E3779B97F4A7C15 mod 2^64) with the
# variant-13 finalizer; a uniform is (z >> 11) * 2^-53; normals come in
# Box-Muller pairs, cos first, then sin.

_GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)


def splitmix64(seed: int, n: int) -> np.ndarray:
    """First n SplitMix64 outputs for state `seed` (uint64 array)."""
    with np.errstate(over="ignore"):
        i = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def gaussian_stream(seed: int, n: int) -> np.ndarray:
    """First n standard normals of the seeded stream (float64)."""
    npairs = (n + 1) // 2
    z = splitmix64(seed, 2 * npairs)
    u = (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    u1 = 1.0 - u[0::2]          # in (0, 1]
    u2 = u[1::2]                # in [0, 1)
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(2 * npairs, dtype=np.float64)
    out[0::2] = r * np.cos(2.0 * math.pi * u2)
    out[1::2] = r * np.sin(2.0 * math.pi * u2)
    return out[:n]


def gaussian_matrix(seed: int, rows: int, cols: int) -> np.ndarray:
    """rows x cols iid N(0,1), filled row-major from the seeded stream."""
    return gaussian_stream(seed, rows * cols).reshape(rows, cols)


# --------------------------------------------------------------------------
# 4. Rotation and QJL matrices  [explainer §2], [3-bit §2.1.1], [3-bit §2.1.2]
# --------------------------------------------------------------------------


def haar_rotation(d: int, seed: int) -> np.ndarray:
    """Haar-random orthogonal Pi (d x d), convention y = Pi @ x.

    The pages ask for a random orthogonal matrix drawn from the Haar law.
    Steps: Gaussian G (row-major from the seeded stream); QR factorization
    G = QR; Pi = Q diag(sign(diag R)), which makes the factorization unique and
    Pi Haar-distributed (Mezzadri, Notices AMS 2007).
    """
    g = gaussian_matrix(seed, d, d)
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]


def qjl_matrix(m: int, d: int, seed: int) -> np.ndarray:
    """QJL projection S (m x d), iid N(0,1) entries [3-bit §2.1.2]."""
    return gaussian_matrix(seed, m, d)


# --------------------------------------------------------------------------
# 5. Encode  [memory-wall §2, stages one and two]
# --------------------------------------------------------------------------


def quantize(y, thresholds) -> np.ndarray:
    """idx_j = #{i : y_j >= t_i}: pure threshold lookup, no scale or zero point.

    Reading: a value equal to a threshold goes to the upper cell; NaN compares
    false everywhere and gets code 0.  The comparison happens in the precision
    of `y` against the stored (fp32) thresholds.
    """
    y = np.asarray(y)
    t = np.asarray(thresholds)
    idx = np.zeros(y.shape, dtype=np.int64)
    for ti in t:
        idx += (y >= ti)
    return idx


def encode(x, Pi, centroids, thresholds, S=None):
    """Encode vectors x[n, d] (any float dtype; arithmetic in float64).

    Stage one: nu = ||x||; u = x / nu (u = 0 when nu = 0); y = Pi u;
    idx = quantize(y).  Stage two (keys only, S given): residual r = y - c[idx]
    in the rotated domain; gamma = ||r||; p = S r; sign bit z = [p > 0].
    Reading: the residual and S live in the rotated domain, which has the same
    law as an original-domain residual with S' = S Pi; gamma is stored because
    the unbiased estimator needs the residual's length.
    Returns a dict with nu, y, idx and (keys) r, gamma, p, z.
    """
    x = np.asarray(x, dtype=np.float64)
    Pi = np.asarray(Pi, dtype=np.float64)
    nu = np.sqrt(np.sum(x * x, axis=1))
    with np.errstate(invalid="ignore", divide="ignore"):
        inv = np.where(nu == 0.0, 0.0, 1.0 / nu)
    u = x * inv[:, None]
    y = u @ Pi.T
    idx = quantize(y, thresholds)
    out = {"nu": nu, "y": y, "idx": idx}
    if S is not None:
        c = np.asarray(centroids, dtype=np.float64)
        r = y - c[idx]
        gamma = np.sqrt(np.sum(r * r, axis=1))
        p = r @ np.asarray(S, dtype=np.float64).T
        out.update(r=r, gamma=gamma, p=p, z=(p > 0))
    return out


def residual_from_rotated(y, idx, centroids):
    """r = y - c[idx] and gamma = ||r|| for given rotated values (float64)."""
    r = np.asarray(y, dtype=np.float64) - np.asarray(centroids, dtype=np.float64)[idx]
    return r, np.sqrt(np.sum(r * r, axis=1))


# --------------------------------------------------------------------------
# 6. Bit packing (storage format of the compressed cache)
# --------------------------------------------------------------------------
# Reading: code j of a vector occupies bits [j*b, (j+1)*b) of that vector's
# bitstream, least significant bit first; stream bit k is bit (k mod 32) of
# little-endian uint32 word k div 32.  Sign bit i is stream bit i of the
# vector's sign words.


def pack_bits(vals, bits: int) -> np.ndarray:
    """Pack small non-negative ints vals[n, d] into uint32 words [n, d*bits/32]."""
    vals = np.asarray(vals, dtype=np.int64)
    n, d = vals.shape
    nwords = (d * bits + 31) // 32
    words = np.zeros((n, nwords), dtype=np.uint64)
    for j in range(d):
        for b in range(bits):
            k = j * bits + b
            bit = ((vals[:, j] >> b) & 1).astype(np.uint64)
            words[:, k // 32] |= bit << np.uint64(k % 32)
    return words.astype(np.uint32)


def unpack_bits(words, d: int, bits: int) -> np.ndarray:
    """Inverse of pack_bits: uint32 words [n, *] -> ints [n, d]."""
    words = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    n = words.shape[0]
    vals = np.zeros((n, d), dtype=np.int64)
    for j in range(d):
        for b in range(bits):
            k = j * bits + b
            bit = (words[:, k // 32] >> np.uint64(k % 32)) & np.uint64(1)
            vals[:, j] |= bit.astype(np.int64) << b
    return vals


# --------------------------------------------------------------------------
# 7. Decode attention  [explainer §4], [memory-wall §2 stage two], [3-bit §2.1.2]
# --------------------------------------------------------------------------


def qjl_estimate(q_rot, S, z, gamma):
    """Unbiased estimate of <q, r> from the 1-bit sketch z = [S r > 0].

    <q, r> ~ sqrt(pi/2) / m * gamma * <S q, 2z - 1>.  Reading: the query is
    projected at full precision (only the key side is 1-bit), and the constant
    follows from E[(s.q) sign(s.r)] = sqrt(2/pi) <q, r>/||r|| for Gaussian s;
    the page's sign(Aq)*sign(Ae) form is biased and is not used.
    q_rot[..., d]; z[..., m] boolean; gamma[...] -> estimate[...].
    """
    S = np.asarray(S, dtype=np.float64)
    m = S.shape[0]
    sq = np.asarray(q_rot, dtype=np.float64) @ S.T
    sgn = np.where(np.asarray(z), 1.0, -1.0)
    return math.sqrt(math.pi / 2.0) / m * np.asarray(gamma, dtype=np.float64) * np.sum(sq * sgn, axis=-1)


def decode_scores(q, Pi_k, ck, S, k_idx, k_nu, k_gamma, k_z, scale):
    """Scaled logits for one query against T compressed keys.

    q[d]; k_idx[T, d]; k_nu[T]; k_gamma[T]; k_z[T, m] (None for MSE-only keys).
    l_t = scale * nu_t * (<Pi q, c[idx_t]> + qjl_estimate).  Rotating the query
    once replaces un-rotating every key: (R q).(R k) = q.k for orthogonal R
    [explainer §2].
    """
    q_rot = np.asarray(Pi_k, dtype=np.float64) @ np.asarray(q, dtype=np.float64)
    khat = np.asarray(ck, dtype=np.float64)[k_idx]
    dot = khat @ q_rot
    if k_z is not None:
        dot = dot + qjl_estimate(q_rot[None, :], S, k_z, k_gamma)
    return scale * np.asarray(k_nu, dtype=np.float64) * dot


def softmax(l):
    """Two-pass softmax with max subtraction (float64)."""
    l = np.asarray(l, dtype=np.float64)
    if l.size == 0:
        return l
    e = np.exp(l - np.max(l))
    return e / np.sum(e)


def dequant_values(Pi_v, cv, v_idx, v_nu):
    """Original-domain dequantized values nu_t * Pi^T c[idx_t]  [T, d]."""
    rot = np.asarray(cv, dtype=np.float64)[v_idx] * np.asarray(v_nu, dtype=np.float64)[:, None]
    return rot @ np.asarray(Pi_v, dtype=np.float64)


def decode_attention(q, kcache, vcache, seq_len, kbook, vbook, scale=None, return_scores=False):
    """Single-query decode attention over a compressed KV cache.

    q[B, Hq, d].  kcache: dict(codes[B,Hkv,Tcap,Wk] u32, signs[B,Hkv,Tcap,Ws] u32
    or None, norms[B,Hkv,Tcap], res_norms or None).  vcache: dict(codes, norms).
    kbook/vbook: dict(bits, centroids, Pi, S (keys, or None)); a split-width
    book (section 8) has n_wide > 0 and the wide / narrow codebooks instead of
    centroids, and its records are read with book_codes / book_table.
    q-head h reads KV head h // (Hq/Hkv).  Scale defaults to 1/sqrt(d).  No
    mask: the decode query sees all seq_len[b] cached tokens.  An empty cache
    (seq_len 0) gives a zero output.  Steps: scores (decode_scores), softmax,
    o = sum_t p_t * nu_t Pi^T c_v[idx_t]  (each token dequantized in the
    original domain).  Returns out[B, Hq, d] (and scores[B, Hq, Tcap], NaN
    past seq_len, when asked).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = kcache["norms"].shape[1]
    Tcap = kcache["norms"].shape[2]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, d))
    scores = np.full((B, Hq, Tcap), np.nan)
    m = 0 if kbook.get("S") is None else np.asarray(kbook["S"]).shape[0]
    for b in range(B):
        T = int(seq_len[b])
        for hk in range(Hkv):
            if T == 0:
                continue
            k_idx = book_codes(kbook, kcache["codes"][b, hk, :T], d)
            k_z = unpack_bits(kcache["signs"][b, hk, :T], m, 1).astype(bool) if m else None
            k_gamma = kcache["res_norms"][b, hk, :T] if m else None
            v_idx = book_codes(vbook, vcache["codes"][b, hk, :T], d)
            vdeq = dequant_values(vbook["Pi"], book_table(vbook), v_idx, vcache["norms"][b, hk, :T])
            for j in range(g):
                h = hk * g + j
                l = decode_scores(q[b, h], kbook["Pi"], book_table(kbook), kbook.get("S"),
                                  k_idx, kcache["norms"][b, hk, :T], k_gamma, k_z, scale)
                scores[b, h, :T] = l
                out[b, h] = softmax(l) @ vdeq
    if return_scores:
        return out, scores
    return out


def chunk_attention(q, kcache, vcache, seq_len, kbook, vbook, scale=None):
    """Causal attention of a chunk of n_new new queries per (b, q head) over the
    compressed cache  [memory-wall §1: each new token attends over the keys and
    values of every token up to itself; memory-wall §2: over the compressed
    cache].

    q[B, Hq, n_new, d].  The new tokens are the last n_new cached ones: query j
    of sequence b sits at position p = seq_len[b] - n_new + j and sees cached
    positions 0 .. p, i.e. clamp(p + 1, 0, Tcap) tokens (none: zero output).
    Each query is then a single-query decode over its own prefix.
    Returns out[B, Hq, n_new, d].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, n_new, d = q.shape
    Tcap = kcache["norms"].shape[2]
    out = np.zeros((B, Hq, n_new, d))
    for j in range(n_new):
        seen = [min(max(int(seq_len[b]) - n_new + j + 1, 0), Tcap) for b in range(B)]
        out[:, :, j] = decode_attention(q[:, :, j], kcache, vcache, seen, kbook, vbook, scale=scale)
    return out


def exact_attention(q, k, v, scale=None):
    """Textbook softmax attention of one query over uncompressed K, V (float64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return softmax(scale * (k @ q)) @ v


# --------------------------------------------------------------------------
# 8. Split bit widths  [explainer §1], [3-bit §2.1], [3-bit §5.1]
# --------------------------------------------------------------------------
# The pages quote fractional average widths (about 2.5 bits per element in the
# explainer's asymmetric mixed-precision item, a "2.5-bit" intermediate in the
# 3-bit article's pipeline figure, 3.5 bits in its limits section) without
# saying how a fraction is reached.  Reading: a fixed split of the d rotated
# coordinates -- the first n_wide get the (b+1)-bit Lloyd-Max codebook, the
# other d - n_wide the b-bit one -- for b + n_wide/d bits per coordinate (keys
# add their 1-bit sketch on top).  Every rotated coordinate follows the same
# law f_d, so each width's codebook is the uniform case's, and which
# coordinates are wide does not change the expected distortion.  Storage: code
# j starts at bit offset sum_{i<j} width_i of the vector's stream (the uniform
# layout of section 6 when every width is equal).


def split_widths(d: int, bits: int, n_wide: int) -> np.ndarray:
    """Per-coordinate widths: bits + 1 for j < n_wide, bits for the rest."""
    if not 0 <= n_wide <= d:
        raise ValueError("n_wide must lie in [0, d]")
    w = np.full(d, bits, dtype=np.int64)
    w[:n_wide] = bits + 1
    return w


def build_split_book(d: int, bits: int, n_wide: int) -> dict:
    """The two stored codebooks of a split: fp32 (centroids, thresholds) of
    widths bits + 1 ("wide") and bits ("narrow"), and the split point."""
    return {"bits": bits, "n_wide": n_wide, "wide": build_codebook(d, bits + 1), "narrow": build_codebook(d, bits)}


def quantize_split(y, split: dict) -> np.ndarray:
    """Each coordinate's code from its own width's thresholds (quantize())."""
    y = np.asarray(y)
    nw = split["n_wide"]
    idx = np.empty(y.shape, dtype=np.int64)
    idx[..., :nw] = quantize(y[..., :nw], split["wide"][1])
    idx[..., nw:] = quantize(y[..., nw:], split["narrow"][1])
    return idx


def dequant_split(idx, split: dict) -> np.ndarray:
    """Rotated reconstruction: coordinate j is its width's centroid c[idx_j]."""
    idx = np.asarray(idx, dtype=np.int64)
    nw = split["n_wide"]
    out = np.empty(idx.shape, dtype=np.float64)
    out[..., :nw] = np.asarray(split["wide"][0], dtype=np.float64)[idx[..., :nw]]
    out[..., nw:] = np.asarray(split["narrow"][0], dtype=np.float64)[idx[..., nw:]]
    return out


def encode_split(x, Pi, split: dict, S=None):
    """encode() with per-coordinate widths: the same stages, each rotated
    coordinate quantized by its own width's codebook; the residual (keys) is
    y minus that reconstruction."""
    x = np.asarray(x, dtype=np.float64)
    nu = np.sqrt(np.sum(x * x, axis=1))
    with np.errstate(invalid="ignore", divide="ignore"):
        inv = np.where(nu == 0.0, 0.0, 1.0 / nu)
    y = (x * inv[:, None]) @ np.asarray(Pi, dtype=np.float64).T
    idx = quantize_split(y, split)
    out = {"nu": nu, "y": y, "idx": idx}
    if S is not None:
        r = y - dequant_split(idx, split)
        gamma = np.sqrt(np.sum(r * r, axis=1))
        p = r @ np.asarray(S, dtype=np.float64).T
        out.update(r=r, gamma=gamma, p=p, z=(p > 0))
    return out


def coord_mse(d: int, centroids, thresholds) -> float:
    """E[(Y - c(Y))^2] for one coordinate Y ~ f_d under the quantizer (c, t)."""
    c = np.asarray(centroids, dtype=np.float64)
    edges = np.concatenate(([-1.0], np.asarray(thresholds, dtype=np.float64), [1.0]))
    mass = np.diff(coord_cdf(edges, d))
    moment = np.diff(coord_partial_mean(edges, d))
    return 1.0 / d - 2.0 * np.sum(c * moment) + np.sum(c * c * mass)


def split_distortion(d: int, split: dict) -> float:
    """E||u - u_hat||^2 of a unit vector under a split: the sum over the d
    rotated coordinates of each one's MSE under its own width's codebook."""
    nw = split["n_wide"]
    total = 0.0
    for j in range(d):
        c, t = split["wide"] if j < nw else split["narrow"]
        total += coord_mse(d, c, t)
    return total


def pack_bits_widths(vals, widths) -> np.ndarray:
    """Pack codes vals[n, d] with per-coordinate widths into uint32 words
    [n, ceil(sum(widths)/32)]: code j at bit offset sum_{i<j} widths_i."""
    vals = np.asarray(vals, dtype=np.int64)
    widths = np.asarray(widths, dtype=np.int64)
    n, d = vals.shape
    words = np.zeros((n, (int(widths.sum()) + 31) // 32), dtype=np.uint64)
    k = 0
    for j in range(d):
        for b in range(int(widths[j])):
            bit = ((vals[:, j] >> b) & 1).astype(np.uint64)
            words[:, k // 32] |= bit << np.uint64(k % 32)
            k += 1
    return words.astype(np.uint32)


def unpack_bits_widths(words, widths) -> np.ndarray:
    """Inverse of pack_bits_widths."""
    words = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    widths = np.asarray(widths, dtype=np.int64)
    n = words.shape[0]
    vals = np.zeros((n, widths.size), dtype=np.int64)
    k = 0
    for j in range(widths.size):
        for b in range(int(widths[j])):
            bit = (words[:, k // 32] >> np.uint64(k % 32)) & np.uint64(1)
            vals[:, j] |= bit.astype(np.int64) << b
            k += 1
    return vals


def book_codes(book: dict, words, d: int):
    """Codes of packed records under a decode book, as indices into
    book_table(book): plain codes for a uniform book; for a split book
    (n_wide > 0) the narrow coordinates' codes are offset past the wide
    codebook's entries, so that one table lookup gives every coordinate its
    own width's centroid."""
    nw = book.get("n_wide", 0)
    if not nw:
        return unpack_bits(words, d, book["bits"])
    idx = unpack_bits_widths(words, split_widths(d, book["bits"], nw))
    idx[..., nw:] += 1 << (book["bits"] + 1)
    return idx


def book_table(book: dict) -> np.ndarray:
    """Centroid table that book_codes indexes (the wide then the narrow
    codebook for a split book)."""
    if not book.get("n_wide", 0):
        return np.asarray(book["centroids"], dtype=np.float64)
    return np.concatenate((np.asarray(book["wide"][0], dtype=np.float64),
                           np.asarray(book["narrow"][0], dtype=np.float64)))
