"""Pins of the oracle's split-width functions (section 8 of oracle/tq_oracle.py)
against closed forms, the uniform case they reduce to, brute force and Monte
Carlo.  CPU only."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle as O


def test_split_widths_average_bits():
    w = O.split_widths(128, 2, 64)
    assert w.sum() == 128 * 2 + 64 and w.mean() == 2.5
    assert np.all(w[:64] == 3) and np.all(w[64:] == 2)
    assert O.split_widths(128, 3, 64).mean() == 3.5
    with pytest.raises(ValueError):
        O.split_widths(8, 2, 9)


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_split_distortion_is_coordinate_weighted_mean(bits):
    # Every rotated coordinate has the law f_d, so the split's distortion is
    # the coordinate-weighted mean of the two widths' D, exactly.
    d = 128
    cw, tw = O.build_codebook(d, bits + 1)
    cn, tn = O.build_codebook(d, bits)
    Dw = O.codebook_distortion(d, cw.astype(np.float64), tw.astype(np.float64))
    Dn = O.codebook_distortion(d, cn.astype(np.float64), tn.astype(np.float64))
    for n_wide in (0, 32, 64, 96, 128):
        D = O.split_distortion(d, O.build_split_book(d, bits, n_wide))
        assert abs(D - (n_wide * Dw + (d - n_wide) * Dn) / d) <= 1e-13 * D
    # strictly between the two widths' distortions for a proper split
    D64 = O.split_distortion(d, O.build_split_book(d, bits, 64))
    assert Dw < D64 < Dn


def test_split_encode_error_matches_distortion_monte_carlo():
    d, bits, n_wide = 128, 2, 64
    Pi = O.haar_rotation(d, 0)
    book = O.build_split_book(d, bits, n_wide)
    x = np.random.default_rng(21).standard_normal((20000, d))
    e = O.encode_split(x, Pi, book)
    u = x / e["nu"][:, None]
    uhat = O.dequant_split(e["idx"], book) @ Pi          # Pi^T y_hat, row form
    err = np.sum((u - uhat) ** 2, axis=1)
    D = O.split_distortion(d, book)
    assert abs(err.mean() - D) < 4.0 * err.std() / math.sqrt(err.size)
    # each half alone: d times its per-coordinate squared error is its width's D
    sq = (e["y"] - O.dequant_split(e["idx"], book)) ** 2
    for sl, (c, t) in ((slice(0, n_wide), book["wide"]), (slice(n_wide, d), book["narrow"])):
        per = d * sq[:, sl].mean(axis=1)
        Dh = O.codebook_distortion(d, c.astype(np.float64), t.astype(np.float64))
        assert abs(per.mean() - Dh) < 4.0 * per.std() / math.sqrt(per.size)


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_split_reduces_to_uniform_encode(bits):
    d, m = 32, 32
    Pi = O.haar_rotation(d, 2)
    S = O.qjl_matrix(m, d, 3)
    x = np.random.default_rng(22 + bits).standard_normal((64, d))
    for n_wide, width in ((0, bits), (d, bits + 1)):
        c, t = O.build_codebook(d, width)
        ref = O.encode(x, Pi, c, t, S)
        got = O.encode_split(x, Pi, O.build_split_book(d, bits, n_wide), S)
        np.testing.assert_array_equal(got["idx"], ref["idx"])
        np.testing.assert_array_equal(got["z"], ref["z"])
        np.testing.assert_allclose(got["gamma"], ref["gamma"], rtol=0, atol=0)
        np.testing.assert_array_equal(O.pack_bits_widths(got["idx"], O.split_widths(d, bits, n_wide)),
                                      O.pack_bits(ref["idx"], width))


def test_split_quantize_halves_use_their_own_codebook():
    # Coordinates in [0, n_wide) are brute-force nearest (b+1)-bit centroids,
    # the rest nearest b-bit centroids.
    d, bits, n_wide = 8, 2, 4
    book = O.build_split_book(d, bits, n_wide)
    y = np.random.default_rng(23).uniform(-0.9, 0.9, size=(500, d))
    idx = O.quantize_split(y, book)
    for sl, c in ((slice(0, n_wide), book["wide"][0]), (slice(n_wide, d), book["narrow"][0])):
        near = np.argmin(np.abs(y[:, sl, None] - c.astype(np.float64)[None, None, :]), axis=2)
        np.testing.assert_array_equal(idx[:, sl], near)
    assert idx[:, :n_wide].max() >= 4 and idx[:, n_wide:].max() <= 3


def test_pack_widths_hand_worked():
    # widths (3, 3, 2, 2), codes (5, 2, 3, 1): 5 | 2 << 3 | 3 << 6 | 1 << 8 = 0x1D5
    w = O.pack_bits_widths(np.array([[5, 2, 3, 1]]), [3, 3, 2, 2])
    assert w.shape == (1, 1) and int(w[0, 0]) == 0x1D5
    # d = 128, 64 x 3 + 64 x 2 bits = 10 words: wide codes all 7 fill words 0..5
    v = np.zeros((1, 128), dtype=np.int64)
    v[0, :64] = 7
    w = O.pack_bits_widths(v, O.split_widths(128, 2, 64))
    assert w.shape == (1, 10)
    assert np.all(w[0, :6] == 0xFFFFFFFF) and np.all(w[0, 6:] == 0)
    # narrow code 64 (first after the wide block) sits at bit 192 = word 6, bit 0
    v = np.zeros((1, 128), dtype=np.int64)
    v[0, 64] = 3
    v[0, 10] = 7          # wide code 10: bits 30..32, straddles words 0 and 1
    w = O.pack_bits_widths(v, O.split_widths(128, 2, 64))
    assert int(w[0, 0]) == 0xC0000000 and int(w[0, 1]) == 1 and int(w[0, 6]) == 3


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_pack_widths_matches_big_integer_stream(bits):
    d, n_wide = 128, 64
    widths = O.split_widths(d, bits, n_wide)
    rng = np.random.default_rng(30 + bits)
    v = np.concatenate((rng.integers(0, 1 << (bits + 1), size=(4, n_wide)),
                        rng.integers(0, 1 << bits, size=(4, d - n_wide))), axis=1)
    w = O.pack_bits_widths(v, widths)
    for r in range(4):
        stream, off = 0, 0
        for j in range(d):
            stream |= int(v[r, j]) << off
            off += int(widths[j])
        assert [int(x) for x in w[r]] == [(stream >> (32 * k)) & 0xFFFFFFFF for k in range(off // 32)]
    np.testing.assert_array_equal(O.unpack_bits_widths(w, widths), v)


def test_book_codes_index_each_width_table():
    d, bits, n_wide = 128, 2, 64
    book = O.build_split_book(d, bits, n_wide)
    rng = np.random.default_rng(24)
    idx = O.quantize_split(rng.uniform(-0.3, 0.3, size=(7, d)), book)
    words = O.pack_bits_widths(idx, O.split_widths(d, bits, n_wide))
    table = O.book_table(book)
    np.testing.assert_array_equal(table[O.book_codes(book, words, d)], O.dequant_split(idx, book))
    # a uniform book reads plain codes
    c, _ = O.build_codebook(d, bits)
    ub = {"bits": bits, "centroids": c}
    np.testing.assert_array_equal(O.book_codes(ub, O.pack_bits(idx % 4, bits), d), idx % 4)


def _split_lossless_cache(rng, B, Hkv, T, d, kbook, vbook, Pi):
    """K, V whose rotated directions are exact split-centroid vectors."""
    def draw(book):
        nw, b = book["n_wide"], book["bits"]
        idx = np.concatenate((rng.integers(0, 1 << (b + 1), size=(B, Hkv, T, nw)),
                              rng.integers(0, 1 << b, size=(B, Hkv, T, d - nw))), axis=-1)
        nu = rng.uniform(0.5, 3.0, size=(B, Hkv, T))
        X = (O.dequant_split(idx, book) @ Pi) * nu[..., None]
        codes = O.pack_bits_widths(idx.reshape(-1, d), O.split_widths(d, b, nw)).reshape(B, Hkv, T, -1)
        return X, codes, nu
    K, kcodes, knu = draw(kbook)
    V, vcodes, vnu = draw(vbook)
    return K, V, {"codes": kcodes, "signs": None, "norms": knu, "res_norms": None}, {"codes": vcodes, "norms": vnu}


def test_split_decode_reduces_to_textbook_attention():
    rng = np.random.default_rng(25)
    B, Hq, Hkv, T, d = 2, 4, 2, 29, 32
    Pi = O.haar_rotation(d, 6)
    kb = dict(O.build_split_book(d, 1, 16), Pi=Pi, S=None)
    vb = dict(O.build_split_book(d, 2, 16), Pi=Pi)
    K, V, kc, vc = _split_lossless_cache(rng, B, Hkv, T, d, kb, vb, Pi)
    q = rng.standard_normal((B, Hq, d))
    seq_len = [T, 9]
    out, sc = O.decode_attention(q, kc, vc, seq_len, kb, vb, return_scores=True)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            Tb = seq_len[b]
            ref = O.exact_attention(q[b, h], K[b, h // g, :Tb], V[b, h // g, :Tb])
            np.testing.assert_allclose(out[b, h], ref, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(sc[b, h, :Tb], K[b, h // g, :Tb] @ q[b, h] / math.sqrt(d), rtol=1e-10, atol=1e-12)


def test_split_keys_logit_unbiased_over_qjl_draws():
    # The QJL correction of the split residual keeps the logit unbiased.
    rng = np.random.default_rng(26)
    d, m, n_draws = 16, 16, 4000
    Pi = O.haar_rotation(d, 5)
    book = O.build_split_book(d, 1, 8)
    k = rng.standard_normal((3, d))
    q = rng.standard_normal(d)
    exact = (k @ q) / math.sqrt(d)
    ests = []
    for _ in range(n_draws):
        S = rng.standard_normal((m, d))
        e = O.encode_split(k, Pi, book, S)
        idx = O.book_codes(book, O.pack_bits_widths(e["idx"], O.split_widths(d, 1, 8)), d)
        ests.append(O.decode_scores(q, Pi, O.book_table(book), S, idx, e["nu"], e["gamma"], e["z"], 1 / math.sqrt(d)))
    ests = np.array(ests)
    se = ests.std(axis=0) / math.sqrt(n_draws)
    assert np.all(np.abs(ests.mean(axis=0) - exact) < 3.5 * se + 1e-12)
