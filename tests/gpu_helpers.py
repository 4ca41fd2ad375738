"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle as O
import online_vector_quantization_amd as T
from online_vector_quantization_amd import synth

DEV = torch.device("cuda", 0)
ROT_SEED, QJL_SEED = 0, 1

_books = {}


def oracle_book(bits: int, m: int, d: int = 128, wide: int = 0):
    """The oracle's decode book; wide > 0: split widths (the first `wide`
    rotated coordinates on the (bits + 1)-bit codebook)."""
    key = (bits, m, d, wide)
    if key not in _books:
        extra = {"Pi": O.haar_rotation(d, ROT_SEED), "S": O.qjl_matrix(m, d, QJL_SEED) if m else None}
        if wide:
            _books[key] = dict(O.build_split_book(d, bits, wide), **extra)
        else:
            c, t = O.build_codebook(d, bits)
            _books[key] = dict({"bits": bits, "centroids": c, "thresholds": t}, **extra)
    return _books[key]


def gpu_book(bits: int, m: int, wide: int = 0) -> T.Codebook:
    return T.Codebook(128, bits, m, ROT_SEED, QJL_SEED, device=0, wide_coords=wide)


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host_values(x: np.ndarray, dtype: str) -> np.ndarray:
    return synth.bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def encode_gpu(cb: T.Codebook, x_dev: torch.Tensor, rows: int = None, dst_row=None, debug=True):
    n = x_dev.shape[0]
    rows = n if rows is None else rows
    codes = torch.zeros(rows, cb.code_words, dtype=torch.int32, device=DEV)
    norms = torch.zeros(rows, dtype=torch.float32, device=DEV)
    signs = torch.zeros(rows, cb.sign_words, dtype=torch.int32, device=DEV) if cb.qjl_dim else None
    res = torch.zeros(rows, dtype=torch.float32, device=DEV) if cb.qjl_dim else None
    dbg_rot = torch.full((n, 128), float("nan"), dtype=torch.float32, device=DEV) if debug else None
    dbg_proj = torch.full((n, cb.qjl_dim), float("nan"), dtype=torch.float32, device=DEV) if (debug and cb.qjl_dim) else None
    T.encode_kv(cb, x_dev, codes, norms, signs, res, dst_row, dbg_rot, dbg_proj)
    torch.cuda.synchronize()
    out = {"codes": u32(codes), "norms": norms.cpu().numpy()}
    if cb.qjl_dim:
        out["signs"] = u32(signs)
        out["res_norms"] = res.cpu().numpy()
    if debug:
        out["y"] = dbg_rot.cpu().numpy()
        if cb.qjl_dim:
            out["p"] = dbg_proj.cpu().numpy()
    return out


def check_encode(x_host: np.ndarray, got: dict, bits: int, m: int, rows=None, tol=1e-4, wide: int = 0):
    """Parity of one encode against the oracle; returns the near-boundary flip count.

    rows[i] is the cache row of input row i (default i); wide > 0: split widths.
    """
    bk = oracle_book(bits, m, wide=wide)
    rows = np.arange(x_host.shape[0]) if rows is None else rows
    if wide:
        ref = O.encode_split(x_host.astype(np.float64), bk["Pi"], bk, bk["S"])
    else:
        ref = O.encode(x_host.astype(np.float64), bk["Pi"], bk["centroids"], bk["thresholds"], bk["S"])
    y = got["y"]
    # rotated values: per vector ||dy||_inf <= tol * ||y||_inf
    scale = np.abs(ref["y"]).max(axis=1)
    dy = np.abs(y.astype(np.float64) - ref["y"]).max(axis=1)
    assert np.all(dy <= tol * scale + 1e-30), f"y mismatch: worst {np.max(dy / np.maximum(scale, 1e-30)):.3e}"
    # norms
    nu = got["norms"][rows].astype(np.float64)
    assert np.all(np.abs(nu - ref["nu"]) <= tol * ref["nu"] + 1e-30), "norm mismatch"
    # codes: the oracle quantizes the GPU's fp32 rotated values -> bit-exact
    if wide:
        idx = O.quantize_split(y, bk)
        np.testing.assert_array_equal(got["codes"][rows], O.pack_bits_widths(idx, O.split_widths(128, bits, wide)))
    else:
        idx = O.quantize(y, bk["thresholds"])
        np.testing.assert_array_equal(got["codes"][rows], O.pack_bits(idx, bits))
    flips = int(np.sum(idx != ref["idx"]))
    if m:
        if wide:
            r = y.astype(np.float64) - O.dequant_split(idx, bk)
            gamma = np.sqrt(np.sum(r * r, axis=1))
        else:
            r, gamma = O.residual_from_rotated(y, idx, bk["centroids"])
        assert np.all(np.abs(got["res_norms"][rows] - gamma) <= tol * gamma + 1e-30), "residual norm mismatch"
        p_ref = r @ bk["S"].T
        pscale = np.abs(p_ref).max(axis=1)
        dp = np.abs(got["p"].astype(np.float64) - p_ref).max(axis=1)
        assert np.all(dp <= tol * pscale + 1e-30), f"projection mismatch: worst {np.max(dp / np.maximum(pscale, 1e-30)):.3e}"
        np.testing.assert_array_equal(got["signs"][rows], O.pack_bits(got["p"] > 0, 1))
        flips += int(np.sum((got["p"] > 0) != ref["z"]))
    return flips


def build_cache(kcb, vcb, k_dev, v_dev, B, Hkv, t_cap, T_fill):
    """Encode K, V [B, Hkv, T_fill, d] (device) into caches of capacity t_cap."""
    kc = T.CompressedCache.allocate(kcb, B, Hkv, t_cap)
    vc = T.CompressedCache.allocate(vcb, B, Hkv, t_cap)
    bb, hh, tt = torch.meshgrid(torch.arange(B), torch.arange(Hkv), torch.arange(T_fill), indexing="ij")
    dst = ((bb * Hkv + hh) * t_cap + tt).reshape(-1).to(DEV)
    T.encode_into_cache(kcb, k_dev.reshape(-1, 128), kc, dst_row=dst)
    T.encode_into_cache(vcb, v_dev.reshape(-1, 128), vc, dst_row=dst)
    return kc, vc


def cache_to_host(c: T.CompressedCache) -> dict:
    return {"codes": u32(c.codes), "norms": c.norms.cpu().numpy(),
            "signs": None if c.signs is None else u32(c.signs),
            "res_norms": None if c.res_norms is None else c.res_norms.cpu().numpy()}


def rne_bf16(x: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f32(synth.bf16_bits(x.astype(np.float32)))


def check_decode(kcb, vcb, q_dev, kc, vc, seq_len, kbits, vbits, m, score_tol=1e-4, out_tol=2e-3, wide=0):
    B, Hq, _ = q_dev.shape
    t_cap = kc.t_cap
    sl = torch.tensor(seq_len, dtype=torch.int32, device=DEV)
    scores = torch.full((B, Hq, t_cap), float("nan"), dtype=torch.float32, device=DEV)
    out32 = T.decode_attention(kcb, vcb, q_dev, kc, vc, sl, out_dtype=torch.float32, dbg_scores=scores)
    out16 = T.decode_attention(kcb, vcb, q_dev, kc, vc, sl, out_dtype=torch.bfloat16)
    out32b = T.decode_attention(kcb, vcb, q_dev, kc, vc, sl, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o32 = out32.cpu().numpy()
    # determinism: bitwise identical re-run
    np.testing.assert_array_equal(o32.view(np.uint32), out32b.cpu().numpy().view(np.uint32))
    # bf16 output is the RNE rounding of the fp32 output
    np.testing.assert_array_equal(out16.float().cpu().numpy(), rne_bf16(o32))
    kb, vb = oracle_book(kbits, m, wide=wide), oracle_book(vbits, 0, wide=wide)
    q_host = q_dev.float().cpu().numpy().astype(np.float64)
    seq_c = [min(max(int(s), 0), t_cap) for s in seq_len]
    ref_out, ref_sc = O.decode_attention(q_host, cache_to_host(kc), cache_to_host(vc), seq_c, kb, vb,
                                         return_scores=True)
    sc = scores.cpu().numpy()
    for b in range(B):
        Tb = seq_c[b]
        for h in range(Hq):
            if Tb == 0:
                continue
            ref = ref_sc[b, h, :Tb]
            err = np.abs(sc[b, h, :Tb] - ref).max()
            assert err <= score_tol * np.abs(ref).max(), f"scores b={b} h={h}: {err:.3e} vs max {np.abs(ref).max():.3e}"
            assert np.all(np.isnan(sc[b, h, Tb:])), "scores written past seq_len"
    err = np.abs(o32 - ref_out).max()
    assert err <= out_tol, f"output max-abs error {err:.3e}"
    return err


def oracle_logits(q_host, kc_host, seq_c, kb, g, scale=None):
    """Oracle scaled logits [B, Hq, t_cap] (NaN past seq_len): decode_scores of
    every (b, q head) over its kv head's first seq_len[b] cached keys."""
    B, Hq, d = q_host.shape
    t_cap = kc_host["norms"].shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    m = 0 if kb["S"] is None else kb["S"].shape[0]
    out = np.full((B, Hq, t_cap), np.nan)
    for b in range(B):
        Tb = seq_c[b]
        if Tb == 0:
            continue
        for hk in range(Hq // g):
            idx = O.book_codes(kb, kc_host["codes"][b, hk, :Tb], d)
            z = O.unpack_bits(kc_host["signs"][b, hk, :Tb], m, 1).astype(bool) if m else None
            gam = kc_host["res_norms"][b, hk, :Tb] if m else None
            for j in range(g):
                out[b, hk * g + j, :Tb] = O.decode_scores(q_host[b, hk * g + j], kb["Pi"], O.book_table(kb), kb["S"],
                                                          idx, kc_host["norms"][b, hk, :Tb], gam, z, scale)
    return out


def check_logits(got: np.ndarray, ref: np.ndarray, seq_c, tol=1e-4):
    """Per (b, q head): max |got - ref| <= tol * max |ref| over t < seq_len;
    entries past seq_len keep the caller's NaN sentinel."""
    B, Hq, _ = ref.shape
    worst = 0.0
    for b in range(B):
        Tb = seq_c[b]
        for h in range(Hq):
            assert np.all(np.isnan(got[b, h, Tb:])), f"logits written past seq_len (b={b} h={h})"
            if Tb == 0:
                continue
            r = ref[b, h, :Tb]
            err = np.abs(got[b, h, :Tb].astype(np.float64) - r).max() / np.abs(r).max()
            assert err <= tol, f"logits b={b} h={h}: relative error {err:.3e}"
            worst = max(worst, err)
    return worst
