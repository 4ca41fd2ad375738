"""Seeded synthetic inputs (keys, values, queries) shared by tests and benchmark.

Holds no step of the method: only random draws with the shapes and value
distributions of the workloads (Llama-3-8B/70B-shaped KV heads, outlier
channels, log-normal token norms, Student-t outlier tokens) and bf16 rounding.
Seeds: numpy SeedSequence(config id) spawned, in order, into streams for
K, V, Q, outlier-channel choice and appended tokens.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

D = 128


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if np.any(nan):
        r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def streams(config_id: int):
    """Independent generators: K, V, Q, outlier channels, appended tokens."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(config_id).spawn(5)]


def kv_block(rng, batch: int, heads: int, tokens: int, outlier_ch: Optional[np.ndarray] = None,
             outlier_scale: float = 20.0, lognormal_sigma: Optional[float] = None,
             student_t_rate: Optional[float] = None, student_t_df: float = 3.0) -> np.ndarray:
    """float32 [batch, heads, tokens, D] of N(0,1) entries plus the config's structure.

    outlier_ch[heads, k]: fixed channels per head multiplied by outlier_scale.
    lognormal_sigma: every token vector is scaled by exp(sigma * xi), xi ~ N(0,1).
    student_t_rate: that fraction of tokens (Bernoulli) is redrawn iid Student-t(df).
    """
    x = rng.standard_normal((batch, heads, tokens, D), dtype=np.float32)
    if student_t_rate:
        mask = rng.random((batch, heads, tokens)) < student_t_rate
        cnt = int(mask.sum())
        if cnt:
            x[mask] = rng.standard_t(student_t_df, size=(cnt, D)).astype(np.float32)
    if lognormal_sigma:
        x *= np.exp(lognormal_sigma * rng.standard_normal((batch, heads, tokens, 1))).astype(np.float32)
    if outlier_ch is not None:
        for h in range(heads):
            x[:, h, :, outlier_ch[h]] *= outlier_scale
    return x


def outlier_channels(rng, heads: int, per_head: int) -> np.ndarray:
    return np.stack([rng.choice(D, size=per_head, replace=False) for _ in range(heads)])


@dataclass
class Workload:
    name: str
    k_bits: int                # total key bits b (b' = b - 1 MSE bits + 1 QJL bit)
    v_bits: int                # value MSE bits
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    k: np.ndarray              # [B, Hkv, T, D] (uint16 bf16 bits, or float32)
    v: Optional[np.ndarray]
    q: np.ndarray              # [B, Hq, D]
    dtype: str                 # "bf16" or "f32"


def tiny() -> Workload:
    """4096 N(0,1) fp32 keys, one N(0,1) query; keys b = 3 (2-bit codes + 1-bit QJL)."""
    rng = np.random.default_rng(0)
    k = rng.standard_normal((1, 1, 4096, D), dtype=np.float32)
    q = rng.standard_normal((1, 1, D), dtype=np.float32)
    return Workload("tiny-4096x128-f32-b3", 3, 0, 1, 1, 1, 4096, k, None, q, "f32")


def llama8b(seq_len: int = 32768, config_id: int = 1) -> Workload:
    """Llama-3-8B-shaped layer: B=1, 32 q heads, 8 KV heads, bf16 N(0,1) K/V,
    4 fixed outlier channels per head x20; keys b=3, values 3-bit."""
    sk, sv, sq, so, _ = streams(config_id)
    ko = outlier_channels(so, 8, 4)
    vo = outlier_channels(so, 8, 4)
    k = bf16_bits(kv_block(sk, 1, 8, seq_len, ko))
    v = bf16_bits(kv_block(sv, 1, 8, seq_len, vo))
    q = bf16_bits(sq.standard_normal((1, 32, D), dtype=np.float32))
    return Workload(f"llama3-8b-layer-b1-s{seq_len}", 3, 3, 1, 32, 8, seq_len, k, v, q, "bf16")


def batched(bits: int, seq_len: int = 8192, batch: int = 16, config_id: int = 2) -> Workload:
    """Batched decode: B=16, 32/8 heads, bf16 N(0,1) with per-token norm
    log-normal(0, 0.5); keys and values at the same bit count."""
    sk, sv, sq, _, _ = streams(config_id)
    k = bf16_bits(kv_block(sk, batch, 8, seq_len, lognormal_sigma=0.5))
    v = bf16_bits(kv_block(sv, batch, 8, seq_len, lognormal_sigma=0.5))
    q = bf16_bits(sq.standard_normal((batch, 32, D), dtype=np.float32))
    return Workload(f"batched-b{batch}-s{seq_len}-bits{bits}", bits, bits, batch, 32, 8, seq_len, k, v, q, "bf16")


def appended_tokens(step: int, batch: int = 16, config_id: int = 2):
    """K, V, q of one appended decode step of the batched workload."""
    rng = np.random.default_rng(np.random.SeedSequence([config_id, 1000 + step]))
    k = bf16_bits(kv_block(rng, batch, 8, 1, lognormal_sigma=0.5))
    v = bf16_bits(kv_block(rng, batch, 8, 1, lognormal_sigma=0.5))
    q = bf16_bits(rng.standard_normal((batch, 32, D), dtype=np.float32))
    return k, v, q


def llama70b(seq_len: int = 131072, config_id: int = 3) -> Workload:
    """Llama-3-70B-shaped long context: B=1, 64 q heads / 8 KV heads, bf16,
    8 outlier channels x20; keys b=3, values 2-bit."""
    sk, sv, sq, so, _ = streams(config_id)
    ko = outlier_channels(so, 8, 8)
    vo = outlier_channels(so, 8, 8)
    k = bf16_bits(kv_block(sk, 1, 8, seq_len, ko))
    v = bf16_bits(kv_block(sv, 1, 8, seq_len, vo))
    q = bf16_bits(sq.standard_normal((1, 64, D), dtype=np.float32))
    return Workload(f"llama3-70b-layer-b1-s{seq_len}", 3, 2, 1, 64, 8, seq_len, k, v, q, "bf16")


def bulk(n: int, config_id: int = 4):
    """Bulk-encode vectors: N(0,1) with 1% Student-t(3) outlier tokens, bf16 [n, D] K and V."""
    sk, sv, sq, _, _ = streams(config_id)
    k = bf16_bits(kv_block(sk, 1, 1, n, student_t_rate=0.01)[0, 0])
    v = bf16_bits(kv_block(sv, 1, 1, n, student_t_rate=0.01)[0, 0])
    q = bf16_bits(sq.standard_normal((1, 64, D), dtype=np.float32))
    return k, v, q


def bulk_device(n: int, device, config_id: int = 4, chunk: int = 1 << 22):
    """Bulk-encode inputs generated on the GPU (seeded torch generator):
    K and V [n, D] bf16, N(0,1) with 1% of tokens redrawn iid Student-t(3)
    (a normal over the square root of a chi-square(3)/3 draw), and 64 N(0,1)
    queries.  Used where a host generator would take minutes."""
    import torch
    g = torch.Generator(device=device)
    out = []
    for which in range(2):
        g.manual_seed(int(np.random.SeedSequence([config_id, which]).generate_state(1)[0]))
        x = torch.empty(n, D, dtype=torch.bfloat16, device=device)
        for s in range(0, n, chunk):
            e = min(n, s + chunk)
            v = torch.randn(e - s, D, generator=g, device=device)
            heavy = torch.rand(e - s, generator=g, device=device) < 0.01
            chi2 = torch.randn(e - s, D, 3, generator=g, device=device).pow(2).sum(-1)
            t3 = torch.randn(e - s, D, generator=g, device=device) / torch.sqrt(chi2 / 3.0)
            v = torch.where(heavy[:, None], t3, v)
            x[s:e] = v.to(torch.bfloat16)
        out.append(x)
    g.manual_seed(int(np.random.SeedSequence([config_id, 2]).generate_state(1)[0]))
    q = torch.randn(1, 64, D, generator=g, device=device).to(torch.bfloat16)
    return out[0], out[1], q
