#!/usr/bin/env python3
"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

One step = the whole path over one batch of synthetic input: encode every key
and value vector of the workload into the compressed cache (two launches),
then one decode-attention step over a compressed cache.

Default run (no flags): the headline line is the largest single-GPU workload,
the prefill-scale bulk encode (16,777,216 bf16 K and V vectors of dim 128;
keys b=4 = 3-bit codes + 1-bit QJL with m=128, values 4-bit), then 64 q heads
(8 per KV head) decoding over a 262,144-token x 8-head view of the cache.  The
other workloads ride along as nested sub-records under "configs": the tiny
quality case, the Llama-3-8B-shaped layer, the batched decode at b=2 and b=4
with its 8-step append loop, and the Llama-3-70B-shaped long context.
`--config NAME` runs one workload as the headline alone.

Inputs are resident in HBM before timing.  To keep the 256 MB Infinity Cache
from serving re-reads, the layer workloads read one of several input replicas
per step and decode a cache replica written many steps earlier (>= 1 GiB of
distinct caches in rotation; --hot disables it); the bulk workload's 8.6 GB of
inputs and 294 MB decode view exceed it by themselves.

Prints ONE JSON line.  `value` is the decode-attention throughput in GB/s of
compressed K+V bytes read; encode throughput (Mvectors/s) and both kernels'
roofline figures are reported alongside.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0

# HBM bytes per key-encode launch, from two
# rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this benchmark with
# --calib-copy 512, each scaled by the ratio of a 512 MiB device copy's known
# bytes to what the same counter read for it.  Valid only for the encode
# sources they were taken on (sha256 over tq_encode.hip and tq_encode_body.inc,
# below); otherwise reported as null.
# Per workload: the key-encode launch's HBM bytes and its matrix-core / vector
# busy fractions (SQ_VALU_MFMA_BUSY_CYCLES over 1,024 SIMDs x kernel cycles;
# SQ_ACTIVE_INST_VALU less MFMA instructions at 4 cycles each).
ENCODE_COUNTERS = {
    "llama3-8b-layer-b1-s32768": {"source_sha256": "dbc0a21f4aafaee72542cda413bf4dcc80614cb20008847cb481c01614e335c1",
                                  "fetch_bytes": 68445280, "write_bytes": 14694704,
                                  "mfma_busy": 0.368, "valu_busy": 0.302},
    "bulk-encode-16777216-kv-then-decode-g8-s262144": {
        "source_sha256": "dbc0a21f4aafaee72542cda413bf4dcc80614cb20008847cb481c01614e335c1",
        "fetch_bytes": 4296307135, "write_bytes": 1207991552, "mfma_busy": 0.557, "valu_busy": 0.453},
}
BF16_MFMA_PEAK_TFLOPS = 2500.0
BULK_NAME = "bulk-encode-16777216-kv-then-decode-g8-s262144"
METRIC = "decode-attn HBM GB/s (% of peak) on compressed KV; encode Mvectors/s"
# "dtype" names the arithmetic: fp32 accumulation throughout (the matrix-core
# products take bf16 hi/lo operand splits, three products per fp32 product);
# the data crossing the boundary are bf16 (fp32 for the tiny workload).
DTYPES = {"input": "bf16", "query": "bf16", "output": "bf16", "accumulate": "f32",
          "mfma_operands": "bf16 hi/lo split of fp32 values"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="all",
                    choices=["all", "llama8b", "llama70b", "batched2", "batched4", "bulk", "tiny"],
                    help="all (default): the bulk workload as the headline plus every other workload as a "
                         "sub-record; bulk: encode 16,777,216 K and V vectors, then 64 queries over a "
                         "262144 x 8 view")
    ap.add_argument("--hot", action="store_true", help="no replica rotation (cache-resident numbers)")
    ap.add_argument("--append-steps", type=int, default=0, metavar="N",
                    help="also time N decode-loop steps (append one token per sequence and head, then attend): "
                         "separate calls, tq_append_decode, and one captured step replayed as a graph")
    ap.add_argument("--key-mode", default="qjl", choices=["qjl", "mse"],
                    help="keys as (b-1)-bit codes + 1-bit QJL (default) or b-bit MSE-only codes")
    ap.add_argument("--chunk", type=int, default=16, metavar="N",
                    help="also time causal attention of N new queries per head over the full cache (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle step until this much CPU time has run")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="before warm-up, run 3 plain device copies of MIB MiB (untimed): the reference "
                         "kernel of known size that scales the HBM byte counters")
    return ap.parse_args()


def workload(name):
    from online_vector_quantization_amd import synth
    if name == "llama8b":
        return synth.llama8b()
    if name == "llama70b":
        return synth.llama70b()
    if name == "batched2":
        return synth.batched(2)
    return synth.batched(4)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import online_vector_quantization_amd as T
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    T.load_library()
    dev = torch.device("cuda", 0)
    if args.config == "all":
        line = bench_bulk(args, T, dev, cpu=not args.no_cpu_baseline)
        subs = {}
        # split widths on the 8B layer: 3.5 bits (keys 2.5-bit codes + QJL,
        # values 3.5-bit codes) and 2.5 bits (1.5 + QJL, 2.5)
        splits = {"llama8b_split_3.5bit": (2, 3), "llama8b_split_2.5bit": (1, 2)}
        for name in ("tiny", "llama8b", "batched2", "batched4", "llama70b", *splits):
            t0 = time.time()
            if name == "tiny":
                rec = bench_tiny(args, T, dev)
            elif name in splits:
                rec = bench_layer(args, T, dev, "llama8b", logits=True, cpu=False, split=splits[name])
            else:
                rec = bench_layer(args, T, dev, name, append_steps=8 if name.startswith("batched") else 0,
                                  chunk=args.chunk if name == "llama8b" else 0, logits=True, cpu=False)
            subs[name] = sub_record(rec)
            print(f"[bench] sub-record {name} done in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
        line["configs"] = subs
        print(json.dumps(line), flush=True)
        return
    if args.config == "bulk":
        print(json.dumps(bench_bulk(args, T, dev, cpu=not args.no_cpu_baseline)), flush=True)
        return
    if args.config == "tiny":
        print(json.dumps(bench_tiny(args, T, dev)), flush=True)
        return
    line = bench_layer(args, T, dev, args.config, append_steps=args.append_steps, chunk=args.chunk, logits=True,
                       cpu=not args.no_cpu_baseline)
    print(json.dumps(line), flush=True)


# keys of a full line that a nested sub-record leaves out (the headline carries them)
_SUB_DROP = ("metric", "unit", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data", "steps", "warmup")


def sub_record(line):
    """A workload's line as a nested sub-record of the headline line."""
    return {k: v for k, v in line.items() if k not in _SUB_DROP}


def bench_layer(args, T, dev, name, append_steps=0, chunk=0, logits=True, cpu=True, split=None):
    """One layer-shaped workload (8B, batched, 70B): encode all of its K and V,
    then one decode over a full cache replica, per step.  split = (key code
    bits b', value bits b'): split widths instead of the workload's widths,
    rotated coordinates 0..63 one bit wider (b' + 0.5 bits per coordinate,
    keys plus their 1-bit QJL sketch)."""
    import torch
    t0 = time.time()
    wl = workload(name)
    B, Hq, Hkv, S = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.seq_len
    kbits_mse = wl.k_bits - 1
    print(f"[bench] workload {wl.name}: generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    if args.key_mode == "mse":
        kbits_mse = wl.k_bits
    qjl_m = 128 if args.key_mode == "qjl" else 0
    tag = wl.name
    if split is None:
        kcb = T.Codebook(128, kbits_mse, qjl_m, 0, 1, device=0)
        vcb = T.Codebook(128, wl.v_bits, 0, 0, 1, device=0)
    else:
        kbits_mse, vbits = split
        kcb = T.Codebook(128, kbits_mse, qjl_m, 0, 1, device=0, wide_coords=64)
        vcb = T.Codebook(128, vbits, 0, 0, 1, device=0, wide_coords=64)
        tag = f"{wl.name}-split-k{kbits_mse + 0.5 + (1 if qjl_m else 0)}-v{vbits + 0.5}"
    n_vec = B * Hkv * S

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev).reshape(-1, 128)

    k0, v0 = up(wl.k), up(wl.v)
    q = torch.from_numpy(np.ascontiguousarray(wl.q).view(np.int16)).view(torch.bfloat16).to(dev)
    in_bytes = 2 * n_vec * 128 * 2
    cache_bytes_one = n_vec * T.compressed_bytes_per_token(kcb, vcb)
    n_in = 1 if args.hot else max(2, math.ceil((512 << 20) / in_bytes))
    n_cache = 1 if args.hot else max(2, math.ceil((1 << 30) / cache_bytes_one))
    ins = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(n_in - 1)]
    caches = [(T.CompressedCache.allocate(kcb, B, Hkv, S), T.CompressedCache.allocate(vcb, B, Hkv, S))
              for _ in range(n_cache)]
    seq = torch.full((B,), S, dtype=torch.int32, device=dev)
    ws = T.alloc_workspace(B, Hq, Hkv, S, dev)
    out = torch.empty(B, Hq, 128, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def encode(i_in, i_c):
        kx, vx = ins[i_in]
        kc, vc = caches[i_c]
        T.encode_into_cache(kcb, kx, kc, stream=stream)
        T.encode_into_cache(vcb, vx, vc, stream=stream)

    def decode(i_c):
        kc, vc = caches[i_c]
        T.decode_attention(kcb, vcb, q, kc, vc, seq, out=out, workspace=ws, stream=stream)

    calib_copy(args, dev)

    # fill every cache replica once (untimed), then warm up
    for i in range(n_cache):
        encode(i % n_in, i)
    for s in range(args.warmup):
        encode(s % n_in, s % n_cache)
        decode((s + n_cache // 2) % n_cache)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [(ev(), ev(), ev(), ev()) for _ in range(args.steps)]
    start, end = ev(), ev()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        e0, e1, e2, e3 = marks[s]
        kx, vx = ins[s % n_in]
        kc, vc = caches[s % n_cache]
        e0.record(stream)
        T.encode_into_cache(kcb, kx, kc, stream=stream)
        e1.record(stream)
        T.encode_into_cache(vcb, vx, vc, stream=stream)
        e2.record(stream)
        decode((s + n_cache // 2) % n_cache)
        e3.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    enc_k = np.array([m[0].elapsed_time(m[1]) for m in marks])
    enc_v = np.array([m[1].elapsed_time(m[2]) for m in marks])
    dec = np.array([m[2].elapsed_time(m[3]) for m in marks])

    ms_step = total_ms / args.steps
    dec_ms = float(dec.mean())
    dec_bytes = cache_bytes_one
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9
    enc_ms = float((enc_k + enc_v).mean())
    enc_mvps = 2 * n_vec / (enc_ms * 1e-3) / 1e6
    k_rec = 4 * kcb.code_words + 4 * kcb.sign_words + 4 + (4 if qjl_m else 0)
    v_rec = 4 * vcb.code_words + 4
    enc_k_bytes = n_vec * (256 + k_rec)
    enc_v_bytes = n_vec * (256 + v_rec)
    enc_k_gbps = enc_k_bytes / (enc_k.mean() * 1e-3) / 1e9
    enc_v_gbps = enc_v_bytes / (enc_v.mean() * 1e-3) / 1e9

    line = {
        "metric": METRIC,
        "value": round(dec_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtypes": DTYPES,
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": B, "seq_len": S, "q_heads": Hq, "kv_heads": Hkv, "head_dim": 128,
            "key_bits": wl.k_bits if split is None else kbits_mse + 0.5 + (1 if qjl_m else 0),
            "value_bits": wl.v_bits if split is None else split[1] + 0.5, "qjl_dim": qjl_m, "input_dtype": "bf16",
            "split_widths": None if split is None else
            {"wide_coords": 64, "key_code_bits": [kbits_mse + 1, kbits_mse], "value_code_bits": [split[1] + 1, split[1]]},
            "key_mode": "(b-1)-bit codes + 1-bit QJL" if qjl_m else "b-bit MSE-only codes",
            "step": "encode all K and V of the layer, then one decode step over a full cache",
            "cold_replicas": {"inputs": n_in, "caches": n_cache, "hot": bool(args.hot)},
        },
        "decode_frac_of_peak": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "decode_us": round(dec_ms * 1e3, 2),
        "encode_mvectors_per_s": round(enc_mvps, 1),
        "encode_us": {"keys": round(float(enc_k.mean()) * 1e3, 2), "values": round(float(enc_v.mean()) * 1e3, 2)},
        "roofline": {
            "kernel": "encode (keys: rotation + QJL)" if qjl_m else "encode (keys: rotation, MSE-only)", "bound": "hbm",
            "achieved": round(enc_k_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(enc_k_gbps / HBM_PEAK_GBPS, 4), "traffic": encode_traffic(tag) if qjl_m else None,
            "algorithmic_bytes_per_launch": enc_k_bytes, "avg_launch_us": round(float(enc_k.mean()) * 1e3, 2),
            "mfma": key_encode_mfma(n_vec, qjl_m, True, float(enc_k.mean()), tag),
        },
        "roofline_values_encode": {
            "bound": "hbm", "achieved": round(enc_v_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(enc_v_gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes_per_launch": enc_v_bytes,
            "avg_launch_us": round(float(enc_v.mean()) * 1e3, 2),
        },
        "roofline_decode": {
            "bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes_per_launch": dec_bytes,
            "avg_us_partial_and_combine": round(dec_ms * 1e3, 2),
            "mfma": decode_mfma_view(B * Hkv * S, Hq // Hkv, qjl_m, dec_ms),
        },
        "wall_s_timed": round(wall, 4),
        "launch_us_percentiles": {
            name: {"p10": round(float(np.percentile(arr, 10)) * 1e3, 2),
                   "median": round(float(np.median(arr)) * 1e3, 2),
                   "p90": round(float(np.percentile(arr, 90)) * 1e3, 2)}
            for name, arr in (("encode_keys", enc_k), ("encode_values", enc_v), ("decode", dec))},
        "copy_gbps_context": copy_bandwidth(dev),
    }
    if logits:
        line["attention_logits"] = logits_only(T, kcb, q, caches, seq, ws, n_vec * k_rec, B * Hq * S * 4, args, dev)
    if chunk > 0:
        line["chunk_attention"] = chunk_only(T, kcb, vcb, caches, S, Hq, chunk, args, dev)
    del caches, ins
    if append_steps > 0:
        line["append_step_us"] = run_append_steps(wl, kcb, vcb, up, append_steps, dev)
    if cpu:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, qjl=bool(qjl_m))
    return line


def calib_copy(args, dev):
    """--calib-copy: three plain device copies of known size (untimed), the
    reference launches that scale the HBM byte counters."""
    import torch
    if not args.calib_copy:
        return
    n_el = args.calib_copy << 18           # MiB of float32
    src = torch.ones(n_el, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def bench_bulk(args, T, dev, cpu=True):
    """Prefill-scale bulk encode: every step encodes 16,777,216 K vectors (b' = 3
    + QJL) and 16,777,216 V vectors (4-bit), then decodes 64 q heads (8 per kv
    head) over the first 2,097,152 rows of each cache viewed as [1, 8, 262144].
    The inputs (8.6 GB) and the decode view (294 MB) exceed the 256 MB
    Infinity Cache, so every launch reads HBM."""
    import torch
    from online_vector_quantization_amd import synth
    n, Tlen, Hkv, Hq = 16_777_216, 262_144, 8, 64
    t0 = time.time()
    kx, vx, q = synth.bulk_device(n, dev)
    torch.cuda.synchronize()
    print(f"[bench] bulk inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    kcb = T.Codebook(128, 3, 128, 0, 1, device=0)
    vcb = T.Codebook(128, 4, 0, 0, 1, device=0)
    kc = T.CompressedCache.allocate(kcb, 1, 1, n)
    vc = T.CompressedCache.allocate(vcb, 1, 1, n)
    rows = Hkv * Tlen
    kview = T.CompressedCache(kc.codes.reshape(-1, kcb.code_words)[:rows].reshape(1, Hkv, Tlen, -1),
                              kc.norms.reshape(-1)[:rows].reshape(1, Hkv, Tlen),
                              kc.signs.reshape(-1, kcb.sign_words)[:rows].reshape(1, Hkv, Tlen, -1),
                              kc.res_norms.reshape(-1)[:rows].reshape(1, Hkv, Tlen))
    vview = T.CompressedCache(vc.codes.reshape(-1, vcb.code_words)[:rows].reshape(1, Hkv, Tlen, -1),
                              vc.norms.reshape(-1)[:rows].reshape(1, Hkv, Tlen))
    seq = torch.full((1,), Tlen, dtype=torch.int32, device=dev)
    ws = T.alloc_workspace(1, Hq, Hkv, Tlen, dev)
    out = torch.empty(1, Hq, 128, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(marks=None):
        if marks:
            marks[0].record(stream)
        T.encode_into_cache(kcb, kx, kc, stream=stream)
        if marks:
            marks[1].record(stream)
        T.encode_into_cache(vcb, vx, vc, stream=stream)
        if marks:
            marks[2].record(stream)
        T.decode_attention(kcb, vcb, q, kview, vview, seq, out=out, workspace=ws, stream=stream)
        if marks:
            marks[3].record(stream)

    calib_copy(args, dev)
    for _ in range(max(1, args.warmup)):
        step()
    steps = max(1, args.steps)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [(ev(), ev(), ev(), ev()) for _ in range(steps)]
    start, end = ev(), ev()
    torch.cuda.synchronize()
    start.record(stream)
    for s_ in range(steps):
        step(marks[s_])
    end.record(stream)
    torch.cuda.synchronize()
    enc_k = np.array([m[0].elapsed_time(m[1]) for m in marks])
    enc_v = np.array([m[1].elapsed_time(m[2]) for m in marks])
    dec = np.array([m[2].elapsed_time(m[3]) for m in marks])
    k_rec = 4 * kcb.code_words + 4 * kcb.sign_words + 8
    v_rec = 4 * vcb.code_words + 4
    dec_bytes = rows * (k_rec + v_rec)
    dec_gbps = dec_bytes / (dec.mean() * 1e-3) / 1e9
    enc_k_bytes, enc_v_bytes = n * (256 + k_rec), n * (256 + v_rec)
    enc_k_gbps = enc_k_bytes / (enc_k.mean() * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(dec_gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(start.elapsed_time(end) / steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "dtypes": DTYPES, "data": "synthetic",
        "config": {"workload": BULK_NAME, "vectors": n, "key_bits": 4,
                   "value_bits": 4, "qjl_dim": 128, "decode_view": [1, Hkv, Tlen], "q_heads": Hq,
                   "input_dtype": "bf16", "key_mode": "(b-1)-bit codes + 1-bit QJL",
                   "step": "encode all K and V vectors, then one decode step over the view"},
        "decode_frac_of_peak": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "decode_us": round(float(dec.mean()) * 1e3, 2),
        "encode_mvectors_per_s": round(2 * n / ((enc_k.mean() + enc_v.mean()) * 1e-3) / 1e6, 1),
        "encode_us": {"keys": round(float(enc_k.mean()) * 1e3, 1), "values": round(float(enc_v.mean()) * 1e3, 1)},
        "roofline": {"kernel": "encode (keys: rotation + QJL)", "bound": "hbm", "achieved": round(enc_k_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(enc_k_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": encode_traffic(BULK_NAME), "algorithmic_bytes_per_launch": enc_k_bytes,
                     "avg_launch_us": round(float(enc_k.mean()) * 1e3, 1),
                     "mfma": key_encode_mfma(n, 128, True, float(enc_k.mean()), BULK_NAME)},
        "roofline_values_encode": {"bound": "hbm", "achieved": round(enc_v_bytes / (enc_v.mean() * 1e-3) / 1e9, 1),
                                   "peak": HBM_PEAK_GBPS, "unit": "GB/s", "algorithmic_bytes_per_launch": enc_v_bytes},
        "roofline_decode": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes_per_launch": dec_bytes,
                            "mfma": decode_mfma_view(Hkv * Tlen, Hq // Hkv, 128, float(dec.mean()))},
    }
    if cpu:
        line["cpu_baseline"] = cpu_baseline_bulk(kx, vx, q, args.cpu_seconds)
    return line


def bench_tiny(args, T, dev):
    """The tiny workload: 4096 fp32 keys (2-bit codes + 128 QJL signs), one query.
    It is latency-bound, so the line reports launch times next to the quality of
    the score estimate: exact q.k against the estimate (bias, RMSE, correlation)
    and softmax at scale 1/sqrt(d) of both (max-abs difference, total
    variation).  The values reuse the keys at 2 bits (the workload has none)."""
    import torch
    from online_vector_quantization_amd import synth
    wl = synth.tiny()
    n = 4096
    kcb = T.Codebook(128, 2, 128, 0, 1, device=0)
    vcb = T.Codebook(128, 2, 0, 0, 1, device=0)
    k = torch.from_numpy(wl.k.reshape(n, 128).copy()).to(dev)
    q = torch.from_numpy(wl.q.copy()).to(dev)
    kc, vc = T.CompressedCache.allocate(kcb, 1, 1, n), T.CompressedCache.allocate(vcb, 1, 1, n)
    seq = torch.tensor([n], dtype=torch.int32, device=dev)
    ws = T.alloc_workspace(1, 1, 1, n, dev)
    out = torch.empty(1, 1, 128, dtype=torch.float32, device=dev)
    scores = torch.zeros(1, 1, n, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    steps = max(args.steps, 1)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.warmup + steps)]
    for i, e in enumerate(ev):
        e[0].record(stream)
        T.encode_into_cache(kcb, k, kc, stream=stream)
        T.encode_into_cache(vcb, k, vc, stream=stream)
        e[1].record(stream)
        T.decode_attention(kcb, vcb, q, kc, vc, seq, out=out, workspace=ws, stream=stream,
                           dbg_scores=scores if i == 0 else None)
        e[2].record(stream)
    torch.cuda.synchronize()
    enc = np.array([e[0].elapsed_time(e[1]) for e in ev[args.warmup:]])
    dec = np.array([e[1].elapsed_time(e[2]) for e in ev[args.warmup:]])
    exact = wl.k.reshape(n, 128).astype(np.float64) @ wl.q.reshape(128).astype(np.float64)
    est = scores.cpu().numpy()[0, 0].astype(np.float64) * math.sqrt(128.0)
    err = est - exact

    def softmax(x):
        e_ = np.exp(x - x.max())
        return e_ / e_.sum()
    p, ph = softmax(exact / math.sqrt(128.0)), softmax(est / math.sqrt(128.0))
    dec_bytes = n * T.compressed_bytes_per_token(kcb, vcb)
    dec_gbps = dec_bytes / (float(dec.mean()) * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": round(dec_gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(float((enc + dec).mean()), 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "dtypes": dict(DTYPES, input="f32", query="f32", output="f32"), "data": "synthetic",
        "config": {"workload": wl.name, "keys": n, "head_dim": 128, "key_bits": 3, "qjl_dim": 128,
                   "input_dtype": "f32", "step": "encode the keys (and the same vectors as 2-bit values), then decode"},
        "encode_us": round(float(enc.mean()) * 1e3, 2), "decode_us": round(float(dec.mean()) * 1e3, 2),
        "quality": {"bias": round(float(err.mean()), 5), "bias_se": round(float(err.std() / math.sqrt(n)), 5),
                    "rmse": round(float(math.sqrt(np.mean(err * err))), 5),
                    "corr": round(float(np.corrcoef(est, exact)[0, 1]), 5),
                    "softmax_max_abs": round(float(np.abs(p - ph).max()), 6),
                    "softmax_tv": round(float(0.5 * np.abs(p - ph).sum()), 5)},
    }


# Dense fp16 / bf16 MFMA peak of MI355X (TFLOP/s).
MFMA_PEAK_TFLOPS = 2500.0


def decode_mfma_view(kv_token_rows, g, qjl_m, ms):
    """The matrix-core decode against the dense fp16/bf16 MFMA roof.  Per 16
    tokens of one kv head it issues 8 key products, 4 sign products (QJL keys)
    and 8 value products of v_mfma_f32_16x16x32 (16384 flops each), with the
    g <= 8 heads' hi and lo parts in 16 columns; the method itself needs
    2 (d + m + d) flops per (token, q head)."""
    issued = kv_token_rows * (16 + (4 if qjl_m else 0)) * 16384 / 16
    algorithmic = kv_token_rows * g * 2 * (128 + qjl_m + 128)
    t = ms * 1e-3
    return {"bound": "mfma", "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "achieved_issued": round(issued / t / 1e12, 1), "frac_issued": round(issued / t / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "achieved_algorithmic": round(algorithmic / t / 1e12, 1),
            "frac_algorithmic": round(algorithmic / t / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "flops_per_launch_issued": float(issued), "flops_per_launch_algorithmic": float(algorithmic)}


def cpu_baseline_bulk(kx, vx, q, min_seconds):
    """The oracle on a bounded sample of the bulk step: encode of the first
    2^17 K and V vectors, decode of the 64 q heads over the 8-head cache of
    16384 tokens built from them; reported as encode vectors/s and decode GB/s
    of compressed bytes read."""
    import torch
    import oracle as O
    from online_vector_quantization_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    ns, Hkv = 1 << 17, 8
    Tlen = ns // Hkv

    def host_f32(t):
        return synth.bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))

    k, v = host_f32(kx[:ns]), host_f32(vx[:ns])
    qh = host_f32(q).astype(np.float64)
    c_k, t_k = O.build_codebook(128, 3)
    c_v, t_v = O.build_codebook(128, 4)
    Pi, Sm = O.haar_rotation(128, 0), O.qjl_matrix(128, 128, 1)
    shape = (1, Hkv, ns // Hkv)
    t_enc = t_dec = 0.0
    reps = 0
    while reps == 0 or t_enc + t_dec < min_seconds:
        t0 = time.perf_counter()
        ek = O.encode(k, Pi, c_k, t_k, Sm)
        ev = O.encode(v, Pi, c_v, t_v)
        kcache = {"codes": O.pack_bits(ek["idx"], 3).reshape(*shape, -1), "signs": O.pack_bits(ek["z"], 1).reshape(*shape, -1),
                  "norms": ek["nu"].reshape(shape), "res_norms": ek["gamma"].reshape(shape)}
        vcache = {"codes": O.pack_bits(ev["idx"], 4).reshape(*shape, -1), "norms": ev["nu"].reshape(shape)}
        t1 = time.perf_counter()
        O.decode_attention(qh, kcache, vcache, [Tlen], {"bits": 3, "centroids": c_k, "Pi": Pi, "S": Sm},
                           {"bits": 4, "centroids": c_v, "Pi": Pi})
        t2 = time.perf_counter()
        t_enc += t1 - t0
        t_dec += t2 - t1
        reps += 1
    rec = (4 * 12 + 16 + 8) + (4 * 16 + 4)
    return {"value": round(reps * Hkv * Tlen * rec / t_dec / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle", "encode_mvectors_per_s": round(reps * 2 * ns / t_enc / 1e6, 4),
            "sample": f"{reps}x: oracle encode of the first {ns} K and {ns} V vectors ({t_enc / reps:.2f}s each), "
                      f"then oracle decode of 64 q heads over {Tlen} tokens x {Hkv} kv heads built from them "
                      f"({t_dec / reps:.2f}s each)"}


def copy_bandwidth(dev, mib=1024, reps=5):
    """A plain 1 GiB device-to-device copy (torch), timed with events: read +
    write bytes per second.  Context for the HBM fractions, not a peak."""
    import torch
    n = mib << 18
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    gbps = 2 * n * 4 * reps / (start.elapsed_time(end) * 1e-3) / 1e9
    del src, dst
    return round(gbps, 1)


def logits_only(T, kcb, q, caches, seq, ws, key_bytes, logit_bytes, args, dev):
    """Scores-only launches (the key phase of the decode, every logit written)
    over the same cold cache replicas, timed after the step loop: mean time per
    launch and algorithmic bytes (key records read + fp32 logits written)."""
    import torch
    stream = torch.cuda.current_stream(dev)
    B, Hq = q.shape[0], q.shape[1]
    logits = torch.empty(B, Hq, caches[0][0].t_cap, dtype=torch.float32, device=dev)
    for s in range(args.warmup):
        T.attention_logits(kcb, q, caches[s % len(caches)][0], seq, logits=logits, workspace=ws, stream=stream)
    n = max(1, args.steps)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # a launch takes less GPU time than its host-side call: a spin kernel
    # first lets the host queue all n launches, which then run back to back
    torch.cuda._sleep(50_000_000)
    start.record(stream)
    for s in range(n):
        T.attention_logits(kcb, q, caches[s % len(caches)][0], seq, logits=logits, workspace=ws, stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / n
    gbps = (key_bytes + logit_bytes) / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "achieved": round(gbps, 1), "unit": "GB/s", "peak": HBM_PEAK_GBPS,
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "bytes_per_launch": key_bytes + logit_bytes,
            "key_record_bytes": key_bytes, "logit_bytes": logit_bytes}


def chunk_only(T, kcb, vcb, caches, S, Hq, n_new, args, dev):
    """Causal attention of n_new new queries per (b, q head), the last
    positions of a full cache, over the same cold cache replicas: mean time per
    launch pair and the cache bytes per launch (each query block re-reads them)."""
    import torch
    stream = torch.cuda.current_stream(dev)
    kc0, vc0 = caches[0]
    B = kc0.codes.shape[0]
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    q = torch.randn(B, Hq, n_new, 128, generator=g, device=dev).to(torch.bfloat16)
    seq = torch.full((B,), S, dtype=torch.int32, device=dev)
    out = torch.empty(B, Hq, n_new, 128, dtype=torch.bfloat16, device=dev)
    ws = T.alloc_chunk_workspace(B, Hq, kc0.codes.shape[1], n_new, kc0.t_cap, dev)
    run = lambda s: T.chunk_attention(kcb, vcb, q, caches[s % len(caches)][0], caches[s % len(caches)][1], seq,
                                      out=out, workspace=ws, stream=stream)
    for s in range(args.warmup):
        run(s)
    n = max(1, args.steps)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(n):
        run(s)
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / n
    Hkv = kc0.codes.shape[1]
    cache_bytes = B * Hkv * S * T.compressed_bytes_per_token(kcb, vcb)
    res = {"n_new": n_new, "us": round(us, 2), "queries_per_s": round(B * Hq * n_new / (us * 1e-6), 1),
           "cache_bytes": cache_bytes}
    g_ = Hq // Hkv
    if T.api.chunk_uses_mfma(g_, n_new):
        # per (query row, token): key dot (d), QJL dot (m) and value sum (d) multiply-adds; the kernel
        # runs each fp32 product as 3 bf16 products (2 for the exact +-1 signs) over 64-row blocks
        rows = g_ * n_new
        blocks = -(-rows // 64)
        m = kcb.qjl_dim
        alg = 2.0 * B * Hkv * rows * S * (128 + m + 128)
        issued = 2.0 * B * Hkv * blocks * 64 * S * (3 * 128 + 2 * m + 3 * 128)
        res.update({"path": "mfma", "tflops_algorithmic": round(alg / (us * 1e-6) / 1e12, 1),
                    "tflops_issued_bf16": round(issued / (us * 1e-6) / 1e12, 1),
                    "frac_of_bf16_peak_issued": round(issued / (us * 1e-6) / 2.5e15, 4)})
    else:
        res["path"] = "decode kernel per query"
    return res


def run_append_steps(wl, kcb, vcb, up, steps, dev):
    """Per-step time of a decode loop over the workload's caches (prefilled with
    seq_len tokens, capacity seq_len + steps): each step appends one key and
    value per (sequence, kv head) and attends the step's queries over the grown
    cache.  Three ways: separate calls (host-built destination rows, two encodes,
    a decode), tq_append_decode, and one captured append step replayed as a
    graph.  The caches stay resident (no replica rotation)."""
    import torch
    import online_vector_quantization_amd as T
    from online_vector_quantization_amd import synth
    B, Hq, Hkv, S = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.seq_len
    t_cap = S + steps
    kc = T.CompressedCache.allocate(kcb, B, Hkv, t_cap)
    vc = T.CompressedCache.allocate(vcb, B, Hkv, t_cap)
    bb, hh, tt = torch.meshgrid(torch.arange(B), torch.arange(Hkv), torch.arange(S), indexing="ij")
    dst = ((bb * Hkv + hh) * t_cap + tt).reshape(-1).to(dev)
    T.encode_into_cache(kcb, up(wl.k), kc, dst_row=dst)
    T.encode_into_cache(vcb, up(wl.v), vc, dst_row=dst)
    del dst
    ins = []
    for s in range(steps):
        ka, va, qa = synth.appended_tokens(s, batch=B) if B == 16 else (None, None, None)
        if ka is None:
            rng = np.random.default_rng(1000 + s)
            ka = synth.bf16_bits(rng.standard_normal((B, Hkv, 1, 128), dtype=np.float32))
            va = synth.bf16_bits(rng.standard_normal((B, Hkv, 1, 128), dtype=np.float32))
            qa = synth.bf16_bits(rng.standard_normal((B, Hq, 128), dtype=np.float32))
        tob = lambda a, shape: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev).reshape(shape)
        ins.append((tob(ka, (B, Hkv, 128)), tob(va, (B, Hkv, 128)), tob(qa, (B, Hq, 128))))
    ws = T.alloc_workspace(B, Hq, Hkv, t_cap, dev)
    out = torch.empty(B, Hq, 128, dtype=torch.bfloat16, device=dev)
    seq = torch.full((B,), S, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(run):
        seq.fill_(S)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(steps):
            run(s)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    def separate(s):
        kn, vn, q = ins[s]
        rows = torch.tensor([(b * Hkv + h) * t_cap + S + s for b in range(B) for h in range(Hkv)],
                            dtype=torch.int64).to(dev, non_blocking=False)
        T.encode_into_cache(kcb, kn.reshape(-1, 128), kc, dst_row=rows, stream=stream)
        T.encode_into_cache(vcb, vn.reshape(-1, 128), vc, dst_row=rows, stream=stream)
        sl = torch.full((B,), S + s + 1, dtype=torch.int32, device=dev)
        T.decode_attention(kcb, vcb, q, kc, vc, sl, out=out, workspace=ws, stream=stream)

    def fused(s):
        kn, vn, q = ins[s]
        T.append_decode(kcb, vcb, kn, vn, q, kc, vc, seq, out=out, workspace=ws, stream=stream)

    kn_s = torch.empty_like(ins[0][0]); vn_s = torch.empty_like(ins[0][1]); q_s = torch.empty_like(ins[0][2])
    timed(fused)                                     # warm-up
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side), torch.cuda.graph(graph, stream=side):
        T.append_decode(kcb, vcb, kn_s, vn_s, q_s, kc, vc, seq, out=out, workspace=ws, stream=side)
    stream.wait_stream(side)

    def replay(s):
        graph.replay()

    # the graph's static inputs hold step 0's token (in a serving loop the
    # projections that produce k, v, q would write them there)
    kn_s.copy_(ins[0][0]); vn_s.copy_(ins[0][1]); q_s.copy_(ins[0][2])
    res = {"steps": steps, "separate_calls": round(timed(separate), 2), "append_decode": round(timed(fused), 2),
           "append_decode_graph": round(timed(replay), 2),
           "decode_only": round(timed(lambda s: T.decode_attention(kcb, vcb, ins[s][2], kc, vc, seq, out=out,
                                                                     workspace=ws, stream=stream)), 2),
           "cache": "resident (no replica rotation)",
           "note": "graph replays reuse one step's inputs, already in the captured buffers"}
    return res


def encode_counters(workload_name):
    """Counter figures of one key-encode launch on this workload, or None when
    they are missing or the encode source changed since they were taken."""
    t = ENCODE_COUNTERS.get(workload_name)
    if t is None or encode_source_sha256() != t["source_sha256"]:
        return None
    return t


def encode_traffic(workload_name):
    """Counter-measured HBM bytes of one key-encode launch (FETCH_SIZE + WRITE_SIZE, scaled), or None."""
    t = encode_counters(workload_name)
    return None if t is None else t["fetch_bytes"] + t["write_bytes"]


def key_encode_mfma(n_vec, qjl_m, x_bf16, ms, workload_name):
    """The key encode against the bf16 matrix-core peak: algorithmic flops
    (2 d^2 for the rotation + 2 m d for the QJL product per vector) and flops
    as issued by the hi/lo operand splits (rotation: 2 products per product for
    bf16 input, 3 for fp32; QJL: 3), plus the counters' busy fractions."""
    alg = n_vec * 2.0 * 128 * (128 + qjl_m)
    rot_passes = 2 if x_bf16 else 3
    issued = n_vec * 2.0 * 128 * (rot_passes * 128 + 3 * qjl_m)
    sec = ms * 1e-3
    c = encode_counters(workload_name)
    return {"bound": "mfma", "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "achieved_algorithmic": round(alg / sec / 1e12, 1), "frac_algorithmic": round(alg / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "achieved_issued": round(issued / sec / 1e12, 1), "frac_issued": round(issued / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "flops_per_launch_algorithmic": alg, "flops_per_launch_issued": issued,
            "counters_mfma_busy": None if c is None else c["mfma_busy"],
            "counters_valu_busy": None if c is None else c["valu_busy"]}


def encode_source_sha256():
    """sha256 over the encode kernel's sources (tq_encode.hip, then tq_encode_body.inc)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("tq_encode.hip", "tq_encode_body.inc"):
        with open(os.path.join(ROOT, "online_vector_quantization_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def cpu_baseline(wl, min_seconds, qjl=True):
    """The CPU oracle (float64 numpy) on the same step: encode every K and V
    vector of the layer, then decode all q heads over the full cache.  The step
    is repeated until at least `min_seconds` of CPU work have run."""
    import oracle as O
    from online_vector_quantization_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    B, Hkv, S = wl.batch, wl.n_kv_heads, wl.seq_len
    kb = wl.k_bits - 1 if qjl else wl.k_bits
    c_k, t_k = O.build_codebook(128, kb)
    c_v, t_v = O.build_codebook(128, wl.v_bits)
    Pi = O.haar_rotation(128, 0)
    Sm = O.qjl_matrix(128, 128, 1) if qjl else None
    kx = synth.bf16_to_f32(wl.k.reshape(-1, 128))
    vx = synth.bf16_to_f32(wl.v.reshape(-1, 128))
    qh = synth.bf16_to_f32(wl.q).astype(np.float64)
    shape = (B, Hkv, S)
    t_enc = t_dec = 0.0
    reps = 0
    while reps == 0 or t_enc + t_dec < min_seconds:
        t0 = time.perf_counter()
        ek = O.encode(kx, Pi, c_k, t_k, Sm)
        ev = O.encode(vx, Pi, c_v, t_v)
        kcache = {"codes": O.pack_bits(ek["idx"], kb).reshape(*shape, -1),
                  "signs": O.pack_bits(ek["z"], 1).reshape(*shape, -1) if qjl else None,
                  "norms": ek["nu"].reshape(shape), "res_norms": ek["gamma"].reshape(shape) if qjl else None}
        vcache = {"codes": O.pack_bits(ev["idx"], wl.v_bits).reshape(*shape, -1), "norms": ev["nu"].reshape(shape)}
        t1 = time.perf_counter()
        O.decode_attention(qh, kcache, vcache, [S] * B, {"bits": kb, "centroids": c_k, "Pi": Pi, "S": Sm},
                           {"bits": wl.v_bits, "centroids": c_v, "Pi": Pi})
        t2 = time.perf_counter()
        t_enc += t1 - t0
        t_dec += t2 - t1
        reps += 1
    n_vec = B * Hkv * S
    rec = (4 * 4 * kb + (16 + 8 if qjl else 4)) + (4 * 4 * wl.v_bits + 4)
    dec_gbps = reps * n_vec * rec / t_dec / 1e9
    return {"value": round(dec_gbps, 4), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
            "encode_mvectors_per_s": round(reps * 2 * n_vec / t_enc / 1e6, 4),
            "sample": f"the whole step on the CPU, {reps}x: oracle encode of all {n_vec} K and {n_vec} V vectors "
                      f"({t_enc / reps:.2f}s each), then oracle decode of all {wl.n_q_heads} q heads over the "
                      f"{S}-token cache ({t_dec / reps:.2f}s each); GB/s = compressed bytes read / decode time",
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
