"""Host-side logic of bench.py (no GPU): the decode's vector-ALU view and the
gate that reports counter-measured encode traffic only for the sources the
counters were taken on."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_decode_mfma_view(bench):
    # the 8B layer: 8 kv heads x 32768 tokens, g = 4, QJL keys, in 31 us.
    # Issued: 20 v_mfma_f32_16x16x32 (16384 flops) per 16 tokens of a kv head;
    # algorithmic: 2 (d + m + d) flops per (token, q head).
    v = bench.decode_mfma_view(8 * 32768, 4, 128, 0.031)
    assert v["flops_per_launch_issued"] == 8 * 32768 * 20 * 16384 / 16
    assert v["flops_per_launch_algorithmic"] == 8 * 32768 * 4 * 768
    assert v["achieved_issued"] == pytest.approx(8 * 32768 * 20480 / 31e-6 / 1e12, rel=1e-3)
    assert v["frac_issued"] == pytest.approx(v["achieved_issued"] / 2500.0, rel=1e-3)
    # MSE-only keys: no sign products
    assert bench.decode_mfma_view(16, 8, 0, 1.0)["flops_per_launch_issued"] == 16 * 16384


def test_encode_traffic_gate(bench, monkeypatch):
    wl, t = next(iter(bench.ENCODE_COUNTERS.items()))
    # counters taken on the current sources are reported, for their workload only
    monkeypatch.setattr(bench, "ENCODE_COUNTERS", {wl: dict(t, source_sha256=bench.encode_source_sha256())})
    assert bench.encode_traffic(wl) == t["fetch_bytes"] + t["write_bytes"]
    assert bench.encode_traffic("another-workload") is None
    assert bench.key_encode_mfma(1000, 128, True, 1.0, wl)["counters_mfma_busy"] == t["mfma_busy"]
    # counters taken on other sources, or none at all, are not
    monkeypatch.setattr(bench, "ENCODE_COUNTERS", {wl: dict(t, source_sha256="0" * 64)})
    assert bench.encode_traffic(wl) is None
    assert bench.key_encode_mfma(1000, 128, True, 1.0, wl)["counters_mfma_busy"] is None
    monkeypatch.setattr(bench, "ENCODE_COUNTERS", {})
    assert bench.encode_traffic(wl) is None


def test_key_encode_mfma_flops(bench):
    # 10^7 bf16 keys with m = 128 in 1 ms: 2 d (d + m) algorithmic flops per key;
    # issued, the rotation takes 2 bf16 products per product and the QJL 3
    n = 10 ** 7
    v = bench.key_encode_mfma(n, 128, True, 1.0, "none")
    assert v["flops_per_launch_algorithmic"] == n * 2 * 128 * 256
    assert v["flops_per_launch_issued"] == n * 2 * 128 * (2 * 128 + 3 * 128)
    assert v["achieved_issued"] == pytest.approx(n * 2 * 128 * 640 / 1e-3 / 1e12, rel=1e-3)
    assert bench.key_encode_mfma(1000, 0, False, 1.0, "none")["flops_per_launch_issued"] == 1000 * 2 * 128 * 3 * 128


def test_sub_record_drops_headline_keys(bench):
    line = {"metric": "m", "value": 1.0, "unit": "GB/s", "config": {"workload": "w"}, "steps": 3}
    assert bench.sub_record(line) == {"value": 1.0, "config": {"workload": "w"}}


def test_committed_counters_are_the_committed_profiles(bench):
    # the encode counters the bench line reports were taken on these sources,
    # and are the figures of the committed byte-counter summaries
    sha = bench.encode_source_sha256()
    summaries = {"llama3-8b-layer-b1-s32768": "encode_decode_llama8b_hbm_counters.md",
                 bench.BULK_NAME: "encode_decode_bulk_hbm_counters.md"}
    assert set(bench.ENCODE_COUNTERS) == set(summaries)
    for wl, t in bench.ENCODE_COUNTERS.items():
        assert t["source_sha256"] == sha, f"{wl}: counters taken on other encode sources"
        text = open(os.path.join(ROOT, "profiles", summaries[wl])).read()
        assert sha in text
        assert f"Key encode: {t['fetch_bytes'] / 1e6:.3f} MB read + {t['write_bytes'] / 1e6:.3f} MB written" in text
        issue = open(os.path.join(ROOT, "profiles", summaries[wl].replace("hbm", "issue"))).read()
        row = [r for r in issue.splitlines() if r.startswith("| encode keys") and r.count("|") > 8]
        assert len(row) == 1 and f"| {100 * t['mfma_busy']:.1f} | {100 * t['valu_busy']:.1f} |" in row[0]


def test_more_than_one_gpu_is_refused():
    # one GPU only: any other count exits with a message before touching a device
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
