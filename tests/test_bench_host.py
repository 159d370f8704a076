"""Host-side rules of bench.py (no GPU): the one-GPU guard, the algorithmic
byte counts behind the roofline fractions, and the rule that counter
summaries from profiles/ are used only when they were taken on the current
kernel sources."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def fake_info(n=4096, k=1024, words=70_000, verbatim=13):
    groups = n * k // 64
    return SimpleNamespace(numel=n * k, n=n, k=k, stream_words=words, segments=groups // 4, groups=groups,
                           verbatim_groups=verbatim)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_algorithmic_bytes_by_hand():
    i = fake_info()
    M = 4096 * 1024
    Z, O, Aux, Vb = 4 * (70_000 + 2), 4 * (M // 256 + 1), 8 * ((M // 64 + 31) // 32), 64 * 13
    assert bench.algorithmic_bytes(i, "decode_full") == Z + O + Aux + Vb + 3 * M
    assert bench.algorithmic_bytes(i, "decode_exponent") == Z + O + Aux + Vb + M
    assert bench.algorithmic_bytes(i, "transcode") == Z + O + Aux + M / 2
    X, Y = 2 * 8 * 1024, 4 * 8 * 4096
    assert bench.algorithmic_bytes(i, "gemv_full", 8) == 2 * M + X + Y
    assert bench.algorithmic_bytes(i, "gemv_direct", 8) == 1.5 * M + Aux + Vb + X + Y


def test_pipeline_bytes_are_preprocessing_plus_gemm():
    i = fake_info()
    for b in (1, 64, 1024):
        pre = {0: "decode_full", 1: "decode_exponent", 2: "transcode"}
        gem = {0: "gemv_full", 1: "gemv_exponent", 2: "gemv_transcode", 3: "gemv_direct"}
        for p in range(4):
            want = (bench.algorithmic_bytes(i, pre[p]) if p in pre else 0) + bench.algorithmic_bytes(i, gem[p], b)
            assert bench.job_bytes(i, p, b) == pytest.approx(want)


def test_counter_summaries_follow_their_sources(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "traffic_gate8b.json")) as f:
        rec = json.load(f)["kernels"]["transcode"]
    with open(os.path.join(ROOT, "profiles", "decode_counters_gate8b.json")) as f:
        dec = json.load(f)["kernels"]["transcode"]
    # taken on these sources: the stored figures are used
    monkeypatch.setattr(bench, "source_sha", lambda stage: rec["source_sha"])
    assert bench.load_traffic("transcode") == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "source_sha", lambda stage: dec["source_sha"])
    assert bench.load_valu_floor("transcode")["valu_floor_us"] == dec["valu_floor_us"]
    # any other source: no figure at all rather than a stale one
    monkeypatch.setattr(bench, "source_sha", lambda stage: "0" * 16)
    assert bench.load_traffic("transcode") is None
    assert bench.load_valu_floor("transcode") is None
    assert bench.load_traffic("gemm_direct_down_b1024", "mlp70b") is None


def test_valu_floor_figures_restate_their_counts():
    with open(os.path.join(ROOT, "profiles", "decode_counters_gate8b.json")) as f:
        d = json.load(f)
    for k in d["kernels"].values():
        floor = k["valu_instr"] * d["valu_cycles_per_instr"] / (d["simds"] * d["clock_ghz"] * 1e3)
        assert k["valu_floor_us"] == pytest.approx(floor, rel=1e-3)
