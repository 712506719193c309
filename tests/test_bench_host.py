"""Host-side pieces of bench.py (CPU): the one-GPU contract, the statistics,
the algorithmic byte counts behind the rooflines, and the committed counter
summaries' bookkeeping."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    """--gpus N > 1 exits with status 2 and says why, before any GPU work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stats_nearest_rank():
    s = bench.stats([5.0, 1.0, 4.0, 2.0, 3.0, 10.0, 6.0, 7.0, 9.0, 8.0, 0.0])
    assert s == {"mean": 5.0, "median": 5.0, "p10": 1.0, "p90": 9.0, "n": 11}


def test_gsa_algorithmic_bytes_at_the_training_shape():
    """q, k, v and the gate logits read once and o written once, bf16: 1152 B
    per token-head at d 128, m 64 (75.5 MB at B8 H4 T2048); the states add
    4 B per element once each way when present."""
    _, nbytes = bench.gsa_alg(8, 4, 2048, 128, 128, 64, 64, 2)
    assert nbytes == 1152 * 8 * 4 * 2048
    _, with_states = bench.gsa_alg(1, 8, 16384, 128, 128, 64, 64, 2, init_state=True, final_state=True)
    assert with_states == 1152 * 8 * 16384 + 2 * 8 * 64 * 256 * 4


def test_rooflines_are_bytes_over_time():
    r = bench.op_roofline(8e9, 1.0)  # 8 GB in 1 ms: the published peak exactly
    assert r["frac"] == 1.0 and r["unit"] == "GB/s" and r["bound"] == "hbm"


def test_counter_summaries_name_one_source_hash():
    """Every entry of profiles/counters.json was taken on one set of kernel
    sources, and every profile summary names that hash; bench.py reports
    traffic only while it matches the current sources."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    cj = json.load(open(path))
    shas = {rec["source_sha"] for rec in cj.values()}
    assert len(shas) == 1
    sha = shas.pop()
    for f in os.listdir(os.path.join(ROOT, "profiles")):
        if f.endswith(".md"):
            text = open(os.path.join(ROOT, "profiles", f)).read()
            m = re.search(r"`kernel_source_sha` ([0-9a-f]{16})", text)
            if m:
                assert m.group(1) == sha, f
    for key, rec in cj.items():
        # each of the three is the scaled counter rounded down on its own
        assert abs(rec["hbm_bytes_per_launch"] - rec["read_bytes"] - rec["write_bytes"]) <= 1, key
    if sha == bench.kernel_source_sha():
        assert bench.load_traffic("gsa_bf16_out", "gsa_bf16_train_T2048") is not None
    else:
        assert bench.load_traffic("gsa_bf16_out", "gsa_bf16_train_T2048") is None
