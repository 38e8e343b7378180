"""Host-side logic of bench.py (no GPU): the committed HBM-traffic summaries it reads,
their arithmetic, the label / source-hash lookup, and the one-GPU refusal."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.txt")))

# GPT-175B shard 0 of tp=8: tokens, hidden, FFN shard width
M, H, FT = 2048, 12288, 6144
ALGORITHMIC = {
    # read V2, W1, b1; write A and Z (bf16)
    "fc1_fwd": M * H * 2 + FT * H * 2 + FT * 2 + 2 * M * FT * 2,
    # read dOut (dgrad and wgrad), W2, A, Z (bf16); write dA (bf16), dW2 (fp32) and the
    # per-128-row column sums of dA (fp32, the FC1 bias gradient's partials)
    "fc2_dgrad_wgrad": 2 * M * H * 2 + H * FT * 2 + 2 * M * FT * 2 + M * FT * 2 + H * FT * 4 + (M // 128) * FT * 4,
}


def _fields(path):
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


def _num(s):
    return float(s.split()[0])


def test_summary_exists_for_the_default_kernel(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    args = bench.parse()
    assert args.dominant == "fc2_dgrad_wgrad" and args.gpus == 1
    assert os.path.exists(bench.traffic_file(args.dominant))


@pytest.mark.parametrize("path", SUMMARIES, ids=[os.path.basename(p) for p in SUMMARIES])
def test_traffic_summary_arithmetic(path):
    kv = _fields(path)
    label = kv["label"]
    assert os.path.basename(path) == os.path.basename(bench.traffic_file(label))
    copy_bytes = 536870912
    ff = copy_bytes / (_num(kv["copy_fetch_kib"]) * 1024)
    fw = copy_bytes / (_num(kv["copy_write_kib"]) * 1024)
    assert abs(ff - 2.0) < 1e-3 and abs(fw - 1.0) < 1e-3  # gfx950: FETCH_SIZE counts half of a copy's reads
    traffic = _num(kv["fetch_kib_per_dispatch"]) * 1024 * ff + _num(kv["write_kib_per_dispatch"]) * 1024 * fw
    assert abs(traffic - _num(kv["traffic_bytes_per_launch"])) <= 1e-5 * traffic
    alg = _num(kv["algorithmic_bytes_per_launch"])
    if label in ALGORITHMIC:
        assert alg == ALGORITHMIC[label]
    assert abs(traffic / alg - _num(kv["traffic_over_algorithmic"])) < 1e-3
    assert traffic >= alg  # counters cannot read below the bytes the kernel must move
    if "kernel_trace_avg_us_timed_pass" in kv:  # the trace and the bench's events time the same launches
        tr, ev = _num(kv["kernel_trace_avg_us_timed_pass"]), _num(kv["event_avg_us_same_command"])
        assert abs(tr - ev) <= 0.05 * ev


@pytest.mark.parametrize("path", SUMMARIES, ids=[os.path.basename(p) for p in SUMMARIES])
def test_traffic_lookup_follows_the_source_hash(path):
    kv = _fields(path)
    got = bench.committed_traffic(kv["label"])
    if kv["gemm_source_hash"] == bench.gemm_source_hash():
        assert got == _num(kv["traffic_bytes_per_launch"])
    else:
        assert got is None  # kernels changed since the counters were taken
    assert bench.committed_traffic("no_such_launch") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_workload_modes_follow_the_green_parity_tests():
    """bench.py reports a workload only in a mode whose oracle parity test exists: the 1T
    shard and the h=8192 stage default to (and only allow) the compensated logits."""
    import bench
    import seeded_inputs as si
    assert set(bench.PARITY_MODES) == set(si.WORKLOADS)
    assert bench.workload_mode("gpt175b_tp8") == "bf16"
    assert bench.workload_mode("gpt175b_tp8", "bf16qk") == "bf16qk"
    assert bench.workload_mode("gpt1t_tp8") == "bf16qk"
    assert bench.workload_mode("gpt_h8192_stage_mb4") == "bf16qk"
    for wl, mode in (("gpt1t_tp8", "bf16"), ("gpt_h8192_stage_mb2", "bf16"), ("gpt175b_tp8", "fp32")):
        with pytest.raises(SystemExit):
            bench.workload_mode(wl, mode)
