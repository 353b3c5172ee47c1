"""Host-side pieces of bench.py: the one-GPU guard, the algorithmic byte
count of a decode launch and the lookup of the committed counter summaries."""

import os
import subprocess
import sys

import bench
import paged_kv_attention_gqa_amd as pkv
from inputs import make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_algorithmic_bytes_by_hand():
    # tiny: two sequences of 17 and 64 tokens, one worker each, written directly
    w = make_config("tiny")
    flat = pkv.pkv_plan_export(pkv.pkv_plan_create(w.kv_indptr, num_cus=256))
    n_workers, n_segs, _, n_slots = flat[:4]
    assert (n_workers, n_segs, n_slots) == (2, 2, 0)
    want = 2048 * 81 + 4 * 81 + 8192 * 2 + 2 * (8192 + 128) + 32 * 2
    assert bench.algorithmic_decode_bytes(w, flat) == want


def test_traffic_summaries_are_consistent():
    """A committed decode summary is used only while the kernel and the plan
    sources are the ones it was taken with; then its counted bytes are within
    2% above the algorithmic bytes of the same plan."""
    for cfg in ("gqa", "edge", "throughput"):
        t = bench.read_traffic(cfg)
        if t is None:      # sources changed since the counters were taken
            continue
        w = make_config(cfg)
        flat = pkv.pkv_plan_export(pkv.pkv_plan_create(w.kv_indptr, num_cus=256))
        ratio = t / bench.algorithmic_decode_bytes(w, flat)
        assert 1.0 <= ratio < 1.02, (cfg, ratio)
    assert bench.read_traffic("no_such_workload") is None
