"""Host-side checks of bench.py (no GPU): the one-GPU guard and the work
counts behind its roofline figures."""
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from sparse_bit_attention_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_attention_work_at_720p():
    """Kept pairs and MFMA work of the Wan-14B-720P layer: 40 heads x 1182
    query blocks x 118 kept blocks; per pair 2*64*64*128 ops for QK^T and as
    many bf16 flops for PV; per query block 4*64*d^2 for the linear epilogue."""
    b = load_bench()
    wl = synth.WORKLOADS["wan14b-720p"]
    i8, bf, pairs = b.attn_work(wl, 118, 1182)
    assert pairs == 40 * 1182 * 118 == 5_579_040
    assert i8 == pairs * 2 * 64 * 64 * 128
    assert bf == pairs * 2 * 64 * 64 * 128 + 40 * 1182 * 4 * 64 * 128 * 128
    z, bf2, _ = b.attn_work(wl, 118, 1182, qk_int8=False)
    assert z == 0 and bf2 == bf + i8
    # no linear term when every block is kept
    wl1 = synth.Workload("all", 1, 1, 640, 128, 1.0)
    assert b.attn_work(wl1, 10, 10)[1] == 10 * 10 * 2 * 64 * 64 * 128


def test_shard_workload_is_the_first_heads_of_720p():
    """The per-GPU share under 8-way head sharding is heads 0..4 of the 720P
    layer itself: same shapes, and the same Q, K, V for its first and last
    head (the generators are keyed by the flat element index)."""
    full, shard = synth.WORKLOADS["wan14b-720p"], synth.WORKLOADS["wan14b-720p-shard8"]
    assert (shard.B, shard.H * 8, shard.N, shard.d, shard.topk) == (full.B, full.H, full.N, full.d, full.topk)
    for h in (0, shard.H - 1):
        for a, c in zip(synth.head_inputs(shard, 0, h), synth.head_inputs(full, 0, h)):
            assert np.array_equal(a, c)
    assert np.array_equal(synth.proj_weight(shard), synth.proj_weight(full))


def test_backward_work_at_720p():
    b = load_bench()
    wl = synth.WORKLOADS["wan14b-720p"]
    pairs = 40 * 1182 * 118
    F = (128 * 128 + 128 + 127) // 128 * 128
    expect = (pairs * 7 * 2 * 64 * 64 * 128 + 40 * 1182 * 7 * 2 * 64 * 128 * 128
              + 40 * 2.0 * 1182 * 1182 * F)
    assert b.bwd_work(wl, 1182, 118) == pytest.approx(expect, rel=1e-12)


def test_traffic_entry_is_null_or_positive():
    """The HBM-traffic figure comes from the committed counter summary and is
    reported only while that summary was taken on the current kernel source."""
    b = load_bench()
    t = b.traffic_entry()
    assert t is None or t > 0
    meta = json.load(open(b.TRAFFIC_FILE))
    if meta.get("kernel_src_sha256_16") == b.src_hash(b.ATTN_SRC):
        assert t == meta["bytes_per_launch"]
    else:
        assert t is None


def test_cpu_baseline_fields_on_the_tiny_workload():
    b = load_bench()
    wl = synth.WORKLOADS["tiny"]
    r = b.cpu_baseline(wl, 8, log_fn=lambda *a: None, full=("tiny",))
    model, nproc = b.host_cpu()
    assert r["kind"] == "oracle" and r["host_cpu"] == model and r["nproc"] == nproc >= 1
    assert r["cores"] == r["all_core"]["threads"] == min(b.oracle_threads(nproc), wl.B * wl.H)
    assert r["value"] > 0 and r["single_core"]["value"] > 0
    assert r["full_runs"]["tiny"]["heads"] == wl.B * wl.H
    # the process affinity is restored after the pinned single-core run
    assert len(os.sched_getaffinity(0)) == nproc


def test_input_sha256_is_of_the_uploaded_bytes():
    import hashlib
    import numpy as np
    b = load_bench()
    a = np.arange(6, dtype=np.uint16).reshape(2, 3)
    assert b.input_sha256(q=a)["q"] == hashlib.sha256(a.tobytes()).hexdigest()
    # e3b0c442...: SHA-256 of the empty string (FIPS 180-4 test vector)
    assert b.input_sha256(e=np.zeros(0, np.uint16))["e"].startswith("e3b0c44298fc1c14")
