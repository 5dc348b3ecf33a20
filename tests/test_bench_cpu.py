"""bench.py's host logic on the CPU: the one-GPU contract, the algorithmic
byte and flop counts the reported rates divide by, and the digest that ties
recorded counter traffic to the kernel source it was taken with."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_options():
    out = _run("--help").stdout
    for opt in ("--steps", "--warmup", "--workload", "--argmax", "--lm-rows", "--load-shard",
                "--timed-events", "--no-breakdown", "--library-gemm", "--copy-probe-mib",
                "--no-extra-workloads", "--logsumexp"):
        assert opt in out, opt


def _owned(w, ids):
    return [int(np.count_nonzero((ids >= w.rank_start(r)) & (ids < w.rank_start(r) + w.shard_rows)))
            for r in w.ranks]


def test_default_step_bytes_and_flops():
    w = wl.WORKLOADS[bench.DEFAULT_WORKLOAD]
    ids = wl.workload_ids(w)
    owned = _owned(w, ids)
    b, f = bench.algorithmic_bytes(w, ids, owned)
    M, R, D, s = w.lm_rows, w.shard_rows, w.dim, 2
    assert (M, R, D) == (256, 75968, 1024)
    # X read + shard read + logits written
    assert b["lmhead"] == [195_002_368] == [M * D * s + R * D * s + M * R * s]
    assert f["lmhead"] == [2 * M * R * D]
    # ids read, every output row written, owned rows read (zeros are written unread)
    assert b["embed"] == [ids.size * 4 + ids.size * D * s + owned[0] * D * s]
    assert 0 < owned[0] < ids.size
    assert set(b) == {"embed", "lmhead"}


def test_all_ranks_and_prefill_bytes():
    w = wl.WORKLOADS["qwen3_0p6b_tp2_all_ranks"]
    ids = wl.workload_ids(w)
    owned = _owned(w, ids)
    b, _ = bench.algorithmic_bytes(w, ids, owned)
    n, D = ids.size, w.dim
    assert sum(owned) == n  # every id in [0, V) is owned by exactly one rank
    assert b["sum"] == [3 * n * D * 2]  # two partials read, the sum written
    assert len(b["lmhead"]) == 2
    w = wl.WORKLOADS["qwen3_0p6b_tp1_prefill"]
    ids = wl.workload_ids(w)
    b, _ = bench.algorithmic_bytes(w, ids, _owned(w, ids), fused_prefill=False)
    assert b["select"] == [w.seqs * (4 + 2 * w.dim * 2)]
    b, _ = bench.algorithmic_bytes(w, ids, _owned(w, ids), fused_prefill=True)
    assert "select" not in b


def test_greedy_pick_bytes():
    w = wl.WORKLOADS[bench.DEFAULT_WORKLOAD]
    ids = wl.workload_ids(w)
    b, f = bench.algorithmic_bytes(w, ids, _owned(w, ids), argmax=True)
    M, R, D = w.lm_rows, w.shard_rows, w.dim
    assert "lmhead" not in b
    assert b["lmhead_argmax"] == [M * D * 2 + R * D * 2 + M * 8]
    assert b["argmax_decode"] == [M * (8 + 8 + 12)]
    assert f["lmhead_argmax"] == [2 * M * R * D]


def test_source_digest_ignores_comments_and_spacing(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("// header\nint f(int x) {\n  return x + 1;  /* one */\n}\n")
    b = tmp_path / "b.hip"
    b.write_text("int f(int x) {   return x + 1; }\n// trailing note\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest(str(a)) == bench.source_digest(str(b))
    assert bench.source_digest(str(a)) != bench.source_digest(str(c))


def test_unknown_traffic_record_is_none():
    assert bench.recorded_traffic("no_such_workload", "lmhead") is None


def test_traffic_key_follows_the_lm_head_configuration():
    k = bench.traffic_key
    assert k("qwen3_0p6b_tp2_rank0", "lmhead") == "qwen3_0p6b_tp2_rank0"
    assert k("qwen3_0p6b_tp2_rank0", "lmhead", 16) == "qwen3_0p6b_tp2_rank0@m16"
    assert k("qwen3_0p6b_tp2_rank0", "lmhead_argmax", 8) == "qwen3_0p6b_tp2_rank0@m8"
    assert k("qwen3_0p6b_tp2_rank0", "embed", 16) == "qwen3_0p6b_tp2_rank0"  # same lookup
    assert k("qwen3_0p6b_tp1_prefill", "lmhead", 0, True) == "qwen3_0p6b_tp1_prefill@unfused"
    assert k("qwen3_0p6b_tp1_prefill", "select", 0, True) == "qwen3_0p6b_tp1_prefill@unfused"
    assert k("qwen3_0p6b_tp1_prefill", "embed", 0, True) == "qwen3_0p6b_tp1_prefill"
    # a configuration whose counters were never recorded reports none
    assert bench.recorded_traffic(k("qwen3_0p6b_tp2_rank0", "lmhead", 3), "lmhead") is None


def test_extra_configurations_cover_every_workload():
    names = {n for n, _ in bench.EXTRA_RUNS}
    assert names | {bench.DEFAULT_WORKLOAD} >= set(wl.WORKLOAD_ORDER) - {"tiny_v4096_d64_f32_tp2"}
    assert ("qwen3_0p6b_tp2_rank0", 1) in bench.EXTRA_RUNS
    assert ("qwen3_0p6b_tp2_rank0", 16) in bench.EXTRA_RUNS


def test_extra_configurations_only_with_the_default_step():
    import argparse
    base = dict(no_extra_workloads=False, workload=bench.DEFAULT_WORKLOAD, lm_rows=0,
                argmax=False, unfused_prefill=False, timed_events="dominant", no_breakdown=False,
                library_gemm=False, copy_probe_mib=0)
    assert bench.want_extra_runs(argparse.Namespace(**base))
    for k, v in [("no_extra_workloads", True), ("workload", "qwen3_0p6b_tp1_prefill"),
                 ("lm_rows", 8), ("argmax", True), ("unfused_prefill", True),
                 ("timed_events", "none"), ("no_breakdown", True), ("library_gemm", True),
                 ("copy_probe_mib", 256)]:
        assert not bench.want_extra_runs(argparse.Namespace(**{**base, k: v})), k


def test_kernel_bound_follows_the_ridge_point():
    # [256, 75968] x 1024: 204 flop/B, under the 312.5 ridge -> HBM
    w = wl.WORKLOADS["qwen3_0p6b_tp2_rank0"]
    b = 256 * 1024 * 2 + 75968 * 1024 * 2 + 256 * 75968 * 2
    assert bench.kernel_bound("lmhead", "bf16", b, 2 * 256 * 75968 * 1024) == "hbm"
    # [1024, 75968] x 1024: 510 flop/B -> MFMA
    b = 1024 * 1024 * 2 + 75968 * 1024 * 2 + 1024 * 75968 * 2
    assert bench.kernel_bound("lmhead", "bf16", b, 2 * 1024 * 75968 * 1024) == "mfma"
    assert bench.kernel_bound("embed", "bf16", 1e6, 0) == "hbm"
    assert bench.kernel_bound("lmhead", "f32", 1.0, 1e9) == "hbm"
    del w


def test_logsumexp_step_bytes():
    w = wl.WORKLOADS["qwen3_0p6b_tp2_all_ranks"]
    ids = wl.workload_ids(w)
    b, f = bench.algorithmic_bytes(w, ids, _owned(w, ids), logsumexp=True)
    M, R, D, s = w.lm_rows, w.shard_rows, w.dim, 2
    assert b["lmhead_lse"] == [M * D * s + R * D * s + M * R * s + M * 4] * 2
    assert b["lse_combine"] == [3 * M * 4]
    assert f["lmhead_lse"] == [2 * M * R * D] * 2
    assert "lmhead" not in b


def test_prefill_logsumexp_step_bytes():
    # fused: the log-sum-exp LM head reads the selected rows itself (no select)
    w = wl.WORKLOADS["qwen3_0p6b_tp1_prefill"]
    ids = wl.workload_ids(w)
    b, f = bench.algorithmic_bytes(w, ids, _owned(w, ids), fused_prefill=True, logsumexp=True)
    M, R, D, s = w.lm_rows, w.shard_rows, w.dim, 2
    assert b["lmhead_lse"] == [M * D * s + R * D * s + M * R * s + M * 4]
    assert "select" not in b and "lse_combine" not in b
    b2, _ = bench.algorithmic_bytes(w, ids, _owned(w, ids), fused_prefill=False, logsumexp=True)
    assert b2["select"] == [w.seqs * (4 + 2 * D * s)]
