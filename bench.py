#!/usr/bin/env python3
"""Benchmark of the vocab-parallel hot path on one MI355X.

A step is one pass of the whole path over one batch of the workload: every
emulated rank's masked embedding lookup, the on-device sum of the partials
(when several ranks run), the prefill last-position select (prefill
workloads), and every rank's LM-head logits written at its column offset.

Default workload: Qwen3-0.6B tp=2 rank-0 shard (table rows [0, 75968) of
151936 x 1024 bf16; 8192 uniform ids; LM head over 256 hidden rows ->
[256, 75968] logits).  Inputs are synthetic (seeded, see workloads.py) and
resident in HBM before timing starts.  Steps rotate through several copies
of every input and output, enough that at least 1 GiB of distinct input bytes
is read between two uses of the same copy, so that a step does not find its
table still in the 256 MB Infinity Cache.

Prints ONE JSON line.  The roofline entry is for the dominant kernel (most
algorithmic bytes): its duration comes from HIP events recorded on the launch
stream around its launches inside the timed region, the only events there
(timing-only events without the system-scope fence, see TimingEvent).
The per-kernel breakdown comes from a separate, untimed pass with events
around every call.

After the default step, the same process times every other workload at its
own size (the fused prefill, both tp=2 ranks concatenated, the hidden-4096
shard) and the default shard's LM head at decode batches of 1 and 16 rows,
each the same way, and reports them under "workloads": per configuration the
step time and, per kernel, its launch time and its fraction of the roofline
that bounds it (HBM bandwidth, or dense bf16 MFMA past the ridge point).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "embed rows/s + GB/s; LM-head logits GB/s (decode) & TFLOP/s (batch); %roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, AMD published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, AMD published
FP32_VECTOR_PEAK_TFLOPS = 157.3
DEFAULT_WORKLOAD = "qwen3_0p6b_tp2_rank0"
CACHE_DEFEAT_BYTES = 1 << 30  # rotate through at least this many bytes of inputs


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--copies", type=int, default=0,
                   help="input copies to rotate through (0 = enough for >= 1 GiB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-threads", type=int, default=0, help="0 = min(16, cores available)")
    p.add_argument("--unfused-prefill", action="store_true",
                   help="prefill workloads: separate last-position select + LM head instead of "
                        "the LM head that reads the last positions itself")
    p.add_argument("--argmax", action="store_true",
                   help="LM head reduced on the fly to each row's greedy pick (largest logit "
                        "and its id) instead of storing the logits")
    p.add_argument("--logsumexp", action="store_true",
                   help="LM head that also reduces every row to its log-sum-exp over the shard "
                        "(vpe_lmhead_logsumexp, or vpe_lmhead_prefill_logsumexp for prefill "
                        "workloads; logits stored), and the ranks' values combined "
                        "(vpe_logsumexp_combine) when several ranks run")
    p.add_argument("--lm-rows", type=int, default=0,
                   help="override the workload's LM-head rows M (decode batch size; "
                        "not for prefill workloads, whose M is the number of sequences)")
    p.add_argument("--load-shard", action="store_true",
                   help="time loading every rank's shard of the workload from the full table "
                        "on the device (the weight_loader step) instead of the hot path")
    p.add_argument("--library-gemm", action="store_true",
                   help="also time torch.mm (the vendor BLAS) on each LM-head shape, untimed "
                        "and outside the step, as a reference point for the LM-head kernels")
    p.add_argument("--timed-events", choices=("dominant", "none"), default="dominant",
                   help="HIP events inside the timed region: around each launch of the dominant "
                        "kernel (default), or none (a diagnostic run for kernel traces of the "
                        "un-instrumented step; the roofline is then not measured)")
    p.add_argument("--no-breakdown", action="store_true",
                   help="skip the separate per-call event pass (a diagnostic run: a kernel "
                        "trace then holds only the warmup and timed steps)")
    p.add_argument("--no-extra-workloads", action="store_true",
                   help="time only the chosen step; by default the unmodified default step is "
                        "followed by every other workload and two decode batch sizes, reported "
                        "under \"workloads\"")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="after timing, run one device-to-device copy of this many MiB "
                        "(a reference kernel for hardware byte counters)")
    return p.parse_args()


class _Hip:
    """The HIP runtime this process already uses (the one torch loaded), for
    timing events that torch's Event does not offer."""
    lib = None

    @classmethod
    def get(cls):
        if cls.lib is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    name = line.split()[-1]
                    if os.path.basename(name).startswith("libamdhip64.so"):
                        path = name
                        break
            if path is None:
                raise RuntimeError("bench.py: the HIP runtime is not loaded")
            lib = ctypes.CDLL(path)
            vp = ctypes.c_void_p
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [vp, vp]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            lib.hipEventDestroy.argtypes = [vp]
            cls.lib = lib
        return cls.lib


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: its
    record is a device timestamp without the system-scope release that a
    default event performs (an L2 writeback and invalidate that also slows the
    next kernel).  Elapsed times are read only after a device synchronize, so
    the event needs no fence to be ordered with the work it brackets."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self._hip = _Hip.get()
        self.ev = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")

    def record(self, stream):
        rc = self._hip.hipEventRecord(self.ev, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        import ctypes
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def __del__(self):
        if getattr(self, "ev", None) and self.ev.value:
            self._hip.hipEventDestroy(self.ev)


def source_digest(path: str) -> str:
    """sha256 of a kernel source with its comments and blank space removed: the
    code the counters were taken with, unchanged by edits to comments alone."""
    import hashlib
    import re
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"\s+", " ", text).strip()
    return hashlib.sha256(text.encode()).hexdigest()


def recorded_traffic(workload: str, kind: str):
    """HBM bytes per dispatch recorded by hardware counters (profiles/traffic.json),
    or None when none were recorded or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        k = rec["kernels"][f"{workload}/{kind}"]
        if source_digest(os.path.join(ROOT, k["source"])) != k["source_digest"]:
            return None
        cp = rec["copy_probes"][workload]
        return int((k["fetch_kib"] * cp["fetch_scale"] + k["write_kib"] * cp["write_scale"]) * 1024)
    except (OSError, KeyError, ValueError):
        return None


def traffic_key(workload: str, kind: str, lm_rows_override: int = 0,
                unfused_prefill: bool = False) -> str:
    """Workload name under which counter traffic of one kernel kind is recorded:
    the LM-head kinds (and the separate select) depend on the LM-head rows and
    on whether the prefill select is fused, the lookup and the sum do not."""
    if kind.startswith("lmhead") or kind == "select":
        if lm_rows_override:
            workload += f"@m{lm_rows_override}"
        if unfused_prefill:
            workload += "@unfused"
    return workload


def algorithmic_bytes(w, ids, ranks_owned, fused_prefill=False, argmax=False, logsumexp=False):
    """Bytes the method must move per step, by kernel kind: a lookup reads its
    ids and owned rows and writes every output row; the sum reads each partial
    and writes one; the select reads the sequence ends and copies the rows;
    an LM head reads X and W once and writes (or, for the greedy pick and the
    log-sum-exp without logits, reduces) the logits."""
    s = w.elem_bytes
    D = w.dim
    idb = ids.dtype.itemsize
    out = {}
    n = ids.size
    # embed per rank: read ids, write every output row, read only owned rows
    out["embed"] = [n * idb + n * D * s + h * D * s for h in ranks_owned]
    if len(w.ranks) > 1:
        out["sum"] = [(len(w.ranks) + 1) * n * D * s]
    if w.seqs and not fused_prefill:
        out["select"] = [w.seqs * (4 + 2 * D * s)]
    M = w.lm_rows
    R = w.shard_rows
    if argmax:
        # keys: 8 bytes per row folded by every shard, then read and cleared by
        # the decode (which also writes 4 + 8 bytes per row), so the next step
        # needs no init
        out["lmhead_argmax"] = [M * D * s + R * D * s + M * 8 for _ in w.ranks]
        out["argmax_decode"] = [M * (8 + 8 + 12)]
        flops = {"lmhead_argmax": [2 * M * R * D for _ in w.ranks]}
    elif logsumexp:
        # as the stored-logits LM head, plus each row's value (4 bytes); the
        # tile pairs live in a workspace of a few MB and are not counted
        out["lmhead_lse"] = [M * D * s + R * D * s + M * R * s + M * 4 for _ in w.ranks]
        flops = {"lmhead_lse": [2 * M * R * D for _ in w.ranks]}
        if len(w.ranks) > 1:
            out["lse_combine"] = [(len(w.ranks) + 1) * M * 4]
    else:
        out["lmhead"] = [M * D * s + R * D * s + M * R * s for _ in w.ranks]
        flops = {"lmhead": [2 * M * R * D for _ in w.ranks]}
    return out, flops


# Configurations timed in the same process after the headline one and
# reported under "workloads": every other workload at its own size, and the
# default shard's LM head at two decode batch sizes (workload name, LM rows or
# 0 for the workload's own).
EXTRA_RUNS = (
    ("qwen3_0p6b_tp1_prefill", 0),
    ("qwen3_0p6b_tp2_all_ranks", 0),
    ("large_v151936_d4096_tp4_rank2", 0),
    ("qwen3_0p6b_tp2_rank0", 1),
    ("qwen3_0p6b_tp2_rank0", 16),
)


def kernel_bound(kind, dtype, nbytes, nflops):
    """The roofline that bounds one launch: 'mfma' for a bf16 contraction past
    the ridge point (flops / bytes above peak flops / peak bytes), else 'hbm'."""
    ridge = (BF16_MFMA_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9)
    if dtype == "bf16" and nflops and nbytes and nflops / nbytes > ridge:
        return "mfma"
    return "hbm"


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: vocab_sharded_embedding_amd runs on one GPU; --gpus {args.gpus} is not supported "
              "(tensor-parallel ranks are emulated on one device)", file=sys.stderr)
        sys.exit(2)

    import torch

    import vocab_sharded_embedding_amd as vpe
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no HIP device visible", file=sys.stderr)
        sys.exit(2)
    if args.workload not in wl.WORKLOADS:
        print(f"bench.py: unknown workload {args.workload}; choose from {wl.WORKLOAD_ORDER}",
              file=sys.stderr)
        sys.exit(2)
    w = wl.WORKLOADS[args.workload]
    if args.lm_rows:
        if w.seqs:
            print("bench.py: --lm-rows applies to decode workloads only", file=sys.stderr)
            sys.exit(2)
        import dataclasses
        w = dataclasses.replace(w, lm_rows=args.lm_rows)
    dev = torch.device("cuda:0")
    lib = vpe.load_library()

    if args.load_shard:
        return bench_load_shard(args, w, lib, dev, _uploader(torch, dev))

    if args.logsumexp and args.argmax:
        print("bench.py: --logsumexp applies to the LM head with stored logits, not to --argmax",
              file=sys.stderr)
        sys.exit(2)
    res = measure(args, w, lib, dev, argmax=args.argmax, unfused_prefill=args.unfused_prefill,
                  timed_events=args.timed_events, breakdown=not args.no_breakdown,
                  library_gemm=args.library_gemm, copy_probe_mib=args.copy_probe_mib,
                  lm_override=args.lm_rows,
                  # (the oracle baseline covers the plain step: not the log-sum-exp variant)
                  with_cpu=not args.no_cpu_baseline and not args.logsumexp,
                  logsumexp=args.logsumexp)

    extras = None
    if want_extra_runs(args):
        extras = {}
        for name, rows in EXTRA_RUNS:
            we = wl.WORKLOADS[name]
            if rows:
                import dataclasses
                we = dataclasses.replace(we, lm_rows=rows)
            key = name + (f"@m{rows}" if rows else "")
            r = measure(args, we, lib, dev, argmax=False, unfused_prefill=False,
                        timed_events="dominant", breakdown=True, library_gemm=False,
                        copy_probe_mib=0, lm_override=rows, with_cpu=False)
            extras[key] = summarize_extra(r)
            torch.cuda.empty_cache()

    w = res["w"]
    line = {
        "metric": METRIC, "value": round(res["value"], 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "vocab": w.vocab, "dim": w.dim, "tp": w.tp,
                   "ranks": list(w.ranks), "n_ids": res["n_ids"], "id_dist": w.id_dist,
                   "lm_rows": w.lm_rows, "seqs": w.seqs, "concat": w.concat,
                   "rotating_copies": res["copies"],
                   "prefill_select": ("fused" if res["fused_prefill"] else "separate")
                   if w.seqs else None,
                   "lm_output": ("argmax" if args.argmax else
                                 "logits+logsumexp" if args.logsumexp else "logits"),
                   "step_algorithmic_bytes": res["step_bytes"]},
        "roofline": res["roofline"],
        "cpu_baseline": res["cpu_baseline"],
        "breakdown": res["breakdown"],
        "workloads": extras,
        "library_gemm": res["library_gemm"],
        "device": torch.cuda.get_device_name(dev),
        "input_gen_s": round(res["gen_s"], 2),
    }
    print(json.dumps(line), flush=True)


def want_extra_runs(args) -> bool:
    """The other configurations run only with the default, unmodified step
    (diagnostic and single-workload runs, e.g. under a profiler, skip them)."""
    return (not args.no_extra_workloads and args.workload == DEFAULT_WORKLOAD
            and not args.lm_rows and not args.argmax and not args.unfused_prefill
            and not getattr(args, "logsumexp", False)
            and args.timed_events == "dominant" and not args.no_breakdown
            and not args.library_gemm and not args.copy_probe_mib)


def summarize_extra(r) -> dict:
    """One configuration's entry under "workloads": the step, and per kernel its
    launch time, rate and fraction of the roofline that bounds it."""
    w = r["w"]
    kernels = {}
    for kind, e in r["breakdown"].items():
        k = {"bound": e["bound"], "us_per_launch": e["us_per_launch"],
             "frac": e["frac"], "hbm_bytes_counted": e["hbm_bytes_counted"]}
        k["GB_per_s"] = e["GB_per_s"]
        if "TFLOP_per_s" in e:
            k["TFLOP_per_s"] = e["TFLOP_per_s"]
        if kind == "embed":
            k["rows_per_s"] = e["rows_per_s"]
        kernels[kind] = k
    roof = r["roofline"]
    return {"workload": w.name, "lm_rows": w.lm_rows, "n_ids": r["n_ids"],
            "rotating_copies": r["copies"], "ms_per_step": round(r["ms_per_step"], 5),
            "step_GB_per_s": round(r["value"], 2),
            "step_algorithmic_bytes": r["step_bytes"],
            "dominant": {"kernel": roof["kernel"], "bound": roof["bound"],
                         "avg_launch_us": roof["avg_launch_us"], "achieved": roof["achieved"],
                         "unit": roof["unit"], "frac": roof["frac"],
                         "traffic": roof["traffic"]},
            "kernels": kernels}


def _uploader(torch, dev):
    import numpy as np

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)
    return up


def measure(args, w, lib, dev, *, argmax, unfused_prefill, timed_events, breakdown,
            library_gemm, copy_probe_mib, lm_override, with_cpu, logsumexp=False):
    """Times args.steps steps of workload w (after args.warmup untimed ones) and
    returns the step rate, the dominant kernel's roofline entry and a per-kernel
    breakdown (see the module docstring for what is timed how)."""
    import numpy as np
    import torch

    import vocab_sharded_embedding_amd as vpe
    import workloads as wl

    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    up = _uploader(torch, dev)

    # ---------------- inputs (host, seeded) ----------------
    t0 = time.time()
    ids_h = wl.workload_ids(w)
    hidden_h = wl.workload_hidden(w)
    cu_h = wl.workload_cu_seqlens(w)
    shards_h = {r: wl.shard_table(w, r) for r in w.ranks}
    gen_s = time.time() - t0
    owned = [int(np.count_nonzero((ids_h >= w.rank_start(r)) &
                                  (ids_h < w.rank_start(r) + w.shard_rows))) for r in w.ranks]

    # ---------------- device copies ----------------
    M = w.lm_rows
    # Copies are counted from the inputs a step reads (tables, ids, hidden
    # states): outputs leave with non-temporal stores and need not evict them
    # from the Infinity Cache, so only distinct input bytes between two reads
    # of the same copy keep a step from finding its table still cached.
    per_copy = sum(a.nbytes for a in shards_h.values()) + ids_h.nbytes + hidden_h.nbytes
    copies = args.copies or max(1, -(-CACHE_DEFEAT_BYTES // per_copy))
    base = {"ids": up(ids_h), "hidden": up(hidden_h),
            "cu": up(cu_h) if cu_h is not None else None,
            "shards": {r: up(a) for r, a in shards_h.items()}}
    if not with_cpu:
        del shards_h
    sets = []
    for c in range(copies):
        d = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in base.items() if k != "shards"}
        d["shards"] = {r: t.clone() for r, t in base["shards"].items()}
        d["partials"] = [torch.empty((ids_h.size, w.dim), dtype=tdt, device=dev)
                         for _ in w.ranks]
        d["embed_out"] = (torch.empty((ids_h.size, w.dim), dtype=tdt, device=dev)
                          if len(w.ranks) > 1 else d["partials"][0])
        d["x"] = (torch.empty((w.seqs, w.dim), dtype=tdt, device=dev) if w.seqs
                  else d["hidden"])
        if argmax:
            d["best"] = torch.empty(M, dtype=torch.int64, device=dev)
            d["pick_val"] = torch.empty(M, dtype=torch.float32, device=dev)
            d["pick_tok"] = torch.empty(M, dtype=torch.int64, device=dev)
        else:
            d["logits"] = torch.empty((M, w.vocab if w.concat else w.shard_rows), dtype=tdt,
                                      device=dev)
        if logsumexp:
            ws_bytes = vpe.vpe_lmhead_logsumexp_workspace(M, w.shard_rows)
            d["lse_ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            d["shard_lse"] = [torch.empty(M, dtype=torch.float32, device=dev) for _ in w.ranks]
            d["lse"] = torch.empty(M, dtype=torch.float32, device=dev)
        sets.append(d)
    del base
    torch.cuda.synchronize()

    # ---------------- C-ABI argument tuples, marshalled once ----------------
    dcode = vpe.VPE_BF16 if w.dtype == "bf16" else vpe.VPE_F32
    icode = vpe.VPE_I32 if ids_h.dtype == np.int32 else vpe.VPE_I64
    import ctypes

    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    fused = bool(w.seqs) and not unfused_prefill
    calls = []  # per copy: list of (kind, fn, args)
    for d in sets:
        seq = []
        for i, r in enumerate(w.ranks):
            seq.append(("embed", lib.vpe_embed,
                        (d["ids"].data_ptr(), icode, ids_h.size, d["shards"][r].data_ptr(), dcode,
                         w.shard_rows, w.dim, w.rank_start(r), d["partials"][i].data_ptr(), sh)))
        if len(w.ranks) > 1:
            arr = (ctypes.c_void_p * len(w.ranks))(*[p.data_ptr() for p in d["partials"]])
            d["_arr"] = arr
            seq.append(("sum", lib.vpe_sum_partials,
                        (arr, len(w.ranks), ids_h.size * w.dim, dcode, d["embed_out"].data_ptr(),
                         sh)))
        if w.seqs and not fused:
            seq.append(("select", lib.vpe_last_token_select,
                        (d["hidden"].data_ptr(), hidden_h.shape[0], w.dim, dcode,
                         d["cu"].data_ptr(), w.seqs, d["x"].data_ptr(), sh)))
        for r in w.ranks:
            if argmax and fused:
                # the greedy pick reads each sequence's last position itself
                seq.append(("lmhead_argmax", lib.vpe_lmhead_prefill_argmax,
                            (d["hidden"].data_ptr(), hidden_h.shape[0], w.dim, d["cu"].data_ptr(),
                             w.seqs, d["shards"][r].data_ptr(), w.shard_rows, dcode,
                             w.rank_start(r), d["best"].data_ptr(), sh)))
            elif argmax:
                seq.append(("lmhead_argmax", lib.vpe_lmhead_argmax,
                            (d["x"].data_ptr(), M, w.dim, d["shards"][r].data_ptr(), w.shard_rows,
                             dcode, w.rank_start(r), d["best"].data_ptr(), sh)))
            elif logsumexp and fused:
                # the log-sum-exp LM head reads each sequence's last position itself
                i = list(w.ranks).index(r)
                seq.append(("lmhead_lse", lib.vpe_lmhead_prefill_logsumexp,
                            (d["hidden"].data_ptr(), hidden_h.shape[0], w.dim, d["cu"].data_ptr(),
                             w.seqs, d["shards"][r].data_ptr(), w.shard_rows, dcode,
                             d["logits"].data_ptr(), d["logits"].shape[1],
                             w.rank_start(r) if w.concat else 0, d["shard_lse"][i].data_ptr(),
                             d["lse_ws"].data_ptr(), d["lse_ws"].numel(), sh)))
            elif fused:
                # the LM head reads each sequence's last position itself
                seq.append(("lmhead", lib.vpe_lmhead_prefill,
                            (d["hidden"].data_ptr(), hidden_h.shape[0], w.dim, d["cu"].data_ptr(),
                             w.seqs, d["shards"][r].data_ptr(), w.shard_rows, dcode,
                             d["logits"].data_ptr(), d["logits"].shape[1],
                             w.rank_start(r) if w.concat else 0, sh)))
            elif logsumexp:
                i = list(w.ranks).index(r)
                seq.append(("lmhead_lse", lib.vpe_lmhead_logsumexp,
                            (d["x"].data_ptr(), M, w.dim, d["shards"][r].data_ptr(), w.shard_rows,
                             dcode, d["logits"].data_ptr(), d["logits"].shape[1],
                             w.rank_start(r) if w.concat else 0, d["shard_lse"][i].data_ptr(),
                             d["lse_ws"].data_ptr(), d["lse_ws"].numel(), sh)))
            else:
                seq.append(("lmhead", lib.vpe_lmhead,
                            (d["x"].data_ptr(), M, w.dim, d["shards"][r].data_ptr(), w.shard_rows,
                             dcode, d["logits"].data_ptr(), d["logits"].shape[1],
                             w.rank_start(r) if w.concat else 0, sh)))
        if logsumexp and len(w.ranks) > 1:
            larr = (ctypes.c_void_p * len(w.ranks))(*[t.data_ptr() for t in d["shard_lse"]])
            d["_larr"] = larr
            seq.append(("lse_combine", lib.vpe_logsumexp_combine,
                        (larr, len(w.ranks), M, d["lse"].data_ptr(), sh)))
        if argmax:
            # the decode clears the keys it reads: the next step's folds need no init
            seq.append(("argmax_decode", lib.vpe_argmax_decode_clear,
                        (d["best"].data_ptr(), M, d["pick_val"].data_ptr(),
                         d["pick_tok"].data_ptr(), sh)))
        calls.append(seq)

    bytes_, flops_ = algorithmic_bytes(w, ids_h, owned, fused_prefill=fused, argmax=argmax,
                                       logsumexp=logsumexp)
    step_bytes = sum(sum(v) for v in bytes_.values())
    # dominant kernel: most algorithmic bytes per step
    dom = max(bytes_, key=lambda k: sum(bytes_[k]))
    kinds = [c[0] for c in calls[0]]
    dom_idx = [j for j, kind in enumerate(kinds) if kind == dom]

    def run_step(k, events=None, which=()):
        """One step; events[j] brackets call j for every j in `which`."""
        for j, (kind, fn, a) in enumerate(calls[k % copies]):
            timed = events is not None and j in which
            if timed:
                events[j][0].record(stream)
            rc = fn(*a)
            if timed:
                events[j][1].record(stream)
            if rc != 0:
                raise RuntimeError(f"{kind} failed: {vpe.status_name(rc)}")

    def new_events():
        return [(TimingEvent(), TimingEvent())
                for _ in kinds]

    with torch.cuda.stream(stream):
        if argmax:
            # once per input copy, outside the steps: every step's decode leaves
            # its copy's keys cleared for that copy's next step
            for d in sets:
                rc = lib.vpe_argmax_init(d["best"].data_ptr(), M, sh)
                if rc != 0:
                    raise RuntimeError(f"argmax_init failed: {vpe.status_name(rc)}")
        for k in range(args.warmup):
            run_step(k)
        torch.cuda.synchronize()
        # timed region: events only around the dominant kernel's launches, so
        # that the step time carries no event records between the other calls
        evs = [new_events() for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        timed_idx = dom_idx if timed_events == "dominant" else ()
        for k in range(args.steps):
            run_step(k, evs[k], timed_idx)
        torch.cuda.synchronize()
        t_total = time.perf_counter() - t_start
        # per-kernel breakdown: a separate, untimed pass with every call bracketed
        n_bd = min(args.steps, 50) if breakdown else 0
        bd_evs = [new_events() for _ in range(n_bd)]
        for k in range(n_bd):
            run_step(k, bd_evs[k], range(len(kinds)))
        torch.cuda.synchronize()

    lib_gemm = None
    if library_gemm and "lmhead" in kinds:
        lib_gemm = library_gemm_reference(torch, sets, w, M, args, stream)

    if copy_probe_mib:
        src = torch.empty(copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def pcts(ms):
        return [round(float(v) * 1e3, 2) for v in np.percentile(ms, [10, 50, 90])]

    per_kind_ms, per_kind_pct = {}, {}
    for j, kind in enumerate(kinds if n_bd else ()):
        ms = [bd_evs[k][j][0].elapsed_time(bd_evs[k][j][1]) for k in range(n_bd)]
        per_kind_ms.setdefault(kind, []).append(float(np.mean(ms)))
        per_kind_pct.setdefault(kind, []).append(pcts(ms))
    dom_all = [[evs[k][j][0].elapsed_time(evs[k][j][1]) for k in range(args.steps)]
               for j in timed_idx]
    dom_ms = [float(np.mean(v)) for v in dom_all]

    ms_per_step = t_total * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    base_rows = wl.WORKLOADS[w.name].lm_rows
    lm_key = lm_override if lm_override and lm_override != base_rows else 0
    unfused = bool(w.seqs) and unfused_prefill

    def counted(kind):
        return recorded_traffic(traffic_key(w.name, kind, lm_key, unfused), kind)

    breakdown_ = {}
    for kind, lst in per_kind_ms.items():
        us = [m * 1e3 for m in lst]
        b = bytes_[kind]
        gbs = [bb / (u * 1e-6) / 1e9 for bb, u in zip(b, us)]
        e = {"us_per_launch": [round(u, 2) for u in us], "launches_per_step": len(us),
             "us_p10_p50_p90": per_kind_pct[kind],
             "GB_per_s": [round(g, 1) for g in gbs],
             "hbm_frac": [round(g / HBM_PEAK_GBS, 4) for g in gbs]}
        if kind == "embed":
            e["rows_per_s"] = [round(ids_h.size / (u * 1e-6), 1) for u in us]
        f = flops_.get(kind)
        if f:
            tf = [ff / (u * 1e-6) / 1e12 for ff, u in zip(f, us)]
            e["TFLOP_per_s"] = [round(t, 2) for t in tf]
            peak = BF16_MFMA_PEAK_TFLOPS if w.dtype == "bf16" else FP32_VECTOR_PEAK_TFLOPS
            e["mfma_frac" if w.dtype == "bf16" else "fp32_frac"] = [round(t / peak, 4) for t in tf]
        e["bound"] = kernel_bound(kind, w.dtype, float(np.mean(b)),
                                  float(np.mean(f)) if f else 0.0)
        e["frac"] = e["mfma_frac"] if e["bound"] == "mfma" else e["hbm_frac"]
        e["hbm_bytes_counted"] = counted(kind)
        breakdown_[kind] = e

    # the dominant kernel's duration, from the events of the timed region
    dom_us = float(np.mean(dom_ms)) * 1e3 if dom_ms else float("nan")
    dom_bytes = float(np.mean(bytes_[dom]))
    dom_flops = float(np.mean(flops_.get(dom, [0])))
    if kernel_bound(dom, w.dtype, dom_bytes, dom_flops) == "mfma":
        ach = dom_flops / (dom_us * 1e-6) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                "algorithmic_flops_per_launch": dom_flops}
    else:
        ach = dom_bytes / (dom_us * 1e-6) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes_per_launch": dom_bytes}
    roof["avg_launch_us"] = round(dom_us, 3)
    roof["launch_us_p10_p50_p90"] = pcts([v for lst in dom_all for v in lst]) if dom_ms else None
    if not dom_ms:
        # no events in the timed region: nothing measured the dominant kernel
        roof.update(achieved=None, frac=None, avg_launch_us=None,
                    note="--timed-events none: no events in the timed region")
    roof["traffic"] = counted(dom)

    # ---------------- CPU baseline: the oracle on the same workload ----------------
    cpu = None
    if with_cpu:
        cpu = cpu_baseline(w, ids_h, hidden_h, cu_h, step_bytes, args.cpu_threads,
                           shards=shards_h)
    del sets, calls
    return {"w": w, "value": value, "ms_per_step": ms_per_step, "step_bytes": step_bytes,
            "roofline": roof, "breakdown": breakdown_, "cpu_baseline": cpu,
            "library_gemm": lib_gemm, "copies": copies, "fused_prefill": fused,
            "n_ids": int(ids_h.size), "gen_s": gen_s}


def library_gemm_reference(torch, sets, w, M, args, stream):
    """torch.mm (hipBLASLt on ROCm) on each LM-head shape: X [M, D] times a shard's
    [R, D]^T into a contiguous [M, R] buffer, rotating through the same input copies.
    A reference point only: the timed step never calls it."""
    import numpy as np
    reps = max(1, min(args.steps, 50))
    out = torch.empty((M, w.shard_rows), dtype=sets[0]["x"].dtype, device=sets[0]["x"].device)
    res = []
    with torch.cuda.stream(stream):
        for r in w.ranks:
            def launch(k):
                d = sets[k % len(sets)]
                torch.mm(d["x"], d["shards"][r].t(), out=out)
            for k in range(3):
                launch(k)
            evs = [(TimingEvent(), TimingEvent())
                   for _ in range(reps)]
            for k in range(reps):
                evs[k][0].record(stream)
                launch(k)
                evs[k][1].record(stream)
            torch.cuda.synchronize()
            res.append(float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3)
    flops = 2.0 * M * w.shard_rows * w.dim
    return {"op": "torch.mm bf16, [M, D] x [R, D]^T -> contiguous [M, R]" if w.dtype == "bf16"
            else "torch.mm fp32, [M, D] x [R, D]^T -> contiguous [M, R]",
            "us_per_launch": [round(u, 2) for u in res],
            "TFLOP_per_s": [round(flops / (u * 1e-6) / 1e12, 2) for u in res]}


def bench_load_shard(args, w, lib, dev, up):
    """Every rank's shard copied out of the full [V, D] table on the device
    (vpe_load_shard); value = algorithmic bytes (read R*D*s + write R*D*s per
    rank) / step time."""
    import numpy as np
    import torch

    import vocab_sharded_embedding_amd as vpe
    import workloads as wl

    t0 = time.time()
    full_h = wl.full_table(w)
    gen_s = time.time() - t0
    full_d = up(full_h)
    tdt = full_d.dtype
    step_bytes = 2 * len(w.ranks) * w.shard_rows * w.dim * w.elem_bytes
    copies = args.copies or max(1, -(-CACHE_DEFEAT_BYTES // (full_h.nbytes + step_bytes // 2)))
    fulls = [full_d] + [full_d.clone() for _ in range(copies - 1)]
    outs = [{r: torch.empty((w.shard_rows, w.dim), dtype=tdt, device=dev) for r in w.ranks}
            for _ in range(copies)]
    dcode = vpe.VPE_BF16 if w.dtype == "bf16" else vpe.VPE_F32
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    calls = [[(lib.vpe_load_shard, (fulls[c].data_ptr(), w.vocab, w.dim, dcode, w.tp, r,
                                    outs[c][r].data_ptr(), sh)) for r in w.ranks]
             for c in range(copies)]

    def run_step(k, evs=None):
        for j, (fn, a) in enumerate(calls[k % copies]):
            if evs is not None:
                evs[j][0].record(stream)
            rc = fn(*a)
            if evs is not None:
                evs[j][1].record(stream)
            if rc != 0:
                raise RuntimeError(f"load_shard failed: {vpe.status_name(rc)}")

    with torch.cuda.stream(stream):
        for k in range(args.warmup):
            run_step(k)
        evs = [[(TimingEvent(), TimingEvent())
                for _ in w.ranks] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for k in range(args.steps):
            run_step(k, evs[k])
        torch.cuda.synchronize()
        t_total = time.perf_counter() - t_start
    us = [float(np.mean([evs[k][j][0].elapsed_time(evs[k][j][1]) for k in range(args.steps)])) * 1e3
          for j in range(len(w.ranks))]
    per_launch = step_bytes / len(w.ranks)
    ms_per_step = t_total * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    ach = per_launch / (float(np.mean(us)) * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        for r in w.ranks:
            oracle.load_shard(full_h, w.tp, r)
        dt = time.perf_counter() - t0
        cpu = {"value": round(step_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "sample": f"every rank's shard once; {dt:.2f} s wall"}
    line = {
        "metric": "shard load GB/s (read + write of every rank's rows)", "value": round(value, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name + "/load_shard", "vocab": w.vocab, "dim": w.dim, "tp": w.tp,
                   "ranks": list(w.ranks), "rotating_copies": copies,
                   "step_algorithmic_bytes": step_bytes},
        "roofline": {"kernel": "load_shard", "bound": "hbm", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": per_launch,
                     "avg_launch_us": round(float(np.mean(us)), 3)},
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(dev),
        "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, ids_h, hidden_h, cu_h, step_bytes, threads, shards=None):
    """The oracle, as it stands, on the same step (bounded: one pass)."""
    import numpy as np

    import oracle
    import workloads as wl

    nt = threads or max(1, min(16, len(os.sched_getaffinity(0))))
    if shards is None:
        shards = {r: wl.shard_table(w, r) for r in w.ranks}
    # LM head: bounded sample of rows when the full product would take too long
    M = w.seqs if w.seqs else hidden_h.shape[0]
    flops_full = 2.0 * M * w.shard_rows * w.dim * len(w.ranks)
    budget_flops = 6e10  # about 30 s of single-thread fp64 loops
    m_s = max(1, min(M, int(M * budget_flops / flops_full)))

    def one_pass():
        t0 = time.perf_counter()
        parts = [oracle.embed(ids_h, shards[r], w.rank_start(r), nthreads=nt) for r in w.ranks]
        if len(parts) > 1:
            oracle.sum_partials(parts)
        x = oracle.last_token_select(hidden_h, cu_h) if w.seqs else hidden_h
        for r in w.ranks:
            oracle.lmhead_f64(x[:m_s], shards[r], nthreads=nt)
        return time.perf_counter() - t0

    # median of three passes when one pass is short, else one pass
    times = [one_pass()]
    if times[0] < 5.0:
        times += [one_pass(), one_pass()]
    t = float(np.median(times))
    frac = m_s / M
    # scale the LM-head part of the step's bytes to the sample taken
    s = w.elem_bytes
    lm_full = sum(M * w.dim * s + w.shard_rows * w.dim * s + M * w.shard_rows * s
                  for _ in w.ranks)
    sample_bytes = step_bytes - lm_full + sum(m_s * w.dim * s + w.shard_rows * w.dim * s +
                                              m_s * w.shard_rows * s for _ in w.ranks)
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(sample_bytes / t / 1e9, 3), "unit": "GB/s", "cores": nt,
            "cpu_model": cpu_model, "passes": len(times),
            "kind": "oracle",
            "sample": f"whole step except LM head on {m_s} of {M} rows; {t:.2f} s wall on "
                      f"{nt} threads (about {t * nt:.0f} core-seconds), median of "
                      f"{len(times)} passes",
            "seconds": round(t, 3)}


if __name__ == "__main__":
    main()
