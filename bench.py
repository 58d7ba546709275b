#!/usr/bin/env python3
"""Benchmark of one context-parallel rank's share of packed varlen attention
on one MI355X, through libcva's C ABI.

A step is one batch through the whole hot path: the host plan (rank metadata
and block-mask tile schedules), its upload, the forward and the backward.
Plans are built by a look-ahead host thread and uploaded on a side stream, so
host planning overlaps the GPU work of the previous step (the look-ahead
planning of the DCP paper's data loader); when planning is slower than the
GPU the step waits for it and the measured time includes that wait.

Prints ONE JSON line.  ``value`` is useful attention TFLOP/s over the step:
only unmasked (query, key) pairs count, forward 2*N*Hq*(Dqk+Dv), backward
2*N*Hq*(3*Dqk+2*Dv) (scores and dP counted once).  A profile pass after the
warm-up records hipEvents around every kernel (the ``kernels`` breakdown) and
picks the kernel that dominates the step; the timed steps then carry events
around that kernel only, so ``roofline`` (its algorithmic rate against the
MI355X peak) is measured on its own stream during the timed steps while the
other kernels run without instrumentation.  ``cpu_baseline`` times the fp64
oracle on a bounded sample of the same workload on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long128k]
                       [--mask M] [--dtype D] [--no-split] [--dropout P]

With ``--dropout P`` the step runs cva_fwd_dropout / cva_bwd_dropout (a fresh
seed per step); ``value`` still counts the same useful MFMA flops.

The forward is cva_fwd_split whenever the plan cuts a Q tile's K/V range (a
tile walking more than 4/3 of the average work per compute unit), else
cva_fwd; ``--no-split`` forces cva_fwd.

The default workload is the largest single-GPU one: one 131072-token sequence,
CP rank 3 of 8, 32/8 heads, D=128, bf16, causal, forward + backward.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import queue
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp32": 157.3}  # dense; 256 CU x 2.4 GHz x 4096 (16-bit)
PEAK_HBM_GBS = 8000.0
METRIC = "useful attention TFLOP/s (bf16 fwd/bwd) and % of MI355X MFMA peak"

DESCRIPTIONS = {
    "gqa16k": "packed varlen GQA, 16384 tokens (log-uniform lengths 128..8192), CP rank 1 of 4, "
              "32/8 heads, D=128, causal + EOD reset",
    "long128k": "single 131072-token sequence, CP rank 3 of 8, 32/8 heads, D=128, causal",
    "sparse8": "8 sequences (log-normal lengths, median 8192), no CP split, 16/16 heads, D=128",
    "mla32k": "32768 packed tokens (uniform lengths 512..16384), CP rank 2 of 4, 16/16 heads, "
              "Dqk=192, Dv=128, causal",
    "tiny": "cu_seqlens [0,64,192,256], CP rank 0 of 2, 4/4 heads, D=64",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_plan(cva, w):
    return cva.Plan(w.cu_seqlens, w.cp_size, w.rank, w.hq, w.hkv, w.d_qk, w.d_v, w.dtype,
                    mask=w.mask, sink=w.sink, window=w.window, branch_bounds=w.branch_bounds, block=w.block)


class LookAheadPlanner:
    """Builds and uploads plans on a host thread, `depth` batches ahead."""

    def __init__(self, cva, w, n, depth=2):
        import torch
        self.cva, self.w, self.n = cva, w, n
        self.q = queue.Queue(maxsize=depth)
        self.stream = torch.cuda.Stream()
        self.build_s = []
        self.err = None
        self.t = threading.Thread(target=self._run, daemon=True)
        self.t.start()

    def _run(self):
        import torch
        try:
            with torch.cuda.stream(self.stream):
                for _ in range(self.n):
                    t0 = time.perf_counter()
                    p = make_plan(self.cva, self.w)
                    self.build_s.append(time.perf_counter() - t0)
                    p.upload(stream=self.stream)  # async; launches on the main stream wait for it
                    self.q.put(p)
        except BaseException as e:  # surfaced to the consumer
            self.err = e
            self.q.put(None)

    def get(self):
        try:
            p = self.q.get(timeout=120)
        except queue.Empty:
            raise RuntimeError("no plan from the planner thread within 120 s (more plans asked for "
                               "than were scheduled?)") from None
        if p is None:
            raise RuntimeError(f"planner thread failed: {self.err!r}")
        return p


def kernel_flops(w, pairs):
    """Algorithmic flops per launch: the useful backward 2*N*Hq*(3*Dqk+2*Dv)
    split over the two backward kernels without counting anything twice.  The
    dK/dV kernel owns the score recompute (Dqk), dP (Dv), dV (Dv) and dK (Dqk);
    the dQ kernel's own product is dQ (Dqk) -- its second score recompute and dP
    are reported as issued work (kernel_flops_issued), not as useful work."""
    hq, dqk, dv = w.hq, w.d_qk, w.d_v
    return {
        "fwd": 2 * pairs * hq * (dqk + dv),
        "bwd_dkdv": 2 * pairs * hq * (2 * dqk + 2 * dv),
        "bwd_dq": 2 * pairs * hq * dqk,
    }


def kernel_flops_issued(w, pairs):
    """Flops a kernel executes on visible pairs, recompute included (where it
    differs from the algorithmic count)."""
    hq, dqk, dv = w.hq, w.d_qk, w.d_v
    return {"bwd_dq": 2 * pairs * hq * (2 * dqk + dv)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def device_info(torch, dev):
    """Name, architecture, compute units and peak engine clock of the GPU, and
    the dense 16-bit MFMA peak they give (4096 flop per clock per CU)."""
    import re
    import subprocess
    props = torch.cuda.get_device_properties(dev)
    info = {"name": props.name, "arch": props.gcnArchName.split(":")[0],
            "compute_units": int(props.multi_processor_count), "max_clock_mhz": None}
    try:
        out = subprocess.run(["rocminfo"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                             text=True, timeout=60).stdout
        for agent in out.split("Agent ")[1:]:
            if re.search(r"Name:\s+" + re.escape(info["arch"]) + r"\b", agent):
                m = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
                c = re.search(r"Compute Unit:\s+(\d+)", agent)
                if m:
                    info["max_clock_mhz"] = int(m.group(1))
                if c:
                    info["compute_units"] = int(c.group(1))
                n = re.search(r"Marketing Name:[ \t]+(\S[^\n]*)", agent)
                if n and not info["name"]:  # torch may report an empty name
                    info["name"] = n.group(1).strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if info["max_clock_mhz"]:
        info["dense_16bit_peak_tflops"] = (info["compute_units"] * info["max_clock_mhz"] * 1e6
                                           * 4096 / 1e12)
    return info


def kernel_bytes(w, split_plan=None):
    """HBM-bound kernels: algorithmic bytes per launch.  The split forward's merge
    reads, per (row, head) of a cut Q tile, every piece's fp32 partial row and
    LSE, and writes the row of O (input dtype) and its LSE."""
    if split_plan is None:
        return {}
    comb = split_plan.tables()["split_combine"]
    if len(comb) == 0:
        return {}
    esz = {"bf16": 2, "fp16": 2, "fp32": 4}[w.dtype]
    rows, npiece = comb[:, 2].astype(np.int64), comb[:, 4].astype(np.int64)
    per_row = npiece * (w.d_v + 1) * 4 + w.d_v * esz + 4
    return {"fwd_merge": int((rows * w.hq * per_row).sum())}


KERNEL_SOURCES = {
    "fwd": ["kernels/fwd.hip"],
    "bwd_dkdv": ["kernels/bwd.hip"], "bwd_dq": ["kernels/bwd.hip"],
    "fwd_merge": ["kernels/fwd.hip"],
}
COMMON_SOURCES = ["kernels/common.hpp", "kernels/launch.hpp", "host/plan.hpp", "host/schedule.cpp"]


def code_text(src):
    """C++/HIP source with comments removed and runs of white space collapsed
    (string literals are kept as written)."""
    import re
    token = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'', re.S)
    src = token.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), src)
    return " ".join(src.split())


def kernel_source_hash(kernel):
    """sha256 over the code (comments and white space left out) of the sources
    a kernel's memory traffic depends on."""
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(ROOT, "context_varlen_attention_amd", "csrc")
    for rel in KERNEL_SOURCES.get(kernel, []) + COMMON_SOURCES:
        with open(os.path.join(base, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_key(w):
    """How counter summaries name a workload: name/mask/dtype."""
    return f"{w.name}/{w.mask}/{w.dtype}"


def measured_traffic(kernel, workload):
    """HBM bytes per launch from a committed counter summary under profiles/.

    Summaries carry lines ``<!-- traffic kernel=K workload=W sha=S bytes=B -->``
    (W as ``traffic_key`` forms it; FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by the factor a plain
    copy of known size gives).  Returns None when no summary matches the
    kernel's current sources.
    """
    import glob
    import re
    want = kernel_source_hash(kernel)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for m in re.finditer(r"<!-- traffic (.*?) -->", f.read()):
                kv = dict(x.split("=", 1) for x in m.group(1).split())
                if kv.get("kernel") == kernel and kv.get("workload") == workload \
                        and kv.get("sha") == want:
                    return float(kv["bytes"])
    return None


def cpu_baseline(w, budget_s=12.0, block_rows=256):
    """The fp64 oracle, forward then backward, on a bounded sample of the same
    batch: blocks of ``block_rows`` local rows of one query head at a time
    (the blocks walk through the rank's rows, the heads rotate), until
    ``budget_s`` of CPU time is spent.  Useful flops are the sampled rows'
    visible pairs times the same per-pair counts as the GPU's.

    The oracle reads K/V over whole sub-sequences and Q/dO at the sampled rows,
    so only K and V are drawn in full; Q and dO are drawn at the sampled rows
    (the values do not change the work)."""
    import oracle
    from oracle.masks import mask_rows_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the visible core count
        threads = os.cpu_count()
    rng = np.random.default_rng([synth.CONFIG_IDS.get(w.name, 0), 7])
    T = w.total_tokens
    cu = np.asarray(w.cu_seqlens, dtype=np.int64)
    loc = np.asarray(oracle.rank_local_positions(cu, w.cp_size, w.rank), dtype=np.int64)
    T_loc = len(loc)
    k = rng.standard_normal((T, w.hkv, w.d_qk), dtype=np.float32)
    v = rng.standard_normal((T, w.hkv, w.d_v), dtype=np.float32)
    q = np.zeros((T, w.hq, w.d_qk), dtype=np.float32)      # filled at the sampled rows
    do_loc = np.zeros((T_loc, w.hq, w.d_v), dtype=np.float32)
    n_blocks = max(1, T_loc // block_rows)
    order = np.random.default_rng(5).permutation(n_blocks)
    done_pairs, elapsed, n_rows, heads_used = 0, 0.0, 0, set()
    for it, b in enumerate(order):
        rows = np.arange(b * block_rows, min(T_loc, (b + 1) * block_rows))
        h = int(it % w.hq)
        q[loc[rows], h] = rng.standard_normal((len(rows), w.d_qk), dtype=np.float32)
        do_loc[rows, h] = rng.standard_normal((len(rows), w.d_v), dtype=np.float32)
        t0 = time.perf_counter()
        oracle.fwd_ref(w, q, k, v, rows=rows, heads=[h])
        oracle.bwd_ref(w, q, k, v, do_loc, heads=[h], rows=rows)
        elapsed += time.perf_counter() - t0
        toks = loc[rows]
        seq = np.searchsorted(cu, toks, side="right") - 1
        for i in np.unique(seq):
            L = int(cu[i + 1] - cu[i])
            pos = toks[seq == i] - cu[i]
            bb = None if w.branch_bounds is None else w.branch_bounds[i]
            done_pairs += int(mask_rows_ref(w.mask, L, pos, w.sink, w.window, bb,
                                            getattr(w, "block", 0)).sum())
        n_rows += len(rows)
        heads_used.add(h)
        if elapsed >= budget_s:
            break
    flops = 2 * done_pairs * ((w.d_qk + w.d_v) + (3 * w.d_qk + 2 * w.d_v))
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle fwd+bwd on {n_rows} of {T_loc} local rows x {len(heads_used)} "
                  f"of {w.hq} query heads (blocks of {block_rows} rows, one head each) of the "
                  f"same batch; {elapsed:.1f} s; useful flops of the sampled rows counted as on "
                  f"the GPU",
        "cpu_model": cpu_model(),
        "seconds": elapsed,
    }


COPY_BYTES = 1 << 30


def calibrate_copy(torch, dev, reps=3):
    """A plain element-wise copy of COPY_BYTES bytes (fp32 x * 1 -> y), `reps` times.

    Profiled with the same HBM byte counters as the attention kernels, it gives
    the factor that turns those counters into bytes.
    """
    n = COPY_BYTES // 4
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy": {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                                         "launches": reps}}), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long128k", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--mask", default=None, choices=[None, "causal", "lambda", "shared_prefix", "blockwise"])
    ap.add_argument("--dtype", default=None, choices=[None, "bf16", "fp16", "fp32"])
    ap.add_argument("--fwd-only", action="store_true", help="time forward only (profiling aid)")
    ap.add_argument("--no-split", action="store_true",
                    help="always cva_fwd (by default the forward is cva_fwd_split whenever the "
                         "plan cuts a Q tile's K/V range, i.e. needs a forward workspace)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--dropout", type=float, default=None,
                    help="attention dropout probability (cva_fwd_dropout / cva_bwd_dropout); each step "
                         "draws its mask from seed + step index")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share on a single MI355X; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: cva has no multi-GPU path",
              file=sys.stderr)
        return 2

    import torch
    import context_varlen_attention_amd as cva
    cva.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    dev = torch.device("cuda", 0)
    if args.calibrate_copy:
        return calibrate_copy(torch, dev)
    w = synth.make_workload(args.workload, mask=args.mask, dtype=args.dtype)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    T, T_loc = w.total_tokens, w.total_tokens // w.cp_size
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 * synth.CONFIG_IDS[w.name] + args.seed)
    q = torch.randn((T_loc, w.hq, w.d_qk), generator=gen, device=dev, dtype=torch.float32).to(tdt)
    k = torch.randn((T, w.hkv, w.d_qk), generator=gen, device=dev, dtype=torch.float32).to(tdt)
    v = torch.randn((T, w.hkv, w.d_v), generator=gen, device=dev, dtype=torch.float32).to(tdt)
    do = torch.randn((T_loc, w.hq, w.d_v), generator=gen, device=dev, dtype=torch.float32).to(tdt)
    o = torch.empty((T_loc, w.hq, w.d_v), device=dev, dtype=tdt)
    lse = torch.empty((w.hq, T_loc), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    ref_plan = make_plan(cva, w)
    pairs = ref_plan.visible_pairs()
    ws = torch.empty(max(int(cva.load_library().cva_bwd_workspace_bytes(ref_plan.handle)), 4),
                     dtype=torch.uint8, device=dev)
    fwd_ws = None
    if not args.no_split and ref_plan.fwd_workspace_bytes() > 0:
        fwd_ws = torch.empty(ref_plan.fwd_workspace_bytes(), dtype=torch.uint8, device=dev)
    fwd_only = args.fwd_only or w.dtype == "fp32"
    log(f"workload {w.name}: T={T} T_loc={T_loc} seqs={len(w.lengths)} pairs/head={pairs} "
        f"fwd_only={fwd_only}")

    n_step = [0]

    def step(plan):
        if args.dropout is None:
            cva.fwd(plan, q, k, v, out=o, lse=lse, workspace=fwd_ws)
            if not fwd_only:
                cva.bwd(plan, q, k, v, o, lse, do, dq=dq, dk_rm=dk, dv_rm=dv, workspace=ws)
            return
        seed = args.seed + n_step[0]
        n_step[0] += 1
        cva.fwd(plan, q, k, v, out=o, lse=lse, workspace=fwd_ws, dropout_p=args.dropout, seed=seed)
        if not fwd_only:
            cva.bwd(plan, q, k, v, o, lse, do, dq=dq, dk_rm=dk, dv_rm=dv, workspace=ws,
                    dropout_p=args.dropout, seed=seed)

    n_prof = max(1, min(args.steps, 10))  # profile-pass steps (see below)
    planner = LookAheadPlanner(cva, w, args.warmup + n_prof + args.steps)
    keep = []  # plans stay alive until the final synchronize (their device tables are in use)
    for _ in range(args.warmup):
        p = planner.get()
        keep.append(p)
        step(p)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # Profile pass (not timed): events around every kernel, for the per-kernel
    # breakdown and to find the kernel that dominates the step.
    cva.timing_select(None)
    cva.timing_enable(True)
    for _ in range(n_prof):
        p = planner.get()
        keep.append(p)
        step(p)
    torch.cuda.synchronize()
    prof_times = cva.timing_read()
    dom = max((n for n in prof_times if prof_times[n][0] > 0), key=lambda n: prof_times[n][1])

    # Timed region: events around the dominant kernel only (its duration for the
    # roofline is measured here; events around every launch would slow the step).
    cva.timing_select([dom])
    cva.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        p = planner.get()
        keep.append(p)
        step(p)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    times = cva.timing_read()
    cva.timing_enable(False)
    cva.timing_select(None)
    log(f"timed {args.steps} steps in {t1 - t0:.3f} s")

    ms_step = (t1 - t0) * 1e3 / args.steps
    fl_fwd = 2 * pairs * w.hq * (w.d_qk + w.d_v)
    fl_bwd = 0 if fwd_only else 2 * pairs * w.hq * (3 * w.d_qk + 2 * w.d_v)
    value = (fl_fwd + fl_bwd) / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    kfl = kernel_flops(w, pairs)
    kfl_issued = kernel_flops_issued(w, pairs)
    kby = kernel_bytes(w, ref_plan if fwd_ws is not None else None)
    kernels = {}
    for name, (n, tot) in prof_times.items():
        if n == 0:
            continue
        steps_seen = n_prof
        if name == dom and times[name][0] > 0:  # the timed region's own measurement
            n, tot = times[name]
            steps_seen = args.steps
        avg = tot / n
        rec = {"launches_per_step": n / steps_seen, "avg_ms": avg, "ms_per_step": tot / steps_seen,
               "measured": "timed region" if steps_seen == args.steps and name == dom else "profile pass"}
        if name in kfl:
            rec.update(bound="mfma", achieved=kfl[name] / (avg * 1e-3) / 1e12, unit="TFLOP/s",
                       peak=peak, flops_per_launch=kfl[name])
            if name in kfl_issued:
                rec["issued_tflops"] = kfl_issued[name] / (avg * 1e-3) / 1e12
        elif name in kby:
            rec.update(bound="hbm", achieved=kby[name] / (avg * 1e-3) / 1e9, unit="GB/s",
                       peak=PEAK_HBM_GBS)
        if "achieved" in rec:
            rec["frac"] = rec["achieved"] / rec["peak"]
        rec["source_sha"] = kernel_source_hash(name)
        kernels[name] = rec
    d = kernels[dom]
    roofline = {"kernel": dom, "bound": d.get("bound"), "achieved": d.get("achieved"),
                "peak": d.get("peak"), "unit": d.get("unit"), "frac": d.get("frac"),
                # (the committed counters are of the kernels without dropout)
                "traffic": None if args.dropout is not None else measured_traffic(dom, traffic_key(w)),
                "per_launch": (f"{kfl[dom]:.4e} flop" if dom in kfl else f"{kby.get(dom, 0)} B")}
    fwd_ms = sum(kernels[n]["ms_per_step"] for n in kernels if n.startswith("fwd")) or None
    bwd_ms = sum(kernels[n]["ms_per_step"] for n in kernels if n.startswith("bwd"))
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "description": DESCRIPTIONS[w.name], "tokens": T,
                   "sub_sequences": int(len(w.lengths)), "cp_size": w.cp_size, "rank": w.rank,
                   "hq": w.hq, "hkv": w.hkv, "d_qk": w.d_qk, "d_v": w.d_v, "mask": w.mask,
                   "step": "plan (look-ahead) + upload + fwd" + ("" if fwd_only else " + bwd"),
                   "fwd_split": fwd_ws is not None, "dropout": args.dropout},
        "pct_of_peak": 100.0 * value / peak,
        "useful_tflop_per_step": (fl_fwd + fl_bwd) / 1e12,
        "fwd_tflops": fl_fwd / (fwd_ms * 1e-3) / 1e12 if fwd_ms else None,
        "bwd_tflops": fl_bwd / (bwd_ms * 1e-3) / 1e12 if bwd_ms and fl_bwd else None,
        "plan_ms_host": 1e3 * float(np.mean(planner.build_s)) if planner.build_s else None,
        "roofline": roofline,
        "kernels": kernels,
        "device": device_info(torch, dev),
    }
    del keep
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a bounded sample (cpu_baseline)")
        cb = cpu_baseline(w)
        out["cpu_baseline"] = {kk: cb[kk] for kk in ("value", "unit", "cores", "kind", "sample",
                                                     "cpu_model")}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
