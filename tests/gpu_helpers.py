"""Shared helpers for the GPU parity tests.

GPU-side inputs are laid out with libcva's own metadata (local rows of the
rank, rank-major gathered K/V); the oracle splits the same full tensors with its
own enumeration.  Tolerances: MindSpeed RFC section 3.5.1 (fp16 atol = rtol =
5e-3, bf16 atol = rtol = 2.5e-2); fp32 uses 1e-4 (no page value; the kernel
accumulates in fp32 so its error is far below that).

Every comparison also records its headroom, max(|err| / (atol + rtol*|ref|)),
one JSON line per (test, output) in ``$CVA_HEADROOM_FILE`` (default
``test_output/parity_headroom.jsonl`` under the repository root): 1.0 would be
the tolerance itself.
"""
import functools
import json
import os
from concurrent.futures import ThreadPoolExecutor, as_completed

import numpy as np

import context_varlen_attention_amd as cva
import oracle
import synth

TOL = {"bf16": 2.5e-2, "fp16": 5e-3, "fp32": 1e-4}
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADROOM_FILE = os.environ.get("CVA_HEADROOM_FILE",
                               os.path.join(ROOT, "test_output", "parity_headroom.jsonl"))
ORACLE_THREADS = 4  # oracle heads computed side by side (numpy releases the GIL)


def torch_dtype(dt):
    import torch
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dt]


def plan_for(w):
    bb = None if w.branch_bounds is None else np.asarray(w.branch_bounds)
    return cva.Plan(w.cu_seqlens, w.cp_size, w.rank, w.hq, w.hkv, w.d_qk, w.d_v, w.dtype,
                    mask=w.mask, sink=w.sink, window=w.window, branch_bounds=bb, block=w.block)


@functools.lru_cache(maxsize=8)
def workload_tensors(name, mask=None, dtype=None, with_dout=True):
    """(workload, [q, k, v(, do)]) of a named workload, kept for every later test
    that asks for the same one (the full-size tensors take up to a minute or two
    to draw; the suite's eight variants hold about 20 GB of host memory)."""
    w = synth.make_workload(name, mask=mask, dtype=dtype)
    return w, synth.make_tensors(w, with_dout=with_dout)


def device_inputs(w, q, k, v, do=None, device="cuda"):
    """Local q / dO rows and rank-major K/V on the GPU, laid out by libcva's metadata."""
    import torch
    dt = torch_dtype(w.dtype)
    loc = cva.local_token_ids(w.cu_seqlens, w.cp_size, w.rank)
    rm = cva.rank_major_token_ids(w.cu_seqlens, w.cp_size)
    out = [torch.from_numpy(np.ascontiguousarray(q[loc])).to(device=device, dtype=dt),
           torch.from_numpy(np.ascontiguousarray(k[rm])).to(device=device, dtype=dt),
           torch.from_numpy(np.ascontiguousarray(v[rm])).to(device=device, dtype=dt)]
    if do is not None:
        out.append(torch.from_numpy(np.ascontiguousarray(do[loc])).to(device=device, dtype=dt))
    return out


def _row_chunks(w, rows, chunk):
    T_loc = w.total_tokens // w.cp_size
    rows = np.arange(T_loc) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    return [rows[i: i + chunk] for i in range(0, len(rows), chunk)]


def _run_tasks(label, tasks, fn, merge):
    """fn(task) on ORACLE_THREADS worker threads, merging each result as it
    lands (so at most a few are held at once) and printing one line per task."""
    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        futs = {ex.submit(fn, t): t for t in tasks}
        for n, f in enumerate(as_completed(futs), 1):
            merge(futs[f], f.result())
            print(f"[oracle] {label}: {n}/{len(tasks)} parts done", flush=True)


def fwd_ref_heads(w, q, k, v, heads, rows=None, scale=None, chunk=4096):
    """oracle.fwd_ref for the listed query heads, in parts of one head and up to
    ``chunk`` local rows computed on worker threads (rows are independent)."""
    T_loc = w.total_tokens // w.cp_size
    o = np.full((T_loc, w.hq, w.d_v), np.nan)
    lse = np.full((w.hq, T_loc), np.nan)
    tasks = [(h, r) for h in heads for r in _row_chunks(w, rows, chunk)]

    def merge(t, res):
        h, r = t
        o[r, h] = res[0][r, h]
        lse[h, r] = res[1][h, r]

    _run_tasks(f"fwd {w.name} heads {list(heads)}", tasks,
               lambda t: oracle.fwd_ref(w, q, k, v, scale=scale, rows=t[1], heads=[t[0]]), merge)
    return o, lse


def bwd_ref_heads(w, q, k, v, do_loc, heads, scale=None, block=512, chunk=4096):
    """oracle.bwd_ref for the listed query heads, in parts of one head and up to
    ``chunk`` local rows on worker threads; dK/dV are the sums of the parts'
    shares (dK and dV are sums over query rows and heads of a group)."""
    T, T_loc = w.total_tokens, w.total_tokens // w.cp_size
    dq = np.zeros((T_loc, w.hq, w.d_qk))
    dk = np.zeros((T, w.hkv, w.d_qk))
    dv = np.zeros((T, w.hkv, w.d_v))
    tasks = [(h, r) for h in heads for r in _row_chunks(w, None, chunk)]

    def merge(t, res):
        h, r = t
        dq[r, h] = res[0][r, h]
        dk[:, h // (w.hq // w.hkv)] += res[1][:, h // (w.hq // w.hkv)]
        dv[:, h // (w.hq // w.hkv)] += res[2][:, h // (w.hq // w.hkv)]

    _run_tasks(f"bwd {w.name} heads {list(heads)}", tasks,
               lambda t: oracle.bwd_ref(w, q, k, v, do_loc, scale=scale, heads=[t[0]], rows=t[1],
                                        block=block), merge)
    return dq, dk, dv


def _record(what, dtype, tol, max_err, ratio, n):
    rec = {"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "output": what,
           "dtype": dtype, "tol": tol, "max_abs_err": max_err, "headroom_ratio": ratio,
           "elements": int(n)}
    try:
        os.makedirs(os.path.dirname(HEADROOM_FILE), exist_ok=True)
        with open(HEADROOM_FILE, "a") as f:
            f.write(json.dumps(rec) + "\n")
    except OSError:  # a read-only checkout: the assertion below still decides
        pass


def assert_close(got, ref, dtype, what, atol_scale=1.0):
    """Element-wise |got - ref| <= a * tol + tol * |ref| (numpy.allclose
    semantics; a = ``atol_scale``, 1 unless a caller's arithmetic multiplies
    the terms that are rounded by a known factor).

    Returns (max |err|, max |err| / bound) and records both."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    tol = TOL[dtype]
    finite = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), finite), f"{what}: non-finite pattern differs"
    err = np.abs(got[finite] - ref[finite])
    bound = atol_scale * tol + tol * np.abs(ref[finite])
    ratio = float((err / bound).max()) if err.size else 0.0
    max_err = float(err.max()) if err.size else 0.0
    _record(what, dtype, tol, max_err, ratio, err.size)
    bad = err > bound
    if bad.any():
        idx = np.argmax(err - bound)
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{err.size} elements outside tol {tol}; worst err "
            f"{err[idx]:.3e} (ref {ref[finite][idx]:.4f}); max err {max_err:.3e}; "
            f"headroom ratio {ratio:.3f}")
    return max_err, ratio
