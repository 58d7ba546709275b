"""Attention dropout on the GPU against the fp64 oracle (every output element).

The keep mask is a function of (seed, sequence, head, in-sequence query and key
positions) -- Philox4x32-10 on both sides, each written from the generator's
published definition -- so the kernels' O, LSE, dQ and rank-major dK/dV must
match ``oracle.fwd_ref`` / ``oracle.bwd_ref`` with ``dropout=(p, seed)`` to the
same tolerances as without dropout.  Covered: every mask, GQA and MHA, Q/K head
dims 64, 128 and 192 (the per-item forward, which dropout always uses), split
K/V ranges, several CP ranks, fp32 forward, p = 0 against the plain path, a
seeded random sweep, and sampled rows of the full-size workloads (positions up
to 131072, the generator's counters far from zero) in the benchmark's launch
configuration.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_close, device_inputs, plan_for, workload_tensors
from tests.random_cases import random_case
from tests.test_bwd_gpu import CASES

pytestmark = pytest.mark.gpu


def _run(w, q, k, v, do, p, seed, split=False, scale=None, bwd=True, atol_scale=1.0):
    import torch
    import context_varlen_attention_amd as cva
    print(f"[drop] {w.name} {w.dtype} mask={w.mask} R={w.cp_size} r={w.rank} T={w.total_tokens} "
          f"H={w.hq}/{w.hkv} D={w.d_qk}/{w.d_v} p={p} seed={seed} split={split}", flush=True)
    plan = plan_for(w)
    if split:
        assert plan.fwd_workspace_bytes() > 0, "the case was meant to split K/V ranges"
    tq, tk, tv, tdo = device_inputs(w, q, k, v, do)
    o, lse = cva.fwd(plan, tq, tk, tv, softmax_scale=scale, workspace=True if split else None,
                     dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd_ref(w, q, k, v, scale=scale, dropout=(p, seed))
    assert_close(o.float().cpu().numpy(), o_ref, w.dtype, "O", atol_scale)
    assert_close(lse.cpu().numpy(), lse_ref, w.dtype, "LSE")  # the undropped normaliser
    if not bwd:
        return
    dq, dk, dv = cva.bwd(plan, tq, tk, tv, o, lse, tdo, softmax_scale=scale, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    loc = cva.local_token_ids(w.cu_seqlens, w.cp_size, w.rank)
    rdq, rdk, rdv = oracle.bwd_ref(w, q, k, v, do[loc], scale=scale, dropout=(p, seed))
    e1, r1 = assert_close(dq.float().cpu().numpy(), rdq, w.dtype, "dQ", atol_scale)
    e2, r2 = assert_close(dk.float().cpu().numpy(), rdk, w.dtype, "dK", atol_scale)
    e3, r3 = assert_close(dv.float().cpu().numpy(), rdv, w.dtype, "dV", atol_scale)
    print(f"[drop]   headroom ratio dQ {r1:.3f} dK {r2:.3f} dV {r3:.3f}", flush=True)


def _case(ci, dtype):
    lens, R, r, hq, hkv, dqk, dv, mask, ex = CASES[ci]
    return synth.custom_workload(lens, R, r, hq, hkv, dqk, dv, dtype, mask=mask,
                                 sink=ex.get("sink", 0), window=ex.get("window", 0),
                                 branch_bounds=ex.get("bounds"), name=f"dsmall{ci}",
                                 block=ex.get("block", 0))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_small_cases(ci, dtype):
    w = _case(ci, dtype)
    q, k, v, do = synth.random_tensors(w, 500 + ci)
    _run(w, q, k, v, do, p=[0.1, 0.25, 0.4][ci % 3], seed=1000 + 7 * ci)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_split_forward(dtype, monkeypatch):
    """Split K/V ranges: every piece applies the mask of its own keys and the
    merge adds the scaled partial outputs."""
    monkeypatch.setenv("CVA_FWD_SPLIT_CAP", "3")
    w = _case(4, dtype)  # [512, 96, 1536], R=2: Q tiles longer than 3 K/V tiles
    q, k, v, do = synth.random_tensors(w, 600)
    _run(w, q, k, v, do, p=0.2, seed=(1 << 40) + 3, split=True, bwd=False)


def test_fp32_forward():
    w = synth.make_workload("tiny")
    q, k, v, do = synth.random_tensors(w, 601)
    _run(w, q, k, v, do, p=0.3, seed=99, bwd=False)


def test_custom_scale():
    w = _case(1, "bf16")
    q, k, v, do = synth.random_tensors(w, 602)
    _run(w, q, k, v, do, p=0.15, seed=5, scale=0.2)


def test_p0_equals_plain_path():
    """p = 0 drops nothing: the dropout entry points give the plain results bit for bit."""
    import torch
    import context_varlen_attention_amd as cva
    w = _case(2, "bf16")
    q, k, v, do = synth.random_tensors(w, 603)
    plan = plan_for(w)
    tq, tk, tv, tdo = device_inputs(w, q, k, v, do)
    o0, l0 = cva.fwd(plan, tq, tk, tv)
    o1, l1 = cva.fwd(plan, tq, tk, tv, dropout_p=0.0, seed=12)
    g0 = cva.bwd(plan, tq, tk, tv, o0, l0, tdo)
    g1 = cva.bwd(plan, tq, tk, tv, o0, l0, tdo, dropout_p=0.0, seed=12)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("ci", [0, 2, 5, 7, 10, 11])
def test_extreme_rates(ci, dtype):
    """The ends of the probability range.

    p = 0.001 rounds to threshold 0 and drops nothing: the plain path's bits.
    p = 0.003 is threshold 1, the smallest realised rate (1/256), through the
    dropout kernels at the standard tolerance.  p = 0.99 (threshold 253, keep
    scale 256/3) and p = 0.999 (clamped to threshold 255, keep scale 256): the
    kernels round P, dS and O to 16 bits as always, but every kept probability
    and every kept dP is multiplied by the keep scale, so the absolute rounding
    error of O, dQ, dK and dV grows by that factor; the absolute part of the
    tolerance is scaled by it, the relative part is unchanged."""
    import torch
    import context_varlen_attention_amd as cva
    w = _case(ci, dtype)
    q, k, v, do = synth.random_tensors(w, 800 + ci)
    plan = plan_for(w)
    tq, tk, tv, tdo = device_inputs(w, q, k, v, do)
    o0, l0 = cva.fwd(plan, tq, tk, tv)
    o1, l1 = cva.fwd(plan, tq, tk, tv, dropout_p=0.001, seed=3)
    g0 = cva.bwd(plan, tq, tk, tv, o0, l0, tdo)
    g1 = cva.bwd(plan, tq, tk, tv, o0, l0, tdo, dropout_p=0.001, seed=3)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)
    _run(w, q, k, v, do, p=0.003, seed=21 + ci)
    for p in (0.99, 0.999):
        _run(w, q, k, v, do, p=p, seed=77 + ci, atol_scale=oracle.keep_scale(p))


def test_seed_changes_mask():
    """Different seeds give different outputs; the same seed the same bits."""
    import torch
    import context_varlen_attention_amd as cva
    w = _case(0, "bf16")
    q, k, v, do = synth.random_tensors(w, 604)
    plan = plan_for(w)
    tq, tk, tv = device_inputs(w, q, k, v)
    a, _ = cva.fwd(plan, tq, tk, tv, dropout_p=0.5, seed=1)
    b, _ = cva.fwd(plan, tq, tk, tv, dropout_p=0.5, seed=1)
    c, _ = cva.fwd(plan, tq, tk, tv, dropout_p=0.5, seed=2)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and not torch.equal(a, c)


@pytest.mark.parametrize("seed", range(12))
def test_random_sweep(seed):
    w = random_case(seed)
    q, k, v, do = synth.random_tensors(w, 700 + seed)
    rng = np.random.default_rng([13, seed])
    _run(w, q, k, v, do, p=float(rng.choice([0.05, 0.2, 0.5, 0.75])), seed=int(rng.integers(0, 1 << 63)))


def _sample_rows(w, n, seed):
    T_loc = w.total_tokens // w.cp_size
    rng = np.random.default_rng(seed)
    rows = set(rng.integers(0, T_loc, size=n).tolist()) | {0, T_loc - 1, T_loc // 2, T_loc // 2 - 1}
    return sorted(rows)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,mask,dtype,heads", [("long128k", None, None, [0, 31]), ("mla32k", None, "bf16", [0, 15]),
                                                   ("mla32k", None, "fp16", [3]), ("sparse8", "blockwise", None, [15]),
                                                   ("sparse8", "lambda", None, [7]), ("sparse8", "shared_prefix", None, [0])])
def test_full_size_sampled_rows(name, mask, dtype, heads):
    """O, LSE and dQ of sampled local rows (a row's dQ depends on that row only)
    with dropout, forward as the benchmark runs it (split where the plan cuts); sparse8
    under the lambda, shared-prefix and blockwise masks."""
    import torch
    import context_varlen_attention_amd as cva
    w, (q, k, v, do) = workload_tensors(name, mask=mask, dtype=dtype)
    rows = _sample_rows(w, 24, 5)
    p, seed = 0.1, (7 << 40) + 11
    print(f"[drop] {w.name} {w.dtype} mask={w.mask} rows={len(rows)} heads={heads} p={p}", flush=True)
    plan = plan_for(w)
    tq, tk, tv, tdo = device_inputs(w, q, k, v, do)
    ws = True if plan.fwd_workspace_bytes() > 0 else None
    o, lse = cva.fwd(plan, tq, tk, tv, workspace=ws, dropout_p=p, seed=seed)
    dq, _, _ = cva.bwd(plan, tq, tk, tv, o, lse, tdo, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd_ref(w, q, k, v, rows=rows, heads=heads, dropout=(p, seed))
    loc = cva.local_token_ids(w.cu_seqlens, w.cp_size, w.rank)
    rdq, _, _ = oracle.bwd_ref(w, q, k, v, do[loc], heads=heads, rows=rows, dropout=(p, seed))
    o, lse, dq = o.float().cpu().numpy(), lse.cpu().numpy(), dq.float().cpu().numpy()
    assert_close(o[rows][:, heads], o_ref[rows][:, heads], w.dtype, "O")
    assert_close(lse[heads][:, rows], lse_ref[heads][:, rows], w.dtype, "LSE")
    assert_close(dq[rows][:, heads], rdq[rows][:, heads], w.dtype, "dQ")
