"""Forward parity: libcva on the GPU against the fp64 oracle.

Small cases are compared element by element on every output.  The full-size
workloads (16k GQA, 128k single sequence, sparse masks, MLA shape) run in the
same launch configuration bench.py uses and are compared on every row of at
least one whole K/V head group -- so every forward work item of that group,
including the longest prefixes -- plus sampled rows of every head.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import (assert_close, device_inputs, fwd_ref_heads, plan_for,
                               workload_tensors)

pytestmark = pytest.mark.gpu


def _run(w, q, k, v, rows=None, scale=None, split=False, heads=None, ref=None):
    import torch
    import context_varlen_attention_amd as cva
    print(f"[fwd] {w.name} {w.dtype} mask={w.mask} R={w.cp_size} r={w.rank} T={w.total_tokens} "
          f"H={w.hq}/{w.hkv} D={w.d_qk}/{w.d_v} split={split} heads={heads}", flush=True)
    plan = plan_for(w)
    dq_, dk_, dv_ = device_inputs(w, q, k, v)
    if split:
        assert plan.fwd_workspace_bytes() > 0, "the case was meant to split K/V ranges"
    o, lse = cva.fwd(plan, dq_, dk_, dv_, softmax_scale=scale, workspace=True if split else None)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    if ref is None:
        ref = (oracle.fwd_ref(w, q, k, v, scale=scale, rows=rows) if heads is None
               else fwd_ref_heads(w, q, k, v, heads, rows=rows, scale=scale))
    o_ref, lse_ref = ref
    if rows is not None:
        o, o_ref, lse, lse_ref = o[rows], o_ref[rows], lse[:, rows], lse_ref[:, rows]
    if heads is not None:
        o, o_ref, lse, lse_ref = o[:, heads], o_ref[:, heads], lse[heads], lse_ref[heads]
    eo, ro = assert_close(o, o_ref, w.dtype, "O")
    el, rl = assert_close(lse, lse_ref, w.dtype, "LSE")
    print(f"[fwd]   max |err| O {eo:.2e} LSE {el:.2e}; headroom ratio O {ro:.3f} LSE {rl:.3f}",
          flush=True)
    return plan


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_tiny(dtype):
    w = synth.make_workload("tiny", dtype=dtype)
    q, k, v = synth.make_tensors(w, with_dout=False)
    _run(w, q, k, v)


SMALL = [
    # lens, R, r, hq, hkv, dqk, dv, mask, extra
    ([64, 128, 64], 2, 1, 4, 4, 64, 64, "causal", {}),
    ([8, 24, 200, 16, 1000], 4, 3, 8, 2, 128, 128, "causal", {}),
    ([8, 24, 200, 16, 1000], 4, 0, 8, 8, 128, 128, "causal", {}),
    ([512, 96, 1536], 2, 1, 6, 3, 128, 128, "causal", {}),
    ([720, 48], 3, 2, 4, 1, 192, 128, "causal", {}),
    ([1024, 640], 1, 0, 2, 2, 128, 128, "lambda", dict(sink=64, window=256)),
    ([1200, 400], 2, 1, 4, 2, 64, 64, "lambda", dict(sink=5, window=77)),
    ([1280, 768], 1, 0, 2, 1, 128, 128, "shared_prefix",
     dict(bounds=[[256, 512, 768, 1024, 1280], [128, 288, 448, 608, 768]])),
    ([2048, 1280], 1, 0, 4, 2, 128, 128, "blockwise", dict(block=256, sink=1, window=2)),
    ([1536, 640, 3072], 2, 1, 4, 4, 64, 64, "blockwise", dict(block=96, sink=2, window=3)),
    ([1920, 960], 2, 0, 2, 2, 192, 128, "blockwise", dict(block=80, sink=1, window=1)),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("ci", range(len(SMALL)))
def test_small_cases(ci, dtype):
    lens, R, r, hq, hkv, dqk, dv, mask, ex = SMALL[ci]
    w = synth.custom_workload(lens, R, r, hq, hkv, dqk, dv, dtype, mask=mask,
                              sink=ex.get("sink", 0), window=ex.get("window", 0),
                              branch_bounds=ex.get("bounds"), name=f"small{ci}",
                              block=ex.get("block", 0))
    q, k, v = synth.random_tensors(w, 100 + ci, with_dout=False)
    _run(w, q, k, v)


# cases whose forward Q tiles walk more than 8 K/V tiles: cva_fwd_split cuts them
SPLIT = [1, 2, 3, 5, 8, 9]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("ci", SPLIT)
def test_small_cases_split(ci, dtype):
    lens, R, r, hq, hkv, dqk, dv, mask, ex = SMALL[ci]
    w = synth.custom_workload(lens, R, r, hq, hkv, dqk, dv, dtype, mask=mask,
                              sink=ex.get("sink", 0), window=ex.get("window", 0),
                              branch_bounds=ex.get("bounds"), name=f"small{ci}",
                              block=ex.get("block", 0))
    q, k, v = synth.random_tensors(w, 100 + ci, with_dout=False)
    _run(w, q, k, v, split=True)


@pytest.mark.parametrize("wgs", ["3", "1"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("ci", range(len(SMALL)))
def test_small_cases_streamed(ci, dtype, wgs, monkeypatch):
    """The streamed forward (one work-group per CU walking its items as one tile
    stream) forced on for every head dim, plain and with split K/V ranges where
    the case cuts: several items per work-group, item boundaries mid-stream.
    With one work-group per head group every item of the case is a boundary of
    one stream (item epilogues' stores then meet the most tile loads in flight)."""
    monkeypatch.setenv("CVA_FWD_STREAM", "1")
    monkeypatch.setenv("CVA_FWD_STREAM_WGS", wgs)  # several items per work-group
    lens, R, r, hq, hkv, dqk, dv, mask, ex = SMALL[ci]
    w = synth.custom_workload(lens, R, r, hq, hkv, dqk, dv, dtype, mask=mask,
                              sink=ex.get("sink", 0), window=ex.get("window", 0),
                              branch_bounds=ex.get("bounds"), name=f"small{ci}",
                              block=ex.get("block", 0))
    q, k, v = synth.random_tensors(w, 100 + ci, with_dout=False)
    plan = _run(w, q, k, v)
    if ci in SPLIT:
        _run(w, q, k, v, split=True)
    wgs, start, _ = plan.tables()["fwd_deal"]
    assert wgs > 0 and np.diff(start).max() >= 2, "no work-group walks several items"


def test_gqa16k_split_all_rows(monkeypatch):
    """cva_fwd_split with every Q tile longer than 24 K/V tiles cut (the default
    leaves this batch whole: its longest tile walks 1.25x the per-CU average)."""
    monkeypatch.setenv("CVA_FWD_SPLIT_CAP", "24")
    w = synth.make_workload("gqa16k")
    q, k, v = synth.make_tensors(w, with_dout=False)
    _run(w, q, k, v, split=True)


def test_tiny_custom_scale():
    w = synth.make_workload("tiny", dtype="bf16")
    q, k, v = synth.make_tensors(w, with_dout=False)
    _run(w, q, k, v, scale=0.05)


def _sample_rows(w, n, seed):
    T_loc = w.total_tokens // w.cp_size
    rng = np.random.default_rng(seed)
    rows = set(rng.integers(0, T_loc, size=n).tolist())
    rows |= {0, T_loc - 1, T_loc // 2, T_loc // 2 - 1}
    return sorted(rows)


def test_gqa16k_all_rows():
    w = synth.make_workload("gqa16k")
    q, k, v = synth.make_tensors(w, with_dout=False)
    _run(w, q, k, v)


# the last K/V group of the 128k sequence: query heads 28..31, all 16384 local
# rows (chunk 3 against a 32768-key prefix, chunk 12 against 106496 keys)
LONG_GROUP = [28, 29, 30, 31]


@functools.lru_cache(maxsize=1)
def _long128k_group_ref():
    w, (q, k, v, do) = workload_tensors("long128k")
    return fwd_ref_heads(w, q, k, v, LONG_GROUP)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("split", [False, True])
def test_long128k_group_all_rows(split, monkeypatch):
    """cva_fwd, and cva_fwd_split with every Q tile longer than 256 K/V tiles cut
    into pieces (the default cut leaves this batch whole: its longest Q tile
    walks fewer K/V tiles than the average compute unit does)."""
    if split:
        monkeypatch.setenv("CVA_FWD_SPLIT_CAP", "256")
    w, (q, k, v, do) = workload_tensors("long128k")
    _run(w, q, k, v, heads=LONG_GROUP, split=split, ref=_long128k_group_ref())


def test_long128k_sampled_rows():
    w, (q, k, v, do) = workload_tensors("long128k")
    _run(w, q, k, v, rows=_sample_rows(w, 48, 2))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mask", ["lambda", "shared_prefix", "blockwise"])
def test_sparse8_head_all_rows(mask):
    """Every row of query head 15 (its own K/V head): all 81408 rows of the batch."""
    w, (q, k, v, do) = workload_tensors("sparse8", mask=mask)
    _run(w, q, k, v, heads=[15])


@pytest.mark.parametrize("mask", ["lambda", "shared_prefix", "blockwise"])
def test_sparse8_sampled_rows(mask):
    w, (q, k, v, do) = workload_tensors("sparse8", mask=mask)
    _run(w, q, k, v, rows=_sample_rows(w, 64, 3))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_mla32k_heads_all_rows(dtype):
    """Every row of query heads 0 and 15 (Q/K head dim 192, V head dim 128)."""
    w, (q, k, v, do) = workload_tensors("mla32k", dtype=dtype)
    _run(w, q, k, v, heads=[0, 15])


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_mla32k_sampled_rows(dtype):
    w, (q, k, v, do) = workload_tensors("mla32k", dtype=dtype)
    _run(w, q, k, v, rows=_sample_rows(w, 64, 4))


def test_deterministic_repeat():
    import torch
    import context_varlen_attention_amd as cva
    w = synth.make_workload("gqa16k")
    q, k, v = synth.make_tensors(w, with_dout=False)
    plan = plan_for(w)
    a, b, c = device_inputs(w, q, k, v)
    o1, l1 = cva.fwd(plan, a, b, c)
    o2, l2 = cva.fwd(plan, a, b, c)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
