"""Backward parity: libcva dQ / rank-major dK / dV on the GPU against the fp64 oracle.

Small shapes are compared element by element on every output (all masks, GQA,
expanded-MLA head dims, several CP ranks).  The full-size workloads (16k GQA,
128k single sequence, sparse masks, 32k MLA shape) run in the benchmark's
launch configuration and are compared on whole K/V head groups: dQ of every
local row of the group's query heads and the group's complete rank-major dK/dV
(every dK/dV work item of that K/V head).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import (assert_close, bwd_ref_heads, device_inputs, plan_for,
                               workload_tensors)

pytestmark = pytest.mark.gpu


def _run(w, q, k, v, do, heads=None, scale=None):
    import torch
    import context_varlen_attention_amd as cva
    print(f"[bwd] {w.name} {w.dtype} mask={w.mask} R={w.cp_size} r={w.rank} T={w.total_tokens} "
          f"H={w.hq}/{w.hkv} D={w.d_qk}/{w.d_v} heads={heads}", flush=True)
    plan = plan_for(w)
    tq, tk, tv, tdo = device_inputs(w, q, k, v, do)
    o, lse = cva.fwd(plan, tq, tk, tv, softmax_scale=scale)
    dq, dk, dv = cva.bwd(plan, tq, tk, tv, o, lse, tdo, softmax_scale=scale)
    torch.cuda.synchronize()
    loc = cva.local_token_ids(w.cu_seqlens, w.cp_size, w.rank)
    if heads is None:
        rdq, rdk, rdv = oracle.bwd_ref(w, q, k, v, do[loc], scale=scale)
    else:
        rdq, rdk, rdv = bwd_ref_heads(w, q, k, v, do[loc], heads, scale=scale)
    dq, dk, dv = (x.float().cpu().numpy() for x in (dq, dk, dv))
    if heads is not None:
        G = w.hq // w.hkv
        groups = sorted({h // G for h in heads})
        dq, rdq = dq[:, heads], rdq[:, heads]
        dk, rdk, dv, rdv = dk[:, groups], rdk[:, groups], dv[:, groups], rdv[:, groups]
    e1, r1 = assert_close(dq, rdq, w.dtype, "dQ")
    e2, r2 = assert_close(dk, rdk, w.dtype, "dK")
    e3, r3 = assert_close(dv, rdv, w.dtype, "dV")
    print(f"[bwd]   max |err| dQ {e1:.2e} dK {e2:.2e} dV {e3:.2e}; headroom ratio "
          f"dQ {r1:.3f} dK {r2:.3f} dV {r3:.3f}", flush=True)
    return dq, dk, dv


CASES = [
    # lens, R, r, hq, hkv, dqk, dv, mask, extra
    ([64, 128, 64], 2, 0, 4, 4, 64, 64, "causal", {}),
    ([64, 128, 64], 2, 1, 4, 2, 128, 128, "causal", {}),
    ([8, 24, 200, 16, 1000], 4, 3, 8, 2, 128, 128, "causal", {}),
    ([8, 24, 200, 16, 1000], 4, 0, 4, 4, 192, 128, "causal", {}),
    ([512, 96, 1536], 2, 1, 6, 3, 128, 128, "causal", {}),
    ([720, 48], 3, 2, 2, 2, 192, 128, "causal", {}),
    ([1024, 640], 1, 0, 2, 2, 128, 128, "lambda", dict(sink=64, window=256)),
    ([1200, 400], 2, 1, 4, 2, 64, 64, "lambda", dict(sink=5, window=77)),
    ([1280, 768], 1, 0, 2, 1, 128, 128, "shared_prefix",
     dict(bounds=[[256, 512, 768, 1024, 1280], [128, 288, 448, 608, 768]])),
    ([2048, 1280], 1, 0, 4, 2, 128, 128, "blockwise", dict(block=256, sink=1, window=2)),
    ([1536, 640, 3072], 2, 1, 4, 4, 64, 64, "blockwise", dict(block=96, sink=2, window=3)),
    ([1920, 960], 2, 0, 2, 2, 192, 128, "blockwise", dict(block=80, sink=1, window=1)),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_small_cases(ci, dtype):
    lens, R, r, hq, hkv, dqk, dv, mask, ex = CASES[ci]
    w = synth.custom_workload(lens, R, r, hq, hkv, dqk, dv, dtype, mask=mask,
                              sink=ex.get("sink", 0), window=ex.get("window", 0),
                              branch_bounds=ex.get("bounds"), name=f"bsmall{ci}",
                              block=ex.get("block", 0))
    q, k, v, do = synth.random_tensors(w, 200 + ci)
    _run(w, q, k, v, do)


def test_sharp_scale_d128():
    """Softmax scale 0.2 at Q/K head dim 128 (2.3x the default): past 1.5x the
    default the forward normalises by the sum of the rounded P (the other
    tests, at the default scale, take the unrounded sum)."""
    lens, R, r, hq, hkv, dqk, dv, mask, ex = CASES[1]
    w = synth.custom_workload(lens, R, r, hq, hkv, dqk, dv, "bf16", mask=mask, name="bsharp")
    q, k, v, do = synth.random_tensors(w, 602)
    _run(w, q, k, v, do, scale=0.2)


def test_tiny_bf16_custom_scale():
    w = synth.make_workload("tiny", dtype="bf16")
    q, k, v, do = synth.make_tensors(w)
    _run(w, q, k, v, do, scale=0.3)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_mla32k_heads_0_15(dtype):
    """Q/K head dim 192: every local row of heads 0 and 15 (each its own K/V head)."""
    w, (q, k, v, do) = workload_tensors("mla32k", dtype=dtype)
    _run(w, q, k, v, do, heads=[0, 15])


@pytest.mark.timeout(600)
def test_gqa16k_first_and_last_group():
    """Full 16k GQA workload in the benchmark's launch configuration: all rows of
    the first and the last K/V group (dQ of their eight query heads, and the two
    groups' complete dK / dV)."""
    w, (q, k, v, do) = workload_tensors("gqa16k")
    _run(w, q, k, v, do, heads=[0, 1, 2, 3, 28, 29, 30, 31])


@pytest.mark.timeout(900)
def test_long128k_last_group():
    """The 131072-token sequence, rank 3 of 8: dQ of all 16384 local rows of
    query heads 28..31 and K/V head 7's complete rank-major dK / dV."""
    w, (q, k, v, do) = workload_tensors("long128k")
    _run(w, q, k, v, do, heads=[28, 29, 30, 31])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mask", ["lambda", "shared_prefix", "blockwise"])
def test_sparse8_one_head(mask):
    """The 8-sequence sparse-mask batch (81408 rows): head 15's dQ, dK and dV."""
    w, (q, k, v, do) = workload_tensors("sparse8", mask=mask)
    _run(w, q, k, v, do, heads=[15])


def test_uncovered_rows_are_zero_and_repeat_is_bitwise():
    import torch
    import context_varlen_attention_amd as cva
    w = synth.custom_workload([64, 256, 128], 4, 2, 4, 2, 128, 128, "bf16")
    q, k, v, do = synth.random_tensors(w, 7)
    plan = plan_for(w)
    tq, tk, tv, tdo = device_inputs(w, q, k, v, do)
    o, lse = cva.fwd(plan, tq, tk, tv)
    dk0 = torch.full_like(tk, 7.0)
    dv0 = torch.full_like(tv, 7.0)
    a = cva.bwd(plan, tq, tk, tv, o, lse, tdo, dk_rm=dk0, dv_rm=dv0)
    b = cva.bwd(plan, tq, tk, tv, o, lse, tdo)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    covered = np.zeros(w.total_tokens, bool)
    covered[plan.metadata["kv_index"]] = True
    dk = a[1].float().cpu().numpy()
    assert (dk[~covered] == 0).all() and (a[2].float().cpu().numpy()[~covered] == 0).all()
