"""Backward parity: libcva dQ / rank-major dK / dV on the GPU against the fp64 oracle.

Small shapes are compared element by element on every output (all masks, GQA,
expanded-MLA head dims, several CP ranks); the 32k MLA-shape and 16k GQA
workloads run at full size and are compared on a subset of heads (all rows of
those heads).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_close, device_inputs, plan_for

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
    rdq, rdk, rdv = oracle.bwd_ref(w, q, k, v, do[loc], scale=scale, heads=heads)
    dq, dk, dv = (x.float().cpu().numpy() for x in (dq, dk, dv))
    if heads is not None:
        G = w.hq // w.hkv
        groups = sorted({h // G for h in heads})
        dq, rdq = dq[:, heads], rdq[:, heads]
        dk, rdk, dv, rdv = dk[:, groups], rdk[:, groups], dv[:, groups], rdv[:, groups]
    e1 = assert_close(dq, rdq, w.dtype, "dQ")
    e2 = assert_close(dk, rdk, w.dtype, "dK")
    e3 = assert_close(dv, rdv, w.dtype, "dV")
    print(f"[bwd]   max |err| dQ {e1:.2e} dK {e2:.2e} dV {e3:.2e}", flush=True)
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


def test_tiny_bf16_custom_scale():
    w = synth.make_workload("tiny", dtype="bf16")
    q, k, v, do = synth.make_tensors(w)
    _run(w, q, k, v, do, scale=0.3)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_mla32k_three_heads(dtype):
    w = synth.make_workload("mla32k", dtype=dtype)
    q, k, v, do = synth.make_tensors(w)
    _run(w, q, k, v, do, heads=[0, 7, 15])


def test_gqa16k_one_group():
    """Full 16k GQA workload in the benchmark's launch configuration: all rows of
    one K/V group's four query heads (dQ of each, and the group's complete
    dK / dV)."""
    w = synth.make_workload("gqa16k")
    q, k, v, do = synth.make_tensors(w)
    _run(w, q, k, v, do, heads=[4, 5, 6, 7])


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
