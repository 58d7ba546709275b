"""cva_bwd_noalloc (backward with no device allocation) against cva_bwd.

Both entry points are called raw through the C ABI on the same inputs; the
allocation-free one keeps its row statistics in the library's own device array
instead of a caller workspace, and runs the same kernels, so its outputs must
equal cva_bwd's bit for bit (and the fp64 oracle within the bf16/fp16
tolerance).  Two calls in a row, the second on a smaller batch, so that the
second reads an array still holding the first call's values.
"""
import ctypes
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_close, device_inputs, plan_for

pytestmark = pytest.mark.gpu

CASES = [
    # lens, R, r, hq, hkv, dqk, dv, dtype
    ([512, 96, 1536, 200], 2, 1, 8, 2, 128, 128, "bf16"),
    ([64, 128, 64], 2, 0, 4, 4, 64, 64, "fp16"),
]


def _bwd(plan, w, tq, tk, tv, o, lse, tdo, noalloc):
    import torch
    import context_varlen_attention_amd as cva
    L = cva.load_library()
    vp = ctypes.c_void_p
    dq, dk, dv = (torch.full_like(x, 3.0) for x in (tq, tk, tv))  # overwritten in full
    scale = ctypes.c_float(1.0 / math.sqrt(w.d_qk))
    s = vp(torch.cuda.current_stream().cuda_stream)
    ptrs = [vp(x.data_ptr()) for x in (tq, tk, tv, o, lse, tdo, dq, dk, dv)]
    if noalloc:
        st = L.cva_bwd_noalloc(plan.handle, *ptrs, scale, s)
    else:
        ws = torch.empty(int(L.cva_bwd_workspace_bytes(plan.handle)), dtype=torch.uint8,
                         device=tq.device)
        st = L.cva_bwd(plan.handle, *ptrs, vp(ws.data_ptr()), ws.numel(), scale, s)
    assert st == 0, L.cva_last_error().decode()
    torch.cuda.synchronize()
    return dq, dk, dv


def test_noalloc_matches_cva_bwd_twice_second_smaller():
    import torch
    import context_varlen_attention_amd as cva
    L = cva.load_library()
    assert int(L.cva_bwd_noalloc_max_bytes()) == 16 << 20
    sizes = []
    for ci, (lens, R, r, hq, hkv, dqk, dv_, dt) in enumerate(CASES):
        w = synth.custom_workload(lens, R, r, hq, hkv, dqk, dv_, dt, name=f"noalloc{ci}")
        print(f"[noalloc] case {ci}: lens={lens} R={R} r={r} H={hq}/{hkv} D={dqk}/{dv_} {dt}",
              flush=True)
        q, k, v, do = synth.random_tensors(w, 600 + ci)
        plan = plan_for(w)
        sizes.append(int(L.cva_bwd_workspace_bytes(plan.handle)))
        tq, tk, tv, tdo = device_inputs(w, q, k, v, do)
        o, lse = cva.fwd(plan, tq, tk, tv)
        a = _bwd(plan, w, tq, tk, tv, o, lse, tdo, noalloc=True)
        b = _bwd(plan, w, tq, tk, tv, o, lse, tdo, noalloc=False)
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        loc = cva.local_token_ids(w.cu_seqlens, w.cp_size, w.rank)
        ref = oracle.bwd_ref(w, q, k, v, do[loc])
        for name, got, rr in zip(("dQ", "dK", "dV"), a, ref):
            assert_close(got.float().cpu().numpy(), rr, dt, name)
    assert sizes[1] < sizes[0]


def test_noalloc_rejects_a_plan_beyond_its_array():
    """Hq * T_loc above 2^21 rows of statistics: CVA_E_WORKSPACE before any launch."""
    import torch
    import context_varlen_attention_amd as cva
    L = cva.load_library()
    w = synth.custom_workload([65536, 4096], 1, 0, 32, 8, 128, 128, "bf16", name="noalloc_big")
    plan = plan_for(w)
    assert int(L.cva_bwd_workspace_bytes(plan.handle)) > int(L.cva_bwd_noalloc_max_bytes())
    plan.upload("cuda")
    dummy = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    vp = ctypes.c_void_p
    p = vp(dummy.data_ptr())
    st = L.cva_bwd_noalloc(plan.handle, p, p, p, p, p, p, p, p, p, ctypes.c_float(0.1),
                           vp(torch.cuda.current_stream().cuda_stream))
    assert st == 13, st  # CVA_E_WORKSPACE
    assert b"at most" in L.cva_last_error()
    torch.cuda.synchronize()
    assert (dummy == 0).all()
