"""Launches on a stream other than the current one (GPU).

The binding allocates outputs and workspaces on the launch stream and marks
caller tensors used there, and launches wait for an asynchronous plan upload
made on another stream; the caching allocator must never hand out memory a
queued kernel still reads or writes.  The test queues fwd + bwd on a side
stream behind a long kernel, drops every reference it can, allocates and
fills fresh tensors on the default stream while the side stream still runs,
then checks the results against the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import assert_close, device_inputs, plan_for

pytestmark = pytest.mark.gpu


def test_side_stream_fwd_bwd_and_async_upload():
    import torch
    import context_varlen_attention_amd as cva
    w = synth.custom_workload([512, 96, 1536, 200], 2, 1, 8, 2, 128, 128, "bf16", name="streams")
    q, k, v, do = synth.random_tensors(w, 701)
    tq, tk, tv, tdo = device_inputs(w, q, k, v, do)
    side = torch.cuda.Stream()
    plan = plan_for(w)
    plan.upload("cuda", stream=side)          # asynchronous, on the side stream
    big = torch.randn(4096, 4096, device="cuda")
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(8):                    # keep the side stream busy for a while
            big = big @ big.T / 64.0
    o, lse = cva.fwd(plan, tq, tk, tv, stream=side)
    dq, dk, dv = cva.bwd(plan, tq, tk, tv, o, lse, tdo, stream=side)
    del tq, tk, tv, tdo                       # caller tensors still used by the side stream
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(64)]
    torch.cuda.synchronize()
    loc = cva.local_token_ids(w.cu_seqlens, w.cp_size, w.rank)
    ro, rl = oracle.fwd_ref(w, q, k, v)
    rdq, rdk, rdv = oracle.bwd_ref(w, q, k, v, do[loc])
    assert_close(o.float().cpu().numpy(), ro, "bf16", "O")
    assert_close(lse.cpu().numpy(), rl, "bf16", "LSE")
    for name, got, ref in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert_close(got.float().cpu().numpy(), ref, "bf16", name)
    assert all(bool((j == 7.0).all()) for j in junk)
