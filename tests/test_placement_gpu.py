"""One device's share of a block placement, run on the GPU (DCP paper, section
4.1: computation blocks; Fig. 9(b): several computation blocks feeding one
output block are reduced by their log-sum-exp).

For every device of a placement the test runs the device's plan
(cva_placement_plan_create + cva_fwd_split) on the packed batch and compares
the rows it writes with the oracle's definition of that share (attention over
the keys of the device's K/V blocks only); rows of other O blocks must stay
untouched.  The devices' partial results are then reduced on the host, as the
owners of the O blocks would, and compared with unsplit attention.  Every case
has an output tile fed by several computation blocks on one device.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.placement import share_fwd_ref
from tests.gpu_helpers import assert_close, torch_dtype

pytestmark = pytest.mark.gpu

LENS = [1280, 640, 2048, 200]
CASES = [
    # n_devices, block, hq, hkv, dqk, dv, mask, mask parameters
    (3, 128, 4, 2, 128, 128, "causal", {}),
    (4, 64, 2, 2, 64, 64, "shared_prefix", {}),
    (2, 256, 8, 1, 128, 128, "lambda", dict(sink=64, window=300)),
    (3, 128, 4, 4, 192, 128, "causal", {}),
    (3, 128, 4, 2, 128, 128, "blockwise", dict(sink=1, window=2, block=128)),
]


def _merge(parts):
    """Log-sum-exp reduction of partial results (o [T,H,D], lse [H,T]) in fp64."""
    lses = np.stack([l for _, l in parts])                      # [n, H, T]
    m = np.max(np.where(np.isfinite(lses), lses, -np.inf), axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - safe_m), 0.0)  # [n, H, T]
    den = w.sum(axis=0)
    num = sum(w[n].T[:, :, None] * np.nan_to_num(parts[n][0]) for n in range(len(parts)))
    o = num / np.where(den > 0, den, 1.0).T[:, :, None]
    lse = np.where(den > 0, safe_m + np.log(np.where(den > 0, den, 1.0)), -np.inf)
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_placement_shares_match_oracle_and_reduce_to_full_attention(ci, dtype):
    import torch
    import context_varlen_attention_amd as cva
    R, B, hq, hkv, dqk, dv, mask, mp = CASES[ci]
    bb = None
    if mask == "shared_prefix":
        bb = np.array([synth.shared_prefix_bounds(L, prefix=256) for L in LENS])
    w = synth.custom_workload(LENS, 1, 0, hq, hkv, dqk, dv, dtype, mask=mask, sink=mp.get("sink", 0),
                              window=mp.get("window", 0), branch_bounds=bb, block=mp.get("block", 0),
                              name=f"placed{ci}")
    print(f"[placement] case {ci} {dtype}: devices={R} block={B} H={hq}/{hkv} D={dqk}/{dv} "
          f"mask={mask}", flush=True)
    q, k, v = synth.random_tensors(w, 900 + ci, with_dout=False)
    pl = cva.Placement(w.cu_seqlens, R, B, hq=hq, hkv=hkv, d_qk=dqk, d_v=dv, dtype=dtype, mask=mask,
                       sink=w.sink, window=w.window, branch_bounds=bb, mask_block=w.block)
    comp_dev = {(int(i), int(qb), int(kb)): int(d) for i, qb, kb, d in pl.comp_blocks}
    fed = {}
    for (i, qb, kb), d in comp_dev.items():
        fed[(d, i, qb)] = fed.get((d, i, qb), 0) + 1
    assert max(fed.values()) >= 2, "no output block fed by two computation blocks on one device"
    dt = torch_dtype(dtype)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt) for x in (q, k, v))
    T = w.total_tokens
    parts = []
    for d in range(R):
        pp = pl.device_plan(d)
        o = torch.full((T, hq, dv), float("nan"), dtype=dt, device="cuda")
        lse = torch.full((hq, T), float("nan"), dtype=torch.float32, device="cuda")
        cva.fwd(pp, tq, tk, tv, out=o, lse=lse, workspace=True)
        torch.cuda.synchronize()
        o, lse = o.double().cpu().numpy(), lse.double().cpu().numpy()
        ro, rl = share_fwd_ref(w, q, k, v, B, comp_dev, d)
        mine = ~np.isnan(rl[0])
        assert np.isnan(o[~mine]).all() and np.isnan(lse[:, ~mine]).all(), "a row of another O block was written"
        assert_close(o[mine], ro[mine], dtype, f"O of device {d}")
        assert_close(lse[:, mine], rl[:, mine], dtype, f"LSE of device {d}")
        parts.append((np.where(mine[:, None, None], o, np.nan), np.where(mine[None, :], lse, np.nan)))
    mo, ml = _merge(parts)
    fo, fl = oracle.fwd_full_ref(w, q, k, v)
    assert_close(mo, fo, dtype, "O reduced over devices")
    assert_close(ml, fl, dtype, "LSE reduced over devices")


@pytest.mark.parametrize("ci", [0, 1, 3, 4])
def test_placement_dropout_reduces_to_full_dropout_attention(ci):
    """Attention dropout on placement shares: the keep mask follows in-sequence
    positions, so the devices' partial outputs, reduced by their LSE, equal
    unsplit attention with the same dropout."""
    import torch
    import context_varlen_attention_amd as cva
    R, B, hq, hkv, dqk, dv, mask, mp = CASES[ci]
    dtype = "bf16"
    bb = None
    if mask == "shared_prefix":
        bb = np.array([synth.shared_prefix_bounds(L, prefix=256) for L in LENS])
    w = synth.custom_workload(LENS, 1, 0, hq, hkv, dqk, dv, dtype, mask=mask, sink=mp.get("sink", 0),
                              window=mp.get("window", 0), branch_bounds=bb, block=mp.get("block", 0),
                              name=f"placed_drop{ci}")
    print(f"[placement dropout] case {ci}: devices={R} block={B} mask={mask}", flush=True)
    q, k, v = synth.random_tensors(w, 950 + ci, with_dout=False)
    pl = cva.Placement(w.cu_seqlens, R, B, hq=hq, hkv=hkv, d_qk=dqk, d_v=dv, dtype=dtype, mask=mask,
                       sink=w.sink, window=w.window, branch_bounds=bb, mask_block=w.block)
    dt = torch_dtype(dtype)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt) for x in (q, k, v))
    T = w.total_tokens
    p, seed = 0.2, 4242 + ci
    parts = []
    for d in range(R):
        pp = pl.device_plan(d)
        o = torch.full((T, hq, dv), float("nan"), dtype=dt, device="cuda")
        lse = torch.full((hq, T), float("nan"), dtype=torch.float32, device="cuda")
        cva.fwd(pp, tq, tk, tv, out=o, lse=lse, workspace=True, dropout_p=p, seed=seed)
        torch.cuda.synchronize()
        o, lse = o.double().cpu().numpy(), lse.double().cpu().numpy()
        mine = ~np.isnan(lse[0])
        parts.append((np.where(mine[:, None, None], o, np.nan), np.where(mine[None, :], lse, np.nan)))
    mo, ml = _merge(parts)
    fo, fl = oracle.fwd_full_ref(w, q, k, v, dropout=(p, seed))
    assert_close(mo, fo, dtype, "O reduced over devices (dropout)")
    assert_close(ml, fl, dtype, "LSE reduced over devices (dropout)")
