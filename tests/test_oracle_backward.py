"""Pins for the oracle's backward (CPU only).

* central finite differences in float64 of L = sum(dO * O) on tiny shapes;
* torch float64 autograd through an explicit-mask scaled_dot_product_attention;
* summing every rank's rank-major dK/dV partials (each rank with its own rows of
  one full dO) gives the dK/dV of unsplit attention, and each rank's dQ rows
  are the unsplit dQ at its positions (MindSpeed RFC section 1.3 and 2: Q/K/V
  gradients equal the non-CP reference; section 3.1: dK/dV index_add_ into the
  rank-major buffer followed by a reduce-scatter).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.split import rank_local_positions, rank_major_row_of_position
from tests.test_oracle_attention import _wl


def _torch_mask(mask, L, bounds):
    """The test cases' masks written directly in torch (sink 2, window 5 for lambda)."""
    qq = torch.arange(L)[:, None]
    kk = torch.arange(L)[None, :]
    if mask == "causal":
        return kk <= qq
    if mask == "lambda":
        return (kk <= qq) & ((kk < 2) | (qq - kk < 5))
    b = [int(x) for x in bounds]
    M = torch.zeros(L, L, dtype=torch.bool)
    M[:b[0], :b[0]] = torch.tril(torch.ones(b[0], b[0], dtype=torch.bool))
    st = b[0]
    for e in b[1:]:
        M[st:e, :b[0]] = True
        M[st:e, st:e] = torch.tril(torch.ones(e - st, e - st, dtype=torch.bool))
        st = e
    return M


def _loss(w, q, k, v, do_loc, scale):
    o, _ = oracle.fwd_ref(w, q, k, v, scale)
    return float((o * do_loc).sum())


@pytest.mark.parametrize("mask", ["causal", "lambda", "shared_prefix"])
def test_finite_differences(mask):
    c = dict(lens=[8, 12], R=2, r=1, hq=2, hkv=1, d=3, mask=mask, sink=1, window=3,
             bounds=[[2, 5, 8], [4, 8, 12]])
    w = _wl(c)
    q, k, v, do_full = [x.astype(np.float64) for x in synth.random_tensors(w, 21)]
    cu = [int(x) for x in w.cu_seqlens]
    loc = rank_local_positions(cu, w.cp_size, w.rank)
    do_loc = do_full[loc]
    scale = 0.6
    dq, dk, dv = oracle.bwd_ref(w, q, k, v, do_loc, scale)
    row_of = rank_major_row_of_position(cu, w.cp_size)
    eps = 1e-6
    rng = np.random.default_rng(1)
    for name, X, grad in (("q", q, None), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in X.shape)
            Xp = X.copy(); Xp[idx] += eps
            Xm = X.copy(); Xm[idx] -= eps
            args_p = dict(q=q, k=k, v=v); args_p[name] = Xp
            args_m = dict(q=q, k=k, v=v); args_m[name] = Xm
            num = (_loss(w, args_p["q"], args_p["k"], args_p["v"], do_loc, scale)
                   - _loss(w, args_m["q"], args_m["k"], args_m["v"], do_loc, scale)) / (2 * eps)
            if name == "q":
                tok = idx[0]
                ana = dq[loc.index(tok), idx[1], idx[2]] if tok in loc else 0.0
            else:
                ana = grad[row_of[idx[0]], idx[1], idx[2]]
            assert abs(num - ana) < 1e-7, (name, idx, num, ana)


@pytest.mark.parametrize("R,r", [(1, 0), (2, 0), (2, 1), (3, 1)])
@pytest.mark.parametrize("mask", ["causal", "lambda", "shared_prefix"])
def test_torch_autograd(R, r, mask):
    lens = [6 * R, 12 * R]
    c = dict(lens=lens, R=R, r=r, hq=4, hkv=2, d=8, mask=mask, sink=2, window=5,
             bounds=[[2 * R, 4 * R, 6 * R], [4 * R, 8 * R, 12 * R]])
    w = _wl(c, dv=6)
    q, k, v, do_full = synth.random_tensors(w, 33)
    cu = [int(x) for x in w.cu_seqlens]
    loc = rank_local_positions(cu, R, r)
    scale = 0.35
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    G = w.hq // w.hkv
    outs = []
    for i in range(len(cu) - 1):
        s0, s1 = cu[i], cu[i + 1]
        M = _torch_mask(mask, s1 - s0, None if w.branch_bounds is None else w.branch_bounds[i])
        Q = tq[s0:s1].permute(1, 0, 2)
        K = tk[s0:s1].permute(1, 0, 2).repeat_interleave(G, dim=0)
        V = tv[s0:s1].permute(1, 0, 2).repeat_interleave(G, dim=0)
        outs.append(torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, attn_mask=M, scale=scale).permute(1, 0, 2))
    O = torch.cat(outs, 0)
    dO_full = torch.zeros_like(O)
    dO_full[loc] = torch.tensor(do_full[loc], dtype=torch.float64)
    (O * dO_full).sum().backward()
    dq, dk, dv = oracle.bwd_ref(w, q, k, v, do_full[loc], scale)
    row_of = rank_major_row_of_position(cu, R)
    np.testing.assert_allclose(dq, tq.grad.numpy()[loc], atol=1e-11)
    np.testing.assert_allclose(dk[row_of], tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv[row_of], tv.grad.numpy(), atol=1e-11)


@pytest.mark.parametrize("R", [2, 4])
@pytest.mark.parametrize("mask", ["causal", "lambda"])
def test_sum_over_ranks_equals_unsplit(R, mask):
    lens = [2 * R * 3, 2 * R * 5]
    c = dict(lens=lens, R=R, r=0, hq=2, hkv=1, d=4, mask=mask, sink=1, window=4)
    w1 = _wl(dict(c, R=1))
    q, k, v, do_full = synth.random_tensors(w1, 44)
    cu = [int(x) for x in w1.cu_seqlens]
    dq1, dk1, dv1 = oracle.bwd_ref(w1, q, k, v, do_full)  # R=1: packed order == rank-major
    dk_sum = np.zeros_like(dk1)
    dv_sum = np.zeros_like(dv1)
    for r in range(R):
        w = _wl(dict(c, r=r))
        loc = rank_local_positions(cu, R, r)
        dq, dk, dv = oracle.bwd_ref(w, q, k, v, do_full[loc])
        dk_sum += dk
        dv_sum += dv
        np.testing.assert_allclose(dq, dq1[loc], atol=1e-12)
    row_of = rank_major_row_of_position(cu, R)
    np.testing.assert_allclose(dk_sum[row_of], dk1, atol=1e-12)
    np.testing.assert_allclose(dv_sum[row_of], dv1, atol=1e-12)


@pytest.mark.parametrize("mask", ["causal", "lambda", "shared_prefix"])
def test_row_subset_and_blocks_against_autograd(mask):
    """bwd_ref(rows=S, block=b): dQ of the rows in S and their share of dK/dV,
    which is what autograd gives when dO is zero outside S (dK and dV are sums
    over query rows)."""
    R, r = 2, 1
    lens = [6 * R, 12 * R]
    c = dict(lens=lens, R=R, r=r, hq=4, hkv=2, d=8, mask=mask, sink=2, window=5,
             bounds=[[2 * R, 4 * R, 6 * R], [4 * R, 8 * R, 12 * R]])
    w = _wl(c, dv=6)
    q, k, v, do_full = synth.random_tensors(w, 35)
    cu = [int(x) for x in w.cu_seqlens]
    loc = rank_local_positions(cu, R, r)
    sel = [1, 2, 3, 7, 8, 13, 17]  # local rows, spread over both sub-sequences
    scale = 0.4
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    G = w.hq // w.hkv
    outs = []
    for i in range(len(cu) - 1):
        s0, s1 = cu[i], cu[i + 1]
        M = _torch_mask(mask, s1 - s0, None if w.branch_bounds is None else w.branch_bounds[i])
        Q = tq[s0:s1].permute(1, 0, 2)
        K = tk[s0:s1].permute(1, 0, 2).repeat_interleave(G, dim=0)
        V = tv[s0:s1].permute(1, 0, 2).repeat_interleave(G, dim=0)
        outs.append(torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, attn_mask=M, scale=scale).permute(1, 0, 2))
    O = torch.cat(outs, 0)
    dO_full = torch.zeros_like(O)
    toks = [loc[n] for n in sel]
    dO_full[toks] = torch.tensor(do_full[toks], dtype=torch.float64)
    (O * dO_full).sum().backward()
    do_loc = np.asarray(do_full[loc], dtype=np.float64)
    for block in (None, 1, 2, 5):
        dq, dk, dv = oracle.bwd_ref(w, q, k, v, do_loc, scale, rows=sel, block=block)
        row_of = rank_major_row_of_position(cu, R)
        np.testing.assert_allclose(dq[sel], tq.grad.numpy()[toks], atol=1e-11)
        others = np.setdiff1d(np.arange(len(loc)), sel)
        assert (dq[others] == 0).all()
        np.testing.assert_allclose(dk[row_of], tk.grad.numpy(), atol=1e-11)
        np.testing.assert_allclose(dv[row_of], tv.grad.numpy(), atol=1e-11)
