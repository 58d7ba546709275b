"""Pins for the oracle's attention dropout (CPU only).

* Philox4x32-10 against its published known-answer vectors
  (tests/golden/philox4x32_10_kat.txt);
* the keep decision's statistics: realised drop fraction t / 256, independence
  across heads, sequences, seeds and the 4 x 4 blocks one generator call covers,
  and E[D * s] = 1 (unbiased output over many seeds);
* p = 0 is plain attention, bit for bit;
* the backward against torch float64 autograd through the defining forward
  expression (softmax, times the 0/1 mask and the scale, times V) and against
  central finite differences;
* the mask follows in-sequence positions: every CP rank's rows equal unsplit
  attention's rows, and the ranks' dK/dV partials add up to the unsplit ones.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.dropout import keep_mask, keep_scale, philox4x32_10, random_bytes, threshold
from oracle.split import rank_local_positions, rank_major_row_of_position
from tests.test_oracle_attention import _wl
from tests.test_oracle_backward import _torch_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        x = [int(t, 16) for t in r]
        out = philox4x32_10(*x[:4], *x[4:6])
        assert [int(o) for o in out] == x[6:10], r


def test_threshold_and_scale():
    assert threshold(0.0) == 0 and keep_scale(0.0) == 1.0
    assert threshold(0.5) == 128 and keep_scale(0.5) == 2.0
    assert threshold(0.1) == 26 and keep_scale(0.1) == 256.0 / 230.0
    assert threshold(0.999) == 255
    for bad in (-0.1, 1.0, 1.5):
        with pytest.raises(ValueError):
            threshold(bad)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.85])
def test_drop_fraction(p):
    q = np.arange(512)
    k = np.arange(768)
    n = 0
    kept = 0
    for seq, head in ((0, 0), (3, 7)):
        D = keep_mask(seq, head, q, k, p, seed=12345)
        n += D.size
        kept += int(D.sum())
    pe = threshold(p) / 256.0
    sd = np.sqrt(n * pe * (1 - pe))
    assert abs((n - kept) - n * pe) < 6 * sd


def test_bytes_uniform_and_blocks_distinct():
    b = random_bytes(2, 1, np.arange(256), np.arange(256), seed=99).astype(np.int64)
    hist = np.bincount(b.ravel(), minlength=256)
    e = b.size / 256.0
    chi2 = float(((hist - e) ** 2 / e).sum())
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)  # 255 degrees of freedom
    # within every 4 x 4 block the 16 bytes are 16 different bytes of one
    # 128-bit output, not one byte repeated
    blk = b.reshape(64, 4, 64, 4).transpose(0, 2, 1, 3).reshape(-1, 16)
    assert (np.array([len(set(r)) for r in blk]) >= 10).all()


def test_independent_across_heads_sequences_seeds():
    q, k = np.arange(256), np.arange(256)
    p = 0.5
    base = keep_mask(0, 0, q, k, p, seed=7)
    for other in (keep_mask(0, 1, q, k, p, seed=7), keep_mask(1, 0, q, k, p, seed=7),
                  keep_mask(0, 0, q, k, p, seed=8), keep_mask(0, 0, q, k, p, seed=7 + (1 << 32))):
        agree = float((base == other).mean())
        assert abs(agree - 0.5) < 6 * np.sqrt(0.25 / base.size)


def test_p0_is_plain_attention():
    w = _wl(dict(lens=[12, 20], R=2, r=1, hq=4, hkv=2, d=8, mask="causal"))
    q, k, v, do = synth.random_tensors(w, 5)
    o0, l0 = oracle.fwd_ref(w, q, k, v)
    o1, l1 = oracle.fwd_ref(w, q, k, v, dropout=(0.0, 77))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    loc = rank_local_positions([int(x) for x in w.cu_seqlens], 2, 1)
    g0 = oracle.bwd_ref(w, q, k, v, do[loc])
    g1 = oracle.bwd_ref(w, q, k, v, do[loc], dropout=(0.0, 77))
    for a, b in zip(g0, g1):
        assert np.array_equal(a, b)


def test_unbiased_over_seeds():
    """E over seeds of the dropped output is the undropped output: the mean of
    400 draws stays within 6 standard errors of it, elementwise."""
    w = _wl(dict(lens=[16, 24], R=1, r=0, hq=2, hkv=1, d=4, mask="causal"))
    q, k, v = synth.random_tensors(w, 6, with_dout=False)
    o_ref, _ = oracle.fwd_ref(w, q, k, v)
    draws = np.stack([oracle.fwd_ref(w, q, k, v, dropout=(0.3, s))[0] for s in range(400)])
    mean, se = draws.mean(0), draws.std(0) / np.sqrt(len(draws))
    assert (np.abs(mean - o_ref) <= 6 * se + 1e-12).all()
    assert not np.allclose(draws[0], o_ref)


def _torch_dropout_attention(w, q, k, v, p, seed, scale):
    """The defining expression in torch float64: softmax rows, times the 0/1 keep
    mask and 1 / (1 - realised p), times V; per sequence and head."""
    cu = [int(x) for x in w.cu_seqlens]
    G = w.hq // w.hkv
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    outs = []
    for i in range(len(cu) - 1):
        s0, s1 = cu[i], cu[i + 1]
        L = s1 - s0
        M = _torch_mask(w.mask, L, None if w.branch_bounds is None else w.branch_bounds[i])
        heads = []
        for h in range(w.hq):
            S = scale * tq[s0:s1, h] @ tk[s0:s1, h // G].T
            P = torch.softmax(S.masked_fill(~M, float("-inf")), dim=1)
            D = torch.tensor(keep_mask(i, h, np.arange(L), np.arange(L), p, seed), dtype=torch.float64)
            heads.append((P * D * keep_scale(p)) @ tv[s0:s1, h // G])
        outs.append(torch.stack(heads, 1))
    return (tq, tk, tv), torch.cat(outs, 0)


@pytest.mark.parametrize("mask", ["causal", "lambda", "shared_prefix"])
@pytest.mark.parametrize("R,r", [(1, 0), (2, 1)])
def test_against_torch_autograd(mask, R, r):
    c = dict(lens=[6 * R, 12 * R], R=R, r=r, hq=4, hkv=2, d=8, mask=mask, sink=2, window=5,
             bounds=[[2 * R, 4 * R, 6 * R], [4 * R, 8 * R, 12 * R]])
    w = _wl(c)
    q, k, v, do_full = synth.random_tensors(w, 31)
    cu = [int(x) for x in w.cu_seqlens]
    loc = rank_local_positions(cu, R, r)
    p, seed, scale = 0.4, 2024, 0.45
    (tq, tk, tv), O = _torch_dropout_attention(w, q, k, v, p, seed, scale)
    o, _ = oracle.fwd_ref(w, q, k, v, scale, dropout=(p, seed))
    np.testing.assert_allclose(o, O.detach().numpy()[loc], atol=1e-12)
    dO = torch.zeros_like(O)
    dO[loc] = torch.tensor(do_full[loc], dtype=torch.float64)
    (O * dO).sum().backward()
    dq, dk, dv = oracle.bwd_ref(w, q, k, v, do_full[loc], scale, dropout=(p, seed))
    row_of = rank_major_row_of_position(cu, R)
    np.testing.assert_allclose(dq, tq.grad.numpy()[loc], atol=1e-11)
    np.testing.assert_allclose(dk[row_of], tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv[row_of], tv.grad.numpy(), atol=1e-11)


def test_finite_differences():
    w = _wl(dict(lens=[8, 12], R=2, r=0, hq=2, hkv=1, d=3, mask="causal"))
    q, k, v, do_full = [x.astype(np.float64) for x in synth.random_tensors(w, 41)]
    cu = [int(x) for x in w.cu_seqlens]
    loc = rank_local_positions(cu, 2, 0)
    drop = (0.35, 5)
    dq, dk, dv = oracle.bwd_ref(w, q, k, v, do_full[loc], 0.7, dropout=drop)
    row_of = rank_major_row_of_position(cu, 2)

    def loss(q, k, v):
        return float((oracle.fwd_ref(w, q, k, v, 0.7, dropout=drop)[0] * do_full[loc]).sum())

    eps = 1e-6
    rng = np.random.default_rng(3)
    for name, X in (("q", q), ("k", k), ("v", v)):
        for _ in range(10):
            idx = tuple(int(rng.integers(0, s)) for s in X.shape)
            a = dict(q=q, k=k, v=v)
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            num = (loss(**dict(a, **{name: Xp})) - loss(**dict(a, **{name: Xm}))) / (2 * eps)
            if name == "q":
                ana = dq[loc.index(idx[0]), idx[1], idx[2]] if idx[0] in loc else 0.0
            else:
                ana = (dk if name == "k" else dv)[row_of[idx[0]], idx[1], idx[2]]
            assert abs(num - ana) < 1e-7, (name, idx, num, ana)


@pytest.mark.parametrize("R", [2, 3])
def test_ranks_equal_unsplit(R):
    """The mask is a function of in-sequence positions: each rank's dropped
    rows are the unsplit dropped rows, and the ranks' rank-major dK/dV partials
    add up to the unsplit gradients."""
    c = dict(lens=[2 * R * 3, 2 * R * 5], R=R, r=0, hq=2, hkv=1, d=4, mask="lambda", sink=1, window=4)
    w1 = _wl(dict(c, R=1))
    q, k, v, do_full = synth.random_tensors(w1, 45)
    cu = [int(x) for x in w1.cu_seqlens]
    drop = (0.25, 31337)
    o1, l1 = oracle.fwd_ref(w1, q, k, v, dropout=drop)
    dq1, dk1, dv1 = oracle.bwd_ref(w1, q, k, v, do_full, dropout=drop)
    dk_sum, dv_sum = np.zeros_like(dk1), np.zeros_like(dv1)
    for r in range(R):
        w = _wl(dict(c, r=r))
        loc = rank_local_positions(cu, R, r)
        o, l = oracle.fwd_ref(w, q, k, v, dropout=drop)
        np.testing.assert_allclose(o, o1[loc], atol=1e-13)
        dq, dk, dv = oracle.bwd_ref(w, q, k, v, do_full[loc], dropout=drop)
        np.testing.assert_allclose(dq, dq1[loc], atol=1e-12)
        dk_sum += dk
        dv_sum += dv
    row_of = rank_major_row_of_position(cu, R)
    np.testing.assert_allclose(dk_sum[row_of], dk1, atol=1e-12)
    np.testing.assert_allclose(dv_sum[row_of], dv1, atol=1e-12)
