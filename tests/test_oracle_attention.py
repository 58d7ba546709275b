"""Pins for the oracle's forward (CPU only).

* brute force: pure-Python loops (math.exp, no numpy matmul) on tiny shapes;
* library routine: torch float64 scaled_dot_product_attention with an explicit
  boolean mask, per sub-sequence (repeat of K/V heads for GQA);
* softmax rows sum to one;
* closed forms: K = 0 gives the mean of the visible V rows; constant V gives a
  constant output;
* the concatenation of every rank's output (undoing the symmetric split)
  equals unsplit attention (MindSpeed RFC, section 2: CP output equals CP=1).
"""
import math
import random

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.split import rank_local_positions


def _brute(w, q, k, v, scale):
    """Independent slow forward: loops over rows, keys and dims in pure Python."""
    G = w.hq // w.hkv
    cu = [int(x) for x in w.cu_seqlens]
    loc = rank_local_positions(cu, w.cp_size, w.rank)
    o = np.zeros((len(loc), w.hq, w.d_v))
    lse = np.zeros((w.hq, len(loc)))
    for n, tok in enumerate(loc):
        i = max(j for j in range(len(cu) - 1) if cu[j] <= tok)
        p = tok - cu[i]
        L = cu[i + 1] - cu[i]
        for h in range(w.hq):
            g = h // G
            logits = []
            for kk in range(L):
                if w.mask == "causal":
                    vis = kk <= p
                elif w.mask == "lambda":
                    vis = kk <= p and (kk < w.sink or p - kk < w.window)
                else:
                    b = list(w.branch_bounds[i])
                    if p < b[0]:
                        vis = kk <= p
                    else:
                        st = b[0]
                        for e in b[1:]:
                            if p < e:
                                break
                            st = e
                        vis = kk < b[0] or (st <= kk <= p)
                if vis:
                    s = 0.0
                    for d in range(w.d_qk):
                        s += float(q[tok, h, d]) * float(k[cu[i] + kk, g, d])
                    logits.append((kk, s * scale))
            mx = max(s for _, s in logits)
            den = sum(math.exp(s - mx) for _, s in logits)
            lse[h, n] = mx + math.log(den)
            for d in range(w.d_v):
                acc = 0.0
                for kk, s in logits:
                    acc += math.exp(s - mx) / den * float(v[cu[i] + kk, g, d])
                o[n, h, d] = acc
    return o, lse


CASES = [
    dict(lens=[8, 16], R=2, r=0, hq=2, hkv=1, d=4, mask="causal"),
    dict(lens=[8, 16], R=2, r=1, hq=2, hkv=2, d=3, mask="causal"),
    dict(lens=[12, 24], R=3, r=2, hq=4, hkv=2, d=4, mask="causal"),
    dict(lens=[16, 24], R=1, r=0, hq=2, hkv=1, d=4, mask="lambda", sink=2, window=5),
    dict(lens=[16, 24], R=2, r=1, hq=2, hkv=2, d=4, mask="lambda", sink=3, window=4),
    dict(lens=[16, 20], R=1, r=0, hq=2, hkv=1, d=4, mask="shared_prefix",
         bounds=[[4, 10, 16], [8, 12, 16, 20]]),
]


def _wl(c, dtype="fp32", dv=None):
    bb = None
    if "bounds" in c:
        n = max(len(b) for b in c["bounds"])
        bb = np.array([b + [b[-1]] * (n - len(b)) for b in c["bounds"]])
    return synth.custom_workload(c["lens"], c["R"], c["r"], c["hq"], c["hkv"], c["d"],
                                 dv or c["d"], dtype, mask=c["mask"], sink=c.get("sink", 0),
                                 window=c.get("window", 0), branch_bounds=bb)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_brute_force(ci):
    w = _wl(CASES[ci])
    q, k, v = synth.random_tensors(w, ci, with_dout=False)
    scale = 0.37
    o, lse = oracle.fwd_ref(w, q, k, v, scale)
    ob, lb = _brute(w, q, k, v, scale)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


def _torch_sdpa_full(w, q, k, v, scale):
    """torch float64 SDPA per sub-sequence with an explicit mask, packed order."""
    G = w.hq // w.hkv
    cu = [int(x) for x in w.cu_seqlens]
    out = np.zeros((cu[-1], w.hq, w.d_v))
    for i in range(len(cu) - 1):
        s0, s1 = cu[i], cu[i + 1]
        L = s1 - s0
        bounds = None if w.branch_bounds is None else w.branch_bounds[i]
        # the mask is built here from scratch (not the oracle's) as an index test
        qq = torch.arange(L)[:, None]
        kk = torch.arange(L)[None, :]
        if w.mask == "causal":
            M = kk <= qq
        elif w.mask == "lambda":
            M = (kk <= qq) & ((kk < w.sink) | (qq - kk < w.window))
        else:
            M = torch.zeros(L, L, dtype=torch.bool)
            P = int(bounds[0])
            M[:P, :P] = torch.tril(torch.ones(P, P, dtype=torch.bool))
            st = P
            for e in bounds[1:]:
                e = int(e)
                M[st:e, :P] = True
                M[st:e, st:e] = torch.tril(torch.ones(e - st, e - st, dtype=torch.bool))
                st = e
        Q = torch.from_numpy(np.asarray(q[s0:s1], np.float64)).permute(1, 0, 2)
        K = torch.from_numpy(np.asarray(k[s0:s1], np.float64)).permute(1, 0, 2)
        V = torch.from_numpy(np.asarray(v[s0:s1], np.float64)).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0)
        V = V.repeat_interleave(G, dim=0)
        O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=M, scale=scale)
        out[s0:s1] = O.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_torch_sdpa(ci):
    c = dict(CASES[ci])
    c["d"] = 16
    w = _wl(c, dv=12)
    q, k, v = synth.random_tensors(w, 10 + ci, with_dout=False)
    scale = 1 / math.sqrt(16)
    full = _torch_sdpa_full(w, q, k, v, scale)
    o, _ = oracle.fwd_ref(w, q, k, v, scale)
    loc = rank_local_positions([int(x) for x in w.cu_seqlens], w.cp_size, w.rank)
    np.testing.assert_allclose(o, full[loc], rtol=1e-12, atol=1e-12)


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(0)
    for _ in range(20):
        S = rng.standard_normal((13, 29)) * 10
        M = rng.random((13, 29)) < 0.6
        M[:, 0] = True
        P, lse = oracle.softmax_rows_ref(S, M)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert (P[~M] == 0).all()
        np.testing.assert_allclose(lse, np.log(np.where(M, np.exp(S), 0).sum(axis=1)), atol=1e-9)
    P, lse = oracle.softmax_rows_ref(np.zeros((2, 3)), np.zeros((2, 3), bool))
    assert (P == 0).all() and np.isneginf(lse).all()


@pytest.mark.parametrize("mask", ["causal", "lambda", "shared_prefix"])
def test_k_zero_gives_mean_of_visible_v(mask):
    c = dict(lens=[16, 32], R=2, r=1, hq=2, hkv=1, d=4, mask=mask, sink=2, window=5,
             bounds=[[4, 10, 16], [8, 20, 32]])
    w = _wl(c)
    q, k, v = synth.random_tensors(w, 3, with_dout=False)
    k = np.zeros_like(k)
    o, _ = oracle.fwd_ref(w, q, k, v)
    cu = [int(x) for x in w.cu_seqlens]
    for n, tok in enumerate(rank_local_positions(cu, w.cp_size, w.rank)):
        i = 0 if tok < cu[1] else 1
        p = tok - cu[i]
        row = oracle.mask_ref(mask, cu[i + 1] - cu[i], 2, 5, w.branch_bounds[i])[p]
        mean = v[cu[i]: cu[i + 1]][row].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(o[n, 0], mean[0], atol=1e-12)
        np.testing.assert_allclose(o[n, 1], mean[0], atol=1e-12)


def test_constant_v_gives_constant_o():
    w = _wl(CASES[2])
    q, k, v = synth.random_tensors(w, 4, with_dout=False)
    v = np.full_like(v, 0.625)
    o, _ = oracle.fwd_ref(w, q, k, v)
    np.testing.assert_allclose(o, 0.625, atol=1e-12)


@pytest.mark.parametrize("R", [1, 2, 4])
@pytest.mark.parametrize("mask", ["causal", "lambda", "shared_prefix"])
def test_concat_of_ranks_equals_unsplit(R, mask):
    rng = random.Random(R)
    lens = [2 * R * rng.randint(1, 6) for _ in range(3)]
    bounds = []
    for L in lens:
        P = L // 3
        b = [P, P + (L - P) // 2, L]
        bounds.append(b)
    c = dict(lens=lens, R=R, r=0, hq=4, hkv=2, d=8, mask=mask, sink=2, window=6, bounds=bounds)
    full_w = _wl(dict(c, R=1, r=0))
    q, k, v = synth.random_tensors(full_w, 5, with_dout=False)
    of, lf = oracle.fwd_full_ref(full_w, q, k, v)
    cu = [int(x) for x in full_w.cu_seqlens]
    o_cat = np.zeros_like(of)
    l_cat = np.zeros_like(lf)
    for r in range(R):
        w = _wl(dict(c, r=r))
        o, l = oracle.fwd_ref(w, q, k, v)
        loc = rank_local_positions(cu, R, r)
        o_cat[loc] = o
        l_cat[:, loc] = l
    np.testing.assert_allclose(o_cat, of, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l_cat, lf, rtol=1e-12, atol=1e-12)


def test_sampled_rows_match_full():
    w = _wl(CASES[2])
    q, k, v = synth.random_tensors(w, 6, with_dout=False)
    o, l = oracle.fwd_ref(w, q, k, v)
    rows = [0, 3, 7, 11]
    o2, l2 = oracle.fwd_ref(w, q, k, v, rows=rows)
    np.testing.assert_allclose(o2[rows], o[rows], atol=1e-13)
    np.testing.assert_allclose(l2[:, rows], l[:, rows], atol=1e-13)
    assert np.isnan(o2[1]).all()
