"""Masked softmax attention and its gradients, fp64, on one CP rank's local rows.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition (DCP paper, background section: standard masked self-attention with
a boolean mask M that removes unwanted query/key interactions; the printed
formula is missing from the page, so the plain reading is used): for every
sub-sequence, query head h and its K/V head h // G (grouped-query attention with
contiguous groups, G = Hq / Hkv),

    S = scale * Q K^T,   S[~M] = -inf,   P = softmax_rows(S),   O = P V,
    LSE = log(sum_k exp(S[q, k])).

The block-wise online-softmax evaluation the kernels use reaches the same
values up to rounding (DCP paper, background: the online softmax trick), and the
RFC requires the CP result to equal non-CP attention for outputs and Q/K/V
gradients (MindSpeed RFC section 1.3 and section 2, correctness).  So the oracle
is simply that definition: each local query row against *all* keys of its own
sub-sequence, K/V taken from the unsplit tensors -- never through the
rank-major index, which keeps it independent of the metadata path.

Backward (standard softmax Jacobian, no recomputation tricks): with dO given on
the local rows (zero on every other row),

    dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dP * P)),
    dQ = scale * dS K,  dK = scale * dS^T Q,

summed over the G query heads of a group for dK and dV, and placed in the
rank-major order of gathered K/V (RFC section 3.1: backward index_add_ of dK/dV
into the rank-major gradient buffer) through the oracle's own enumeration of
positions.  Rows no local query sees stay zero.

A query row that sees no key gets O = 0, LSE = -inf and dQ = 0 (unreachable for
the masks here, every row sees itself).

With ``dropout=(p, seed)`` both directions apply the attention dropout of
``oracle.dropout`` (keep mask D from Philox4x32-10 at the pair's in-sequence
positions): O = (D * P * s) V with s = 1 / (1 - realised p), the LSE of the
undropped softmax; dV = (D * P * s)^T dO and dP = D * s * (dO V^T) in the
Jacobian above.

Parity: pinned (tests/test_oracle_attention.py -- pure-Python brute force,
torch float64 scaled_dot_product_attention with an explicit mask, softmax rows
summing to one, closed forms, concatenation of all ranks against unsplit
attention; tests/test_oracle_backward.py -- central finite differences, torch
float64 autograd, sum over ranks of rank-major partial gradients).
"""
from __future__ import annotations

import math

import numpy as np

from .dropout import keep_mask, keep_scale
from .masks import mask_rows_ref
from .split import rank_local_positions, rank_major_row_of_position


def default_scale(d_qk):
    return 1.0 / math.sqrt(d_qk)


def softmax_rows_ref(S, M):
    """Row softmax of S over the entries where M is True; returns (P, LSE)."""
    S = np.where(M, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    E = np.where(M, np.exp(S - m), 0.0)
    l = E.sum(axis=1, keepdims=True)
    P = np.where(l > 0, E / np.where(l > 0, l, 1.0), 0.0)
    lse = np.where(l[:, 0] > 0, m[:, 0] + np.log(np.where(l[:, 0] > 0, l[:, 0], 1.0)), -np.inf)
    return P, lse


def _seq_of(cu, tok):
    return int(np.searchsorted(cu, tok, side="right") - 1)


def _local_rows_by_seq(w, rows=None):
    """{sub-sequence: (local row ids, in-sequence positions)} for the rank's share."""
    cu = np.asarray(w.cu_seqlens, dtype=np.int64)
    loc = rank_local_positions(cu, w.cp_size, w.rank)
    sel = range(len(loc)) if rows is None else sorted(set(int(x) for x in rows))
    groups = {}
    for n in sel:
        tok = loc[n]
        i = _seq_of(cu, tok)
        g = groups.setdefault(i, ([], []))
        g[0].append(n)
        g[1].append(tok - int(cu[i]))
    return loc, groups


def _mask_for(w, i, L, positions):
    bounds = None if w.branch_bounds is None else w.branch_bounds[i]
    return mask_rows_ref(w.mask, L, positions, w.sink, w.window, bounds, getattr(w, "block", 0))


def _dropped(P, dropout, i, h, qpos, L):
    """D * P * s for sequence i, head h (P unchanged without dropout)."""
    if dropout is None:
        return P
    p, seed = dropout
    return np.where(keep_mask(i, h, qpos, np.arange(L), p, seed), P * keep_scale(p), 0.0)


def fwd_ref(w, q, k, v, scale=None, rows=None, block=512, heads=None, dropout=None):
    """Forward on rank (w.cp_size, w.rank)'s local rows.

    q, k, v are the *full unsplit* tensors [T, H, D] (any float dtype; upcast
    to float64).  Returns o [T_loc, Hq, Dv] and lse [Hq, T_loc] as float64;
    when ``rows`` (local row ids) or ``heads`` (query heads) are given only
    those are computed and the rest are NaN.  ``dropout`` = (p, seed) or None.
    """
    scale = default_scale(w.d_qk) if scale is None else float(scale)
    G = w.hq // w.hkv
    cu = np.asarray(w.cu_seqlens, dtype=np.int64)
    loc, groups = _local_rows_by_seq(w, rows)
    T_loc = len(loc)
    o = np.full((T_loc, w.hq, w.d_v), np.nan)
    lse = np.full((w.hq, T_loc), np.nan)
    for i, (lrows, pos) in groups.items():
        s0, L = int(cu[i]), int(cu[i + 1] - cu[i])
        Ki = np.asarray(k[s0: s0 + L], dtype=np.float64)
        Vi = np.asarray(v[s0: s0 + L], dtype=np.float64)
        lrows = np.asarray(lrows)
        pos = np.asarray(pos)
        for b in range(0, len(lrows), block):
            lr, ps = lrows[b: b + block], pos[b: b + block]
            toks = s0 + ps
            Qb = np.asarray(q[toks], dtype=np.float64)
            M = _mask_for(w, i, L, ps)
            for h in (range(w.hq) if heads is None else heads):
                S = scale * (Qb[:, h, :] @ Ki[:, h // G, :].T)
                P, l = softmax_rows_ref(S, M)
                o[lr, h, :] = _dropped(P, dropout, i, h, ps, L) @ Vi[:, h // G, :]
                lse[h, lr] = l
    return o, lse


def fwd_full_ref(w, q, k, v, scale=None, dropout=None):
    """Unsplit attention over every packed token (no CP), o [T, Hq, Dv], lse [Hq, T]."""
    scale = default_scale(w.d_qk) if scale is None else float(scale)
    G = w.hq // w.hkv
    cu = np.asarray(w.cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    o = np.zeros((T, w.hq, w.d_v))
    lse = np.zeros((w.hq, T))
    for i in range(len(cu) - 1):
        s0, L = int(cu[i]), int(cu[i + 1] - cu[i])
        M = _mask_for(w, i, L, np.arange(L))
        Qi = np.asarray(q[s0: s0 + L], dtype=np.float64)
        Ki = np.asarray(k[s0: s0 + L], dtype=np.float64)
        Vi = np.asarray(v[s0: s0 + L], dtype=np.float64)
        for h in range(w.hq):
            P, l = softmax_rows_ref(scale * (Qi[:, h] @ Ki[:, h // G].T), M)
            o[s0: s0 + L, h] = _dropped(P, dropout, i, h, np.arange(L), L) @ Vi[:, h // G]
            lse[h, s0: s0 + L] = l
    return o, lse


def bwd_ref(w, q, k, v, do_local, scale=None, heads=None, rows=None, block=None, dropout=None):
    """Backward on rank (w.cp_size, w.rank)'s share.

    q, k, v: full unsplit tensors.  do_local: [T_loc, Hq, Dv] gradient of the
    local output rows.  Returns dq_local [T_loc, Hq, Dqk] and rank-major
    dk [T, Hkv, Dqk], dv [T, Hkv, Dv], all float64.  ``heads`` restricts the
    work to those query heads (their dQ, and their K/V groups' dK/dV -- complete
    only for groups whose every head is listed); other entries stay zero.

    ``rows`` (local row ids) restricts the work to those query rows: their dQ
    and their share of dK/dV.  dK and dV are sums over query rows of per-row
    terms (the index_add_ of per-segment gradients in MindSpeed RFC section
    3.1), so the shares of disjoint row sets add up to the full gradient.
    ``block`` takes the rows of a sub-sequence that many at a time and adds the
    blocks' shares (the same sum in another order; None: all rows at once).
    ``dropout`` = (p, seed) or None, as in the forward.
    """
    scale = default_scale(w.d_qk) if scale is None else float(scale)
    G = w.hq // w.hkv
    cu = np.asarray(w.cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    loc, groups = _local_rows_by_seq(w, rows)
    dq = np.zeros((len(loc), w.hq, w.d_qk))
    dk_seq = np.zeros((T, w.hkv, w.d_qk))   # packed (unsplit) order first
    dv_seq = np.zeros((T, w.hkv, w.d_v))
    dO = np.asarray(do_local, dtype=np.float64)
    for i, (lrows_all, pos_all) in groups.items():
        s0, L = int(cu[i]), int(cu[i + 1] - cu[i])
        lrows_all, pos_all = np.asarray(lrows_all), np.asarray(pos_all)
        Ki = np.asarray(k[s0: s0 + L], dtype=np.float64)
        Vi = np.asarray(v[s0: s0 + L], dtype=np.float64)
        step = len(lrows_all) if block is None else int(block)
        for b in range(0, len(lrows_all), step):
            lrows, pos = lrows_all[b: b + step], pos_all[b: b + step]
            Qi = np.asarray(q[s0 + pos], dtype=np.float64)
            M = _mask_for(w, i, L, pos)
            for h in (range(w.hq) if heads is None else heads):
                g = h // G
                P, _ = softmax_rows_ref(scale * (Qi[:, h] @ Ki[:, g].T), M)
                dOh = dO[lrows, h, :]
                dv_seq[s0: s0 + L, g] += _dropped(P, dropout, i, h, pos, L).T @ dOh
                dP = dOh @ Vi[:, g].T
                if dropout is not None:  # the dropped entries pass no gradient back
                    dP = np.where(keep_mask(i, h, pos, np.arange(L), *dropout), dP * keep_scale(dropout[0]),
                                  0.0)
                dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
                dq[lrows, h] = scale * (dS @ Ki[:, g])
                dk_seq[s0: s0 + L, g] += scale * (dS.T @ Qi[:, h])
    row_of = rank_major_row_of_position(cu, w.cp_size)
    dk = np.zeros_like(dk_seq)
    dv = np.zeros_like(dv_seq)
    for tok in range(T):
        dk[row_of[tok]] = dk_seq[tok]
        dv[row_of[tok]] = dv_seq[tok]
    return dq, dk, dv
