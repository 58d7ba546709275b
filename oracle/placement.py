"""Data blocks, computation blocks and communication volumes of a block placement.

TEST INFRASTRUCTURE ONLY (see the package docstring).

DCP paper, section 4.1: every sequence is cut along its length into blocks of
``B`` tokens; the Q, K/V and O rows of one block are data blocks that live on
one device (all heads together here: a token's heads are produced on the device
that holds the token).  A computation block pairs a Q block with a K/V block of
the same sequence and exists only where the mask between them is not all zero;
it contributes to the O block of its Q block.

Two volumes are defined on an assignment of data and computation blocks to
devices:

* the per-computation-block volume of section 4.1: for every computation
  block, the sizes of its input blocks (Q, K/V) and output block (O) that live
  on another device;
* the connectivity of the page's hypergraph (one hyperedge per data block,
  joining it to the computation blocks that read or write it): the sum over
  data blocks of size * (devices spanned - 1), the bytes moved when a device
  fetches a remote block once and reuses it.

Per-device send / receive bytes follow the connectivity: an input block is sent
by its owner to every other device that computes with it; a partial output
block is sent back to its owner by every other device that contributes to it.

Parity: pinned (tests/test_oracle_placement.py -- the page's Fig. 9 / Fig. 12
example under the shared question mask, hand-computed volumes of small
placements, the pure-DP placement of Fig. 10 at zero volume, pair counts
against closed forms).
"""
from __future__ import annotations

import numpy as np

from .masks import mask_ref


def blocks_ref(cu, B, kind="causal", sink=0, window=0, bounds=None, mask_block=0):
    """(data, comp): data = [(seq, first token, tokens)], comp = {(seq, qb, kb): pairs}.

    ``bounds`` is a list of shared-prefix bounds per sequence (or None)."""
    cu = [int(x) for x in cu]
    data, comp = [], {}
    for i in range(len(cu) - 1):
        L = cu[i + 1] - cu[i]
        M = mask_ref(kind, L, sink, window, None if bounds is None else bounds[i], mask_block)
        nb = -(-L // B)
        for b in range(nb):
            data.append((i, b * B, min(B, L - b * B)))
        for qb in range(nb):
            for kb in range(nb):
                n = int(M[qb * B:(qb + 1) * B, kb * B:(kb + 1) * B].sum())
                if n:
                    comp[(i, qb, kb)] = n
    return data, comp


def volumes_ref(data_dev, comp_dev, sizes, n_devices):
    """Loads and volumes of an assignment.

    ``data_dev``: {(seq, block): (tokens, device)}; ``comp_dev``: {(seq, qb, kb):
    (pairs, device)}; ``sizes`` = (q_row, kv_row, o_row) bytes per token.
    Returns a dict of numpy arrays / ints."""
    q_row, kv_row, o_row = sizes
    R = n_devices
    tokens = np.zeros(R, np.int64)
    pairs = np.zeros(R, np.int64)
    for (tok, dev) in data_dev.values():
        tokens[dev] += tok
    # per-computation-block volume (section 4.1)
    block_volume = 0
    users_q, users_kv = {}, {}
    for (i, qb, kb), (n, dev) in comp_dev.items():
        pairs[dev] += n
        qtok, qdev = data_dev[(i, qb)]
        ktok, kdev = data_dev[(i, kb)]
        inputs = [(qtok * q_row, qdev), (ktok * kv_row, kdev)]
        outputs = [(qtok * o_row, qdev)]
        for size, home in inputs + outputs:
            if home != dev:
                block_volume += size
        users_q.setdefault((i, qb), set()).add(dev)
        users_kv.setdefault((i, kb), set()).add(dev)
    # connectivity of the hypergraph: one hyperedge per Q, K/V and O data block
    connectivity = 0
    send = np.zeros(R, np.int64)
    recv = np.zeros(R, np.int64)
    for key, (tok, home) in data_dev.items():
        for row, users, is_output in ((q_row, users_q, False), (kv_row, users_kv, False),
                                      (o_row, users_q, True)):
            span = set(users.get(key, set())) | {home}
            size = tok * row
            connectivity += size * (len(span) - 1)
            for dev in span - {home}:
                if is_output:
                    send[dev] += size
                    recv[home] += size
                else:
                    send[home] += size
                    recv[dev] += size
    return {"tokens": tokens, "pairs": pairs, "block_volume": int(block_volume),
            "connectivity": int(connectivity), "send": send, "recv": recv}


def share_fwd_ref(w, q, k, v, B, comp_dev, device, scale=None):
    """Forward of one device's share of a placement, from the definition.

    DCP paper, section 4.1: a computation block (sequence i, Q block qb, K/V
    block kb) is the attention of the query rows of block qb against the keys
    of block kb; a device computes the blocks assigned to it, and the partial
    results of the blocks that feed one output block are reduced (Fig. 9(b)).
    A device's share for Q block (i, qb) is therefore masked softmax attention
    of those rows over the keys of every K/V block kb with (i, qb, kb) on that
    device: S = scale * Q K^T, S[~(M and key in the device's blocks)] = -inf,
    softmax, O = P V, LSE = log sum exp.  Merging all devices' shares of an
    output block by log-sum-exp gives unsplit attention.

    ``w``: the batch (cu_seqlens, heads, mask; unsplit); q, k, v the packed
    tensors [T, H, D]; ``comp_dev``: {(seq, qb, kb): device}.  Returns o
    [T, Hq, Dv] and lse [Hq, T] (float64), NaN at rows of Q blocks the device
    has no computation block for.
    """
    from .attention import default_scale, softmax_rows_ref
    scale = default_scale(w.d_qk) if scale is None else float(scale)
    G = w.hq // w.hkv
    cu = [int(x) for x in w.cu_seqlens]
    T = cu[-1]
    o = np.full((T, w.hq, w.d_v), np.nan)
    lse = np.full((w.hq, T), np.nan)
    mine = {}
    for (i, qb, kb), dev in comp_dev.items():
        if dev == device:
            mine.setdefault((i, qb), []).append(kb)
    for (i, qb), kbs in sorted(mine.items()):
        s0, L = cu[i], cu[i + 1] - cu[i]
        rows = np.arange(qb * B, min(L, (qb + 1) * B))
        bounds = None if w.branch_bounds is None else w.branch_bounds[i]
        M = mask_ref(w.mask, L, w.sink, w.window, bounds, getattr(w, "block", 0))[rows]
        keys = np.zeros(L, dtype=bool)
        for kb in kbs:
            keys[kb * B: (kb + 1) * B] = True
        M = M & keys[None, :]
        Q = np.asarray(q[s0 + rows], dtype=np.float64)
        K = np.asarray(k[s0: s0 + L], dtype=np.float64)
        V = np.asarray(v[s0: s0 + L], dtype=np.float64)
        for h in range(w.hq):
            P, l = softmax_rows_ref(scale * (Q[:, h] @ K[:, h // G].T), M)
            o[s0 + rows, h] = P @ V[:, h // G]
            lse[h, s0 + rows] = l
    return o, lse
