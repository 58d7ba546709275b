"""Attention masks, materialised as boolean matrices.

TEST INFRASTRUCTURE ONLY (see the package docstring).

M[q, k] is True when query position q may attend to key position k of the same
sub-sequence (positions count from the start of the sub-sequence, so every
sub-sequence restarts its mask: the EOD reset of the MindSpeed RFC, section 2).

* causal        -- k <= q.
* lambda        -- causal, restricted to the first ``sink`` tokens (attention
                   sink) plus a sliding window of the ``window`` most recent
                   tokens, the diagonal included (DCP paper, sparse masks,
                   Fig. 6(b); evaluation: 64 sink tokens and window 4096).
* blockwise     -- causal blockwise: the sequence is cut into blocks of
                   ``block`` tokens; a query sees, causally, the first ``sink``
                   blocks (attention sink) and the ``window`` blocks ending with
                   its own block; a query of the last block (the test example)
                   sees every earlier token (DCP paper, sparse masks, Fig. 6(c);
                   evaluation: block 256, window 2 blocks, one sink block, one
                   test block).
* shared_prefix -- one shared question followed by several answers; the
                   question is causal, every answer sees the whole question and
                   itself causally, never another answer (DCP paper, Fig. 6(d)
                   "shared question mask").  ``bounds`` = [prefix_end,
                   end_of_answer_0, ..., end_of_answer_{B-1}].

Parity: pinned (tests/test_oracle_masks.py -- hand-written small matrices,
reductions to the causal mask in the degenerate settings, pair counts against
closed forms).
"""
from __future__ import annotations

import numpy as np


def mask_rows_ref(kind, L, rows, sink=0, window=0, bounds=None, block=0):
    """Mask rows ``rows`` (query positions) of a length-L sub-sequence: bool [len(rows), L]."""
    q = np.asarray(rows, dtype=np.int64)[:, None]
    k = np.arange(L, dtype=np.int64)[None, :]
    causal = k <= q
    if kind == "causal":
        return causal
    if kind == "lambda":
        return causal & ((k < sink) | (q - k < window))
    if kind == "blockwise":
        bq, bk = q // block, k // block
        test = bq == (L - 1) // block
        return causal & (test | (bk < sink) | (bq - bk < window))
    if kind == "shared_prefix":
        b = [int(x) for x in bounds]
        P = b[0]
        M = np.zeros((q.shape[0], L), dtype=bool)
        for n, qq in enumerate(q[:, 0]):
            if qq < P:
                M[n, : qq + 1] = True
                continue
            start = P
            for end in b[1:]:
                if qq < end:
                    M[n, :P] = True
                    M[n, start: qq + 1] = True
                    break
                start = end
        return M
    raise ValueError(f"unknown mask {kind}")


def mask_ref(kind, L, sink=0, window=0, bounds=None, block=0):
    """Full [L, L] mask of one sub-sequence."""
    return mask_rows_ref(kind, L, np.arange(L), sink, window, bounds, block)


def visible_pairs_ref(workload, rows_by_seq=None, block=2048):
    """Number of visible (query, key) pairs on the rank's local rows, per head.

    ``rows_by_seq`` maps sub-sequence i to the in-sequence query positions the
    rank holds; by default they come from the oracle's own split.
    """
    from .split import rank_local_positions
    cu = [int(x) for x in workload.cu_seqlens]
    if rows_by_seq is None:
        loc = rank_local_positions(cu, workload.cp_size, workload.rank)
        rows_by_seq = {}
        for tok in loc:
            i = int(np.searchsorted(cu, tok, side="right") - 1)
            rows_by_seq.setdefault(i, []).append(tok - cu[i])
    total = 0
    for i, rows in rows_by_seq.items():
        L = cu[i + 1] - cu[i]
        bounds = None if workload.branch_bounds is None else workload.branch_bounds[i]
        rows = np.asarray(rows)
        for s in range(0, len(rows), block):
            M = mask_rows_ref(workload.mask, L, rows[s: s + block], workload.sink,
                              workload.window, bounds, getattr(workload, "block", 0))
            total += int(M.sum())
    return total
