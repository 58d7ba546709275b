"""The symmetric context-parallel split and its metadata, by plain enumeration.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: MindSpeed RFC "KVAllGather CP: EOD-aware load balancing for THD"
(gitcode Ascend/MindSpeed issue 232):

* section 2 (use cases): every EOD sub-sequence is cut into 2*CP equal chunks;
  rank r holds chunk r and chunk 2*CP-r-1; the per-rank workload is
  sum(q_len*kv_len) and must be equal on every rank.
* section 3.1: each rank all-gathers its local K/V, giving a rank-major K/V;
  a direct index selects every local Q chunk's causal K/V prefix from it; the
  metadata builder returns local and global token counts, actual_seq_qlen and
  actual_seq_kvlen, and that index.
* glossary: rank-major means the all-gather result concatenated in rank order.

Readings taken where the page is silent:

* a rank's local layout is sub-sequence by sub-sequence, and inside each the
  earlier chunk (r) comes first, then chunk 2R-1-r;
* actual_seq_qlen / actual_seq_kvlen are cumulative with a leading 0, one entry
  per (sub-sequence, chunk) segment in local order;
* a segment of chunk j holds query positions j*c .. (j+1)*c-1 of its
  sub-sequence and its K/V prefix is positions 0 .. (j+1)*c-1 (causal,
  bottom-right aligned), listed in position order.

Everything here is computed by walking positions one at a time; nothing uses a
closed form for the index.

Parity: pinned (tests/test_oracle_metadata.py -- hand-derived values for the
[0,64,192,256] example, closed-form counts, permutation and position-tagging
invariants, workload equality for R=2 and R=4).
"""
from __future__ import annotations

import numpy as np


def _check(cu, R, r):
    cu = [int(x) for x in cu]
    if R < 1 or not (0 <= r < R):
        raise AssertionError("bad cp_size / rank")
    if len(cu) < 2 or cu[0] != 0:
        raise AssertionError("cu_seqlens must start at 0 and hold at least one sub-sequence")
    for a, b in zip(cu[:-1], cu[1:]):
        if b - a <= 0:
            raise AssertionError("sub-sequence lengths must be positive")
        if (b - a) % (2 * R) != 0:
            raise AssertionError("sub-sequence length must be divisible by 2*cp_size")
    return cu


def _chunks_of_rank(R, r):
    """The two chunk ids a rank holds, in local order."""
    return [r, 2 * R - 1 - r]


def rank_local_positions(cu, R, r):
    """Packed (global) token ids that rank r holds, in its local order."""
    cu = _check(cu, R, r)
    out = []
    for i in range(len(cu) - 1):
        L = cu[i + 1] - cu[i]
        c = L // (2 * R)
        for j in _chunks_of_rank(R, r):
            for a in range(c):
                out.append(cu[i] + j * c + a)
    return out


def rank_major_order(cu, R):
    """Packed token id held at each row of the rank-major gathered buffer."""
    order = []
    for s in range(R):
        order.extend(rank_local_positions(cu, R, s))
    return order


def rank_major_row_of_position(cu, R):
    """Inverse of :func:`rank_major_order`: row of every packed token id."""
    order = rank_major_order(cu, R)
    inv = [-1] * len(order)
    for row, tok in enumerate(order):
        inv[tok] = row
    return inv


def metadata_ref(cu, R, r):
    """Metadata of rank r, built by enumeration.

    Returns a dict with int64 numpy arrays:
      local_tokens, global_tokens, local_cu [n+1], actual_seq_qlen [2n+1],
      actual_seq_kvlen [2n+1], kv_index [sum kv_len], seg_q_pos0 [2n],
      workload_per_rank [R].
    """
    cu = _check(cu, R, r)
    n = len(cu) - 1
    row_of = rank_major_row_of_position(cu, R)
    q_cum, kv_cum, kv_index, q_pos0, local_cu = [0], [0], [], [], [0]
    local_count = 0
    for i in range(n):
        L = cu[i + 1] - cu[i]
        c = L // (2 * R)
        for j in _chunks_of_rank(R, r):
            q_len = c
            kv_len = (j + 1) * c
            q_cum.append(q_cum[-1] + q_len)
            kv_cum.append(kv_cum[-1] + kv_len)
            q_pos0.append(j * c)
            for p in range(kv_len):
                kv_index.append(row_of[cu[i] + p])
            local_count += q_len
        local_cu.append(local_count)
    return {
        "local_tokens": local_count,
        "global_tokens": cu[-1],
        "local_cu": np.array(local_cu, dtype=np.int64),
        "actual_seq_qlen": np.array(q_cum, dtype=np.int64),
        "actual_seq_kvlen": np.array(kv_cum, dtype=np.int64),
        "kv_index": np.array(kv_index, dtype=np.int64),
        "seg_q_pos0": np.array(q_pos0, dtype=np.int64),
        "workload_per_rank": np.array([workload_ref(cu, R, s) for s in range(R)], dtype=np.int64),
    }


def workload_ref(cu, R, s):
    """sum(q_len * kv_len) over rank s's segments (RFC section 2, load balance)."""
    cu = _check(cu, R, s)
    w = 0
    for i in range(len(cu) - 1):
        c = (cu[i + 1] - cu[i]) // (2 * R)
        for j in _chunks_of_rank(R, s):
            w += c * ((j + 1) * c)
    return w
