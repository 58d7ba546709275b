"""fp64 CPU oracle for one context-parallel rank's share of packed varlen attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes anything here: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` do.  The oracle shares no code with the HIP
path; the only thing the two have in common is the seeded input generator in
``synth``.

What it computes, written the plain way (numpy float64, boolean masks
materialised, softmax taken directly):

* ``split``     -- the symmetric 2R-chunk split of every EOD sub-sequence and the
                   rank-major layout of gathered K/V, by enumerating positions
                   (MindSpeed RFC on EOD load-balanced KVAllGather CP, section 2
                   "use cases": chunking rule; section 3.1: rank-major AllGather
                   and the causal-prefix index; glossary: "rank-major").
* ``metadata_ref`` -- token counts, actual_seq_qlen / actual_seq_kvlen, the
                   causal-prefix KV index and the per-rank workload
                   sum(q_len*kv_len) (RFC section 3.1 and interface
                   get_thd_load_balanced_cp_metadata, section 3.5.2.1).
* ``mask_ref``  -- causal (EOD reset), lambda (sink + sliding window) and
                   shared-prefix masks (DCP paper, section on sparse attention
                   masks, Fig. 6 (b) and (d); evaluation "Attention Masks").
* ``placement`` -- data and computation blocks of a batch and the
                   communication volumes of an assignment of them to devices
                   (DCP paper, section 4.1 and its placement model).
* ``fwd_ref`` / ``bwd_ref`` -- masked softmax attention and its gradients on the
                   rank's local rows, K/V read from the unsplit tensors (DCP
                   paper, background: masked self-attention; RFC section 1.3:
                   outputs and Q/K/V gradients equal non-CP attention), with
                   optional attention dropout.
* ``dropout``   -- the dropout keep mask of every (sequence, head, query, key)
                   from Philox4x32-10 (RFC section 3.5.2.2: attention_dropout).

Parity status of each function is stated in its docstring; every one of them
is pinned by tests under ``tests/test_oracle_*.py``.
"""
from .split import (rank_local_positions, rank_major_order, rank_major_row_of_position,
                    metadata_ref, workload_ref)
from .masks import mask_ref, visible_pairs_ref
from .attention import fwd_ref, bwd_ref, fwd_full_ref, softmax_rows_ref
from .dropout import philox4x32_10, keep_mask, keep_scale, threshold

__all__ = [
    "rank_local_positions", "rank_major_order", "rank_major_row_of_position",
    "metadata_ref", "workload_ref", "mask_ref", "visible_pairs_ref",
    "fwd_ref", "bwd_ref", "fwd_full_ref", "softmax_rows_ref",
    "philox4x32_10", "keep_mask", "keep_scale", "threshold",
]
