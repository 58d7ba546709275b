"""Block placement (cva_placement_*), host only.

The assignment is a heuristic of this library (the DCP paper's planner is a
hypergraph partitioner); what is fixed by the page and checked here:
* data and computation blocks (section 4.1) equal the oracle's, built from
  materialised masks, bit for bit;
* every block has exactly one valid device;
* reported token / pair loads, per-device send and receive bytes and both
  communication volumes equal the oracle's recomputation from the assignment;
* the balance constraints of the placement model hold (tokens within one block
  of the mean, visible pairs within (1 + epsilon) of the mean);
* the zig-zag comparison equals the oracle's per-rank pairs.
"""
import numpy as np
import pytest

import context_varlen_attention_amd as cva
import synth
from oracle.masks import visible_pairs_ref
from oracle.placement import blocks_ref, volumes_ref

CASES = [
    dict(lens=[64, 32, 104], R=2, B=16, mask="causal"),
    dict(lens=[40, 88, 24, 96], R=4, B=8, mask="lambda", sink=3, window=20),
    dict(lens=[120, 72, 48], R=3, B=16, mask="blockwise", sink=1, window=2, mask_block=8),
    dict(lens=[96, 60], R=2, B=12, mask="shared_prefix", bounds=[[20, 50, 70, 96], [12, 36, 60, 60]]),
    dict(lens=[256], R=8, B=8, mask="causal"),
    dict(lens=[37, 5, 130, 1, 64], R=3, B=10, mask="causal"),
    dict(lens=[300, 200], R=4, B=25, mask="lambda", sink=0, window=7),
    dict(lens=[512, 256, 768], R=8, B=32, mask="blockwise", sink=1, window=2, mask_block=32),
]


def _bounds(c):
    return None if c.get("bounds") is None else [list(b) for b in c["bounds"]]


def _place(c, hq=4, hkv=2, d_qk=64, d_v=32, dtype="bf16", eps=0.1):
    cu = np.concatenate([[0], np.cumsum(c["lens"])])
    bounds = c.get("bounds")
    if bounds is not None:
        # fill the padding answer (end == previous end) the way the mask expects
        bounds = [[int(x) for x in b] for b in bounds]
        for b in bounds:
            for k in range(2, len(b)):
                b[k] = max(b[k], b[k - 1])
    p = cva.Placement(cu, c["R"], c["B"], hq=hq, hkv=hkv, d_qk=d_qk, d_v=d_v, dtype=dtype,
                      mask=c["mask"], sink=c.get("sink", 0), window=c.get("window", 0),
                      branch_bounds=bounds, mask_block=c.get("mask_block", 0), epsilon=eps)
    return cu, p


def _oracle(c, cu):
    return blocks_ref(cu, c["B"], c["mask"], c.get("sink", 0), c.get("window", 0), _bounds(c),
                      c.get("mask_block", 0))


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_blocks_match_oracle(ci):
    c = CASES[ci]
    cu, p = _place(c)
    data, comp = _oracle(c, cu)
    assert [tuple(r[:3]) for r in p.data_blocks.tolist()] == data
    got = {tuple(r[:3]): int(n) for r, n in zip(p.comp_blocks.tolist(), p.comp_pairs)}
    assert got == comp
    assert len(got) == p.comp_blocks.shape[0]  # no duplicates


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_loads_and_volumes_match_oracle(ci):
    c = CASES[ci]
    hq, hkv, d_qk, d_v = 4, 2, 64, 32
    cu, p = _place(c, hq, hkv, d_qk, d_v)
    R, B = c["R"], c["B"]
    assert ((p.data_blocks[:, 3] >= 0) & (p.data_blocks[:, 3] < R)).all()
    assert ((p.comp_blocks[:, 3] >= 0) & (p.comp_blocks[:, 3] < R)).all()
    d = {(int(i), int(t0) // B): (int(tok), int(dev)) for i, t0, tok, dev in p.data_blocks}
    cd = {(int(i), int(qb), int(kb)): (int(n), int(dev))
          for (i, qb, kb, dev), n in zip(p.comp_blocks, p.comp_pairs)}
    sizes = (hq * d_qk * 2, hkv * (d_qk + d_v) * 2, hq * d_v * 2)
    v = volumes_ref(d, cd, sizes, R)
    assert (p.device_tokens == v["tokens"]).all()
    assert (p.device_pairs == v["pairs"]).all()
    assert (p.device_send_bytes == v["send"]).all()
    assert (p.device_recv_bytes == v["recv"]).all()
    assert p.total_comm_bytes == v["connectivity"]
    assert p.block_comm_bytes == v["block_volume"]
    assert p.zigzag_comm_bytes == (R - 1) * int(cu[-1]) * sizes[1]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_balance_constraints(ci):
    c = CASES[ci]
    cu, p = _place(c, eps=0.1)
    R, B = c["R"], c["B"]
    assert p.device_tokens.sum() == cu[-1]
    assert p.device_tokens.max() <= cu[-1] / R + B
    mean = p.device_pairs.sum() / R
    # a single computation block heavier than the slack can force the cap open
    slack = max(0.1 * mean, float(p.comp_pairs.max()))
    assert p.device_pairs.max() <= mean + slack


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_zigzag_pairs_match_oracle(ci):
    c = CASES[ci]
    cu, p = _place(c)
    R = c["R"]
    ok = all(L % (2 * R) == 0 for L in c["lens"])
    assert (p.zigzag_pairs is not None) == ok
    if ok:
        for r in range(R):
            w = synth.custom_workload(c["lens"], R, r, 4, 2, 64, 32, mask=c["mask"],
                                      sink=c.get("sink", 0), window=c.get("window", 0),
                                      branch_bounds=c.get("bounds"), block=c.get("mask_block", 0))
            assert p.zigzag_pairs[r] == visible_pairs_ref(w)


def test_one_device_needs_no_communication():
    cu, p = _place(dict(lens=[64, 40], R=1, B=16, mask="causal"))
    assert (p.data_blocks[:, 3] == 0).all() and (p.comp_blocks[:, 3] == 0).all()
    assert p.total_comm_bytes == 0 and p.block_comm_bytes == 0 and p.zigzag_comm_bytes == 0


def test_causal_balanced_like_zigzag():
    # causal rows: the placement balances pairs as the zig-zag split does, with
    # no more traffic than the zig-zag K/V all-gather
    cu, p = _place(dict(lens=[4096, 2048, 2048], R=4, B=256, mask="causal"), hq=8, hkv=1,
                   d_qk=128, d_v=128)
    assert p.device_pairs.max() <= 1.1 * p.device_pairs.mean()
    assert p.device_pairs.max() <= 1.1 * p.zigzag_pairs.max()
    assert p.total_comm_bytes <= p.zigzag_comm_bytes


@pytest.mark.parametrize("mask", ["blockwise", "lambda", "shared_prefix"])
def test_sparse8_balance_beats_zigzag(mask):
    # the eight-sequence sparse-mask batch over 8 devices: the zig-zag split is
    # unbalanced under sparse masks; the placement stays within epsilon
    w = synth.make_workload("sparse8", mask=mask)
    lens = [int(x) for x in w.lengths]
    R = 8
    bounds = None if w.branch_bounds is None else w.branch_bounds.tolist()
    p = cva.Placement(w.cu_seqlens, R, 1024, hq=w.hq, hkv=w.hkv, d_qk=w.d_qk, d_v=w.d_v,
                      mask=mask, sink=w.sink, window=w.window, branch_bounds=bounds,
                      mask_block=w.block, epsilon=0.1)
    assert p.device_pairs.max() <= 1.1 * p.device_pairs.mean() + p.comp_pairs.max()
    if p.zigzag_pairs is not None:
        # zig-zag per-rank pairs as the plan reports them
        plan = cva.Plan(w.cu_seqlens, R, 0, w.hq, w.hkv, w.d_qk, w.d_v, mask=mask, sink=w.sink,
                        window=w.window, branch_bounds=bounds, block=w.block)
        assert (plan.metadata["visible_pairs_per_rank"] == p.zigzag_pairs).all()
        assert p.device_pairs.max() <= p.zigzag_pairs.max()
    assert sum(lens) == p.device_tokens.sum()


@pytest.mark.parametrize("kw,status", [
    (dict(cu=[0]), "CVA_E_CU_SEQLENS"),
    (dict(cu=[0, 8, 8]), "CVA_E_CU_SEQLENS"),
    (dict(cu=[2, 8]), "CVA_E_CU_SEQLENS"),
    (dict(R=0), "CVA_E_RANK"),
    (dict(R=65), "CVA_E_RANK"),
    (dict(B=0), "CVA_E_ARG"),
    (dict(eps=-0.5), "CVA_E_ARG"),
    (dict(hq=0), "CVA_E_HEADS"),
    (dict(mask="lambda", window=0), "CVA_E_MASK"),
    (dict(mask="blockwise", window=2, sink=1, mask_block=0), "CVA_E_MASK"),
])
def test_invalid_placements_rejected(kw, status):
    a = dict(cu=[0, 16], R=2, B=4, hq=2, mask="causal", sink=0, window=0, mask_block=0, eps=0.1)
    a.update(kw)
    with pytest.raises(cva.CvaError) as ei:
        cva.Placement(a["cu"], a["R"], a["B"], hq=a["hq"], mask=a["mask"], sink=a["sink"],
                      window=a["window"], mask_block=a["mask_block"], epsilon=a["eps"])
    assert ei.value.status_name == status, str(ei.value)


# ---- one device's share as a plan: its forward items cover exactly its blocks ----

from oracle.masks import mask_ref as _mask_ref_oracle  # noqa: E402


@pytest.mark.parametrize("mask", ["causal", "lambda", "shared_prefix", "blockwise"])
def test_placed_plan_items_cover_exactly_the_device_blocks(mask):
    """Every visible (query, key) pair of a device's computation blocks is in exactly
    one forward item of its plan and no other pair is; a span marked full has every
    valid row seeing every key of its tiles; items of one Q tile merge together."""
    lens = [640, 384, 1000]
    cu = np.concatenate([[0], np.cumsum(lens)])
    bb = None
    if mask == "shared_prefix":
        bb = np.array([synth.shared_prefix_bounds(L, prefix=128) for L in lens])
    kw = dict(sink=32, window=200) if mask == "lambda" else dict(sink=1, window=2, mask_block=64)
    pl = cva.Placement(cu, 3, 128, hq=4, hkv=2, d_qk=128, mask=mask, branch_bounds=bb, **kw)
    masks = [_mask_ref_oracle(mask, L, kw.get("sink", 0), kw.get("window", 0),
                              None if bb is None else bb[i], kw.get("mask_block", 0))
             for i, L in enumerate(lens)]
    B = 128
    multi = 0
    for d in range(3):
        pp = pl.device_plan(d)
        t = pp.tables()
        segs = t["segs"]
        tile_q, tile_kv, tiles, spans = pp.schedule(3)
        cnt = [np.zeros((L, L), np.int64) for L in lens]
        for (sg, q0, rows, s0, ns) in tiles:
            i, qb, qlen = segs[sg, 0], segs[sg, 1], segs[sg, 2]
            assert segs[sg, 4] == cu[i] + qb * B and qlen == min(B, lens[i] - qb * B)
            qrows = np.arange(qb * B + q0, qb * B + q0 + rows)
            for (t0, t1, partial, _) in spans[s0: s0 + ns]:
                keys = np.arange(t0 * tile_kv, min(t1 * tile_kv, lens[i]))
                vis = masks[i][np.ix_(qrows, keys)]
                cnt[i][np.ix_(qrows, keys)] += vis
                if not partial:
                    assert vis.all(), "a span marked full has a masked element"
        want = [np.zeros((L, L), np.int64) for L in lens]
        for (i, qb, kb, dev) in pl.comp_blocks:
            if dev == d:
                want[i][qb * B:(qb + 1) * B, kb * B:(kb + 1) * B] = masks[i][qb * B:(qb + 1) * B,
                                                                               kb * B:(kb + 1) * B]
        for i in range(len(lens)):
            assert np.array_equal(cnt[i], want[i]), (d, i)
        # merge records: one per Q tile of every segment, over the slots of its items
        comb = t["split_combine"]
        slot_of_item = t["split_slot"]
        for (sg, q0, rows, slot0, npiece) in comb:
            items = [n for n in range(len(tiles)) if tiles[n, 0] == sg and tiles[n, 1] == q0]
            assert sorted(slot_of_item[items]) == list(range(slot0, slot0 + npiece))
            multi = max(multi, npiece)
    assert multi >= 2  # some output tile is fed by several computation blocks
