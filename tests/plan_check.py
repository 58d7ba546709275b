"""Bounds checker for a plan's device tables (test helper, CPU only).

Walks every table the kernels read -- segments, the prefix index, per-row
visible intervals, the forward / dQ / dK-dV / split schedules and their spans,
the zero-fill ranges, the split slots and merge records -- and asserts that
every index a kernel dereferences through them lies inside the buffer it
addresses (the tile records' segment ids, every row a tile covers, every
prefix-index entry a K/V tile loads (rank-major row < T), the rows of each
zero-fill range, every partial slot, every streamed-forward item list), and
that the forward and dQ tiles partition every segment's rows.  It reads the tables through the C ABI
(cva_plan_get_tables / cva_plan_get_schedule) and shares no code with the
library that builds them.
"""
import numpy as np

# per-item span capacities of the kernels (forward, dQ, dK/dV, split forward)
MAX_SPANS = {0: 8, 1: 8, 2: 16, 3: 8}
ZERO_ROWS_PER_BLOCK = 8
STREAM_MAX_ITEMS = 48


def _req(cond, msg):
    if not cond:
        raise AssertionError(msg)


def check_plan_tables(plan, n_seqs, T, T_loc):
    """Raise AssertionError naming the first table entry a kernel would read out of bounds."""
    t = plan.tables()
    segs, kvi, iv = t["segs"], t["kv_index"], t["row_iv"]
    n_segs = len(segs)
    _req(n_segs >= 1, "no segments")
    seq, _chunk, q_len, kv_len, row0, kv_off, _qpos0, _seqlen = segs.T
    _req(((seq >= 0) & (seq < n_seqs)).all(), "segment: sequence id out of range")
    _req((q_len >= 1).all(), "segment: no queries")
    _req(((row0 >= 0) & (row0 + q_len <= T_loc)).all(), "segment: local rows outside [0, T_loc)")
    _req(((kv_len >= 1) & (kv_off >= 0) & (kv_off + kv_len <= len(kvi))).all(),
         "segment: prefix outside kv_index")
    _req(len(kvi) == 0 or (kvi.min() >= 0 and kvi.max() < T), "kv_index: row outside [0, T)")
    _req(len(iv) == T_loc, f"row_iv has {len(iv)} rows, expected {T_loc}")
    for s in range(n_segs):
        r = iv[row0[s]: row0[s] + q_len[s]]
        for lo, hi in ((r[:, 0], r[:, 1]), (r[:, 2], r[:, 3])):
            nonempty = hi > lo
            _req(((lo[nonempty] >= 0) & (hi[nonempty] <= kv_len[s])).all(),
                 f"row_iv: a visible interval of segment {s} leaves its prefix")

    slots = t["split_slot"]
    for which in (0, 1, 3):
        tile_q, tile_kv, tiles, spans = plan.schedule(which)
        if which == 3:
            _req(len(slots) == len(tiles), "split slots: one per item of schedule 3")
        if len(tiles) == 0:
            continue
        sg, q0, rows, s0, ns = tiles.T
        _req(((sg >= 0) & (sg < n_segs)).all(), f"schedule {which}: segment id out of range")
        _req(((q0 >= 0) & (q0 < q_len[sg])).all(), f"schedule {which}: first query outside its segment")
        _req(((rows >= 1) & (rows <= np.minimum(tile_q, q_len[sg] - q0))).all(),
             f"schedule {which}: row count")
        if which in (0, 1):  # each row of every segment in exactly one tile (the split repeats tiles)
            cover = np.zeros(int(q_len.sum()), np.int32)
            seg0 = np.concatenate([[0], np.cumsum(q_len)[:-1]])
            for g, a0, n in zip(sg, q0, rows):
                cover[seg0[g] + a0: seg0[g] + a0 + n] += 1
            _req((cover == 1).all(), f"schedule {which}: tiles do not partition the segments' rows")
        _req(((ns >= 0) & (ns <= MAX_SPANS[which]) & (s0 >= 0) & (s0 + ns <= len(spans))).all(),
             f"schedule {which}: span range")
        if which == 3:
            _req((ns[slots >= 0] >= 1).all(), "split: an item writing a partial slot has no K/V tile")
        for i in range(len(tiles)):
            sp = spans[s0[i]: s0[i] + ns[i]]
            if len(sp) == 0:
                continue
            _req(((sp[:, 0] >= 0) & (sp[:, 0] < sp[:, 1])).all(), f"schedule {which}: empty or negative span")
            _req(((sp[:, 1] - 1) * tile_kv < kv_len[sg[i]]).all(),
                 f"schedule {which}: a K/V tile starts past its segment's prefix")
            _req(np.isin(sp[:, 2], (0, 1)).all(), f"schedule {which}: partial flag")

    tile_q, tile_kv, tiles, spans = plan.schedule(2)
    if len(tiles):
        sq, k0, keys, s0, ns = tiles.T
        _req(((sq >= 0) & (sq < n_seqs)).all(), "dK/dV: sequence id out of range")
        kvmax = np.zeros(n_seqs, np.int64)
        np.maximum.at(kvmax, seq, kv_len)
        _req(((k0 >= 0) & (keys >= 1) & (k0 + keys <= kvmax[sq])).all(),
             "dK/dV: keys outside the sequence's longest prefix")
        _req(((ns >= 0) & (ns <= MAX_SPANS[2]) & (s0 >= 0) & (s0 + ns <= len(spans))).all(),
             "dK/dV: span range")
        for i in range(len(tiles)):
            sp = spans[s0[i]: s0[i] + ns[i]]
            if len(sp) == 0:
                continue
            g = sp[:, 0]
            _req(((g >= 0) & (g < n_segs)).all(), "dK/dV: span segment out of range")
            _req((seq[g] == sq[i]).all(), "dK/dV: span segment of another sequence")
            nqt = (q_len[g] + tile_q - 1) // tile_q
            _req(((sp[:, 1] >= 0) & (sp[:, 1] < sp[:, 2]) & (sp[:, 2] <= nqt)).all(),
                 "dK/dV: Q tile range outside its segment")
            _req(np.isin(sp[:, 3], (0, 1)).all(), "dK/dV: partial flag")

    zr = t["zero_rows"]
    if len(zr):
        _req(((zr[:, 0] >= 0) & (zr[:, 0] < zr[:, 1]) & (zr[:, 1] <= T)).all(), "zero rows: range")
        _req((zr[:, 1] - zr[:, 0] <= ZERO_ROWS_PER_BLOCK).all(), "zero rows: range longer than a block")
        covered = np.zeros(T, bool)
        covered[kvi] = True
        for a, b in zr:
            _req(not covered[a:b].any(), "zero rows: a range overlaps rows the backward writes")

    # streamed forward deals: every item of the schedule dealt exactly once, at
    # most STREAM_MAX_ITEMS per work-group (the kernel's LDS table)
    for key, which in (("fwd_deal", 0), ("split_deal", 3)):
        wgs, start, items = t[key]
        n_items = len(plan.schedule(which)[2])
        if wgs == 0:
            continue
        _req(len(start) == wgs + 1 and start[0] == 0 and start[-1] == len(items), f"{key}: start table")
        sizes = np.diff(start)
        _req(((sizes >= 1) & (sizes <= STREAM_MAX_ITEMS)).all(), f"{key}: items per work-group")
        _req(np.array_equal(np.sort(items), np.arange(n_items)), f"{key}: every item exactly once")

    n_slots, comb = t["n_split_slots"], t["split_combine"]
    _req(((slots >= -1) & (slots < n_slots)).all(), "split: slot out of range")
    used = slots[slots >= 0]
    _req(len(np.unique(used)) == len(used), "split: two items share a slot")
    if len(comb):
        cs, cq0, crows, cslot0, cnp = comb.T
        _req(((cs >= 0) & (cs < n_segs)).all(), "merge: segment id out of range")
        _req(((cq0 >= 0) & (cq0 < q_len[cs])).all(), "merge: first query outside its segment")
        _req(((cnp >= 0) & (cslot0 >= 0) & (cslot0 + cnp <= n_slots)).all(), "merge: slot range")
        owner = np.full(n_slots, -1)
        for c in range(len(comb)):
            _req((owner[cslot0[c]: cslot0[c] + cnp[c]] == -1).all(), "merge: a slot in two records")
            owner[cslot0[c]: cslot0[c] + cnp[c]] = c
        _req(np.isin(used, np.nonzero(owner >= 0)[0]).all(), "merge: a written slot is never merged")
    return True
