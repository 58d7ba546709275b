"""Pins for the oracle's block placement model (CPU only).

DCP paper, section 4.1: data blocks, computation blocks that exist only where
the mask is not all zero, the per-computation-block communication volume and
the hypergraph connectivity.  Pinned against the page's Fig. 9 / Fig. 12
example, volumes of small placements worked out by hand, the pure data-parallel
placement of Fig. 10 (no communication), and pair counts in closed form.
"""
import json
import os

import numpy as np
import pytest

from oracle.placement import blocks_ref, volumes_ref

GOLD = os.path.join(os.path.dirname(__file__), "golden", "dcp_fig9_blocks.json")


def _assign(data, comp, B, data_dev, comp_dev):
    d = {(i, t0 // B): (tok, data_dev[n]) for n, (i, t0, tok) in enumerate(data)}
    c = {k: (comp[k], comp_dev[k]) for k in comp}
    return d, c


def test_fig9_shared_question_blocks():
    g = json.load(open(GOLD))
    L, B = g["seq_len"], g["block"]
    data, comp = blocks_ref([0, L], B, "shared_prefix", bounds=[g["bounds"]])
    assert len(data) == g["data_blocks_per_tensor"]
    assert 3 * len(data) == g["hyperedges"]  # one hyperedge per Q, KV and O block
    exp = {(0, qb, kb): n for qb, kb, n in g["comp_blocks"]}
    assert comp == exp
    last_two = sorted(comp)[-2:]
    assert {qb for (_, qb, _) in last_two} == {g["output_of_last_two"]}


def test_causal_block_counts_closed_form():
    for L, B in [(12, 4), (13, 4), (64, 8), (7, 7), (5, 1)]:
        data, comp = blocks_ref([0, L], B)
        nb = -(-L // B)
        assert len(data) == nb
        assert len(comp) == nb * (nb + 1) // 2
        assert sum(comp.values()) == L * (L + 1) // 2
        for (_, qb, kb), n in comp.items():  # diagonal blocks are triangles
            if qb == kb:
                t = min(B, L - qb * B)
                assert n == t * (t + 1) // 2
            else:
                assert n == min(B, L - qb * B) * B


def test_lambda_window_inside_block_drops_far_blocks():
    # sink 0, window 2, block 4: a query sees itself and one earlier key, so only
    # the diagonal blocks and the block just before (for the first row of a block)
    L, B = 16, 4
    _, comp = blocks_ref([0, L], B, "lambda", sink=0, window=2)
    assert set(comp) == {(0, b, b) for b in range(4)} | {(0, b, b - 1) for b in range(1, 4)}
    assert all(comp[(0, b, b - 1)] == 1 for b in range(1, 4))
    assert sum(comp.values()) == L + (L - 1)


def test_volumes_by_hand():
    # one causal sequence of 4 tokens, block 2, two devices; row sizes 3 / 5 / 7 bytes
    sizes = (3, 5, 7)
    data, comp = blocks_ref([0, 4], 2)
    assert comp == {(0, 0, 0): 3, (0, 1, 0): 4, (0, 1, 1): 3}
    # data block 0 on device 0, block 1 on device 1; computation at the Q block's owner
    d, c = _assign(data, comp, 2, [0, 1], {(0, 0, 0): 0, (0, 1, 0): 1, (0, 1, 1): 1})
    v = volumes_ref(d, c, sizes, 2)
    assert v["block_volume"] == 2 * 5          # K/V block 0 fetched once
    assert v["connectivity"] == 2 * 5
    assert list(v["send"]) == [10, 0] and list(v["recv"]) == [0, 10]
    assert list(v["tokens"]) == [2, 2] and list(v["pairs"]) == [3, 7]
    # move C(1,0) to device 0: Q block 1 goes there and its partial O comes back
    d, c = _assign(data, comp, 2, [0, 1], {(0, 0, 0): 0, (0, 1, 0): 0, (0, 1, 1): 1})
    v = volumes_ref(d, c, sizes, 2)
    assert v["block_volume"] == 2 * 3 + 2 * 7
    assert v["connectivity"] == 2 * 3 + 2 * 7
    assert list(v["send"]) == [14, 6] and list(v["recv"]) == [6, 14]
    assert list(v["pairs"]) == [7, 3]


def test_volumes_reuse_counts_once_in_connectivity():
    # 6 tokens, block 2, causal: Q block 2 on device 1 uses K/V blocks 0 and 1 of
    # device 0; computing C(2,0) and C(2,1) on device 0 moves Q2 and O2 once
    # (connectivity) but twice in the per-computation-block sum
    sizes = (1, 10, 100)
    data, comp = blocks_ref([0, 6], 2)
    dev = {k: (1 if k[1] == 2 else 0) for k in comp}
    dev[(0, 2, 0)] = dev[(0, 2, 1)] = 0
    d, c = _assign(data, comp, 2, [0, 0, 1], dev)
    v = volumes_ref(d, c, sizes, 2)
    assert v["block_volume"] == 2 * (2 * 1 + 2 * 100)
    assert v["connectivity"] == 2 * 1 + 2 * 100
    # C(2,2) stays on device 1 with all its blocks
    assert list(v["pairs"]) == [3 + 4 + 3 + 4 + 4, 3]


def test_pure_data_parallel_placement_has_no_communication():
    # Fig. 10: sequences 1 and 2 on device 0, sequence 3 on device 1
    cu = [0, 6, 10, 20]
    B = 2
    data, comp = blocks_ref(cu, B)
    data_dev = [0 if i < 2 else 1 for (i, _, _) in data]
    comp_dev = {k: (0 if k[0] < 2 else 1) for k in comp}
    d, c = _assign(data, comp, B, data_dev, comp_dev)
    v = volumes_ref(d, c, (2, 4, 2), 2)
    assert v["block_volume"] == 0 and v["connectivity"] == 0
    assert list(v["tokens"]) == [10, 10]
    assert list(v["pairs"]) == [21 + 10, 55]
    assert not v["send"].any() and not v["recv"].any()


def test_send_equals_receive_in_total():
    rng = np.random.default_rng(3)
    cu = [0, 10, 17, 40]
    data, comp = blocks_ref(cu, 3, "lambda", sink=2, window=5)
    data_dev = list(rng.integers(0, 4, size=len(data)))
    comp_dev = {k: int(rng.integers(0, 4)) for k in comp}
    d, c = _assign(data, comp, 3, data_dev, comp_dev)
    v = volumes_ref(d, c, (2, 3, 5), 4)
    assert v["send"].sum() == v["recv"].sum() == v["connectivity"]
    assert v["connectivity"] <= v["block_volume"]


# ---- one device's share of a placement: forward from the definition ----

import math  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402
from oracle.placement import share_fwd_ref  # noqa: E402


def _share_case(mask, dtype="fp32"):
    lens = [10, 7, 13]
    bb = None
    if mask == "shared_prefix":
        bb = [[3, 6, 8, 10], [2, 4, 6, 7], [4, 7, 10, 13]]
    w = synth.custom_workload(lens, 1, 0, 4, 2, 8, 6, dtype, mask=mask, sink=2, window=4,
                              branch_bounds=bb)
    return w, synth.random_tensors(w, 71, with_dout=False)


@pytest.mark.parametrize("mask", ["causal", "lambda", "shared_prefix"])
def test_share_with_every_block_on_one_device_is_full_attention(mask):
    w, (q, k, v) = _share_case(mask)
    B = 3
    _, comp = blocks_ref(w.cu_seqlens, B, mask, sink=2, window=4,
                         bounds=None if w.branch_bounds is None else w.branch_bounds)
    o, lse = share_fwd_ref(w, q, k, v, B, {c: 0 for c in comp}, 0, scale=0.5)
    ro, rl = oracle.fwd_full_ref(w, q, k, v, scale=0.5)
    np.testing.assert_allclose(o, ro, atol=1e-13)
    np.testing.assert_allclose(lse, rl, atol=1e-13)
    o1, _ = share_fwd_ref(w, q, k, v, B, {c: 0 for c in comp}, 1, scale=0.5)
    assert np.isnan(o1).all()  # device 1 computes nothing


@pytest.mark.parametrize("mask", ["causal", "lambda", "shared_prefix"])
def test_lse_merge_of_all_shares_is_full_attention(mask):
    """Fig. 9(b): the partial outputs of the computation blocks of one output block,
    spread over devices, reduce to the unsplit result."""
    w, (q, k, v) = _share_case(mask)
    B, R = 2, 3
    _, comp = blocks_ref(w.cu_seqlens, B, mask, sink=2, window=4,
                         bounds=None if w.branch_bounds is None else w.branch_bounds)
    rng = np.random.default_rng(4)
    comp_dev = {c: int(rng.integers(0, R)) for c in comp}
    shares = [share_fwd_ref(w, q, k, v, B, comp_dev, d, scale=0.7) for d in range(R)]
    ro, rl = oracle.fwd_full_ref(w, q, k, v, scale=0.7)
    T = w.total_tokens
    for h in range(w.hq):
        for t in range(T):
            parts = [(o[t, h], l[h, t]) for o, l in shares if not np.isnan(l[h, t])]
            assert parts, (h, t)  # every row has a visible key on some device
            ls = np.array([l for _, l in parts])
            m = ls[np.isfinite(ls)].max()
            wts = np.exp(ls - m)
            merged = sum(wt * o for wt, (o, _) in zip(wts, parts)) / wts.sum()
            np.testing.assert_allclose(merged, ro[t, h], atol=1e-12)
            assert abs(m + math.log(wts.sum()) - rl[h, t]) < 1e-12


def test_share_of_one_block_by_brute_force():
    """Q block 2 of a 10-token causal sequence (block 3) against K/V block 1 only:
    rows 6..8 over keys 3..5, written as plain loops."""
    w = synth.custom_workload([10], 1, 0, 2, 1, 3, 2, "fp32")
    q, k, v = synth.random_tensors(w, 72, with_dout=False)
    o, lse = share_fwd_ref(w, q, k, v, 3, {(0, 2, 1): 5, (0, 2, 2): 4}, 5, scale=0.9)
    for h in range(2):
        for t in (6, 7, 8):
            s = [0.9 * sum(float(q[t, h, d]) * float(k[j, 0, d]) for d in range(3)) for j in (3, 4, 5)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            den = sum(e)
            for d in range(2):
                want = sum(e[n] * float(v[j, 0, d]) for n, j in enumerate((3, 4, 5))) / den
                assert abs(o[t, h, d] - want) < 1e-12
            assert abs(lse[h, t] - (mx + math.log(den))) < 1e-12
    assert np.isnan(o[:6]).all() and np.isnan(o[9:]).all()
