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
