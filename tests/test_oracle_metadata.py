"""Pins for the oracle's split and metadata (CPU only).

The oracle builds everything by enumerating positions; these tests hold it to
(a) values worked out by hand from the MindSpeed RFC's chunking rule (section 2)
and rank-major layout (section 3.1), (b) closed forms that follow from that rule,
and (c) invariants: the ranks' local positions partition [0, T), every index is in
range, indexing a position-tagged K with the index reads each segment's own
prefix, and the per-rank workload sum(q_len*kv_len) is equal for R=2 and R=4
(RFC section 3.5.1, acceptance).
"""
import json
import os
import random

import numpy as np
import pytest

import oracle
from oracle.split import rank_local_positions, rank_major_order

GOLD = os.path.join(os.path.dirname(__file__), "golden", "tiny_r2_metadata.json")


def _expand(runs):
    out = []
    for a, b in runs:
        out.extend(range(a, b + 1))
    return out


def _random_cu(rng, R, n_max=6, c_max=9):
    n = rng.randint(1, n_max)
    lens = [2 * R * rng.randint(1, c_max) for _ in range(n)]
    return [0] + list(np.cumsum(lens))


def test_tiny_hand_derived_values():
    g = json.load(open(GOLD))
    cu, R = g["cu_seqlens"], g["cp_size"]
    for r_str, exp in g["ranks"].items():
        r = int(r_str)
        md = oracle.metadata_ref(cu, R, r)
        assert md["local_tokens"] == exp["local_tokens"]
        assert md["global_tokens"] == exp["global_tokens"]
        assert md["local_cu"].tolist() == exp["local_cu"]
        assert md["actual_seq_qlen"].tolist() == exp["actual_seq_qlen"]
        assert md["actual_seq_kvlen"].tolist() == exp["actual_seq_kvlen"]
        assert md["seg_q_pos0"].tolist() == exp["seg_q_pos0"]
        assert md["kv_index"].tolist() == _expand(exp["kv_index_runs"])
        assert rank_local_positions(cu, R, r) == _expand(exp["local_positions_runs"])
        assert md["workload_per_rank"].tolist() == [exp["workload"]] * R


@pytest.mark.parametrize("R", [1, 2, 3, 4, 8])
def test_closed_forms(R):
    rng = random.Random(100 + R)
    for _ in range(20):
        cu = _random_cu(rng, R)
        lens = np.diff(cu)
        c = lens // (2 * R)
        T = cu[-1]
        for r in range(R):
            md = oracle.metadata_ref(cu, R, r)
            assert md["local_tokens"] == T // R
            assert md["local_cu"].tolist() == [x // R for x in cu]
            ql = np.repeat(c, 2)
            kvl = np.stack([(r + 1) * c, (2 * R - r) * c], axis=1).reshape(-1)
            assert md["actual_seq_qlen"].tolist() == [0] + np.cumsum(ql).tolist()
            assert md["actual_seq_kvlen"].tolist() == [0] + np.cumsum(kvl).tolist()
            assert len(md["kv_index"]) == T * (2 * R + 1) // (2 * R)
            assert md["workload_per_rank"].tolist() == [(2 * R + 1) * int((c * c).sum())] * R


@pytest.mark.parametrize("R", [1, 2, 4, 8])
def test_partition_and_index_range(R):
    rng = random.Random(7 + R)
    for _ in range(10):
        cu = _random_cu(rng, R)
        T = cu[-1]
        allpos = []
        for r in range(R):
            allpos += rank_local_positions(cu, R, r)
            idx = oracle.metadata_ref(cu, R, r)["kv_index"]
            assert idx.min() >= 0 and idx.max() < T
        assert sorted(allpos) == list(range(T))
        assert sorted(rank_major_order(cu, R)) == list(range(T))


@pytest.mark.parametrize("R", [1, 2, 3, 4])
def test_position_tagging(R):
    """Tag K_full[p] = p, split + all-gather rank-major, read through kv_index."""
    rng = random.Random(31 + R)
    for _ in range(10):
        cu = _random_cu(rng, R)
        tag = np.arange(cu[-1])
        gathered = np.concatenate([tag[rank_local_positions(cu, R, s)] for s in range(R)])
        for r in range(R):
            md = oracle.metadata_ref(cu, R, r)
            got = gathered[md["kv_index"]]
            akv = md["actual_seq_kvlen"]
            seg = 0
            for i in range(len(cu) - 1):
                for _j in range(2):
                    run = got[akv[seg]: akv[seg + 1]]
                    assert run.tolist() == list(range(cu[i], cu[i] + len(run)))
                    seg += 1


@pytest.mark.parametrize("R", [2, 4])
def test_workload_equal(R):
    rng = random.Random(55 + R)
    for _ in range(25):
        cu = _random_cu(rng, R, n_max=10, c_max=40)
        ws = [oracle.workload_ref(cu, R, s) for s in range(R)]
        assert len(set(ws)) == 1
        # brute force: q_len * kv_len from the chunk sizes, nothing shared with the oracle
        brute = 0
        for i in range(len(cu) - 1):
            c = (cu[i + 1] - cu[i]) // (2 * R)
            brute += c * (c * 1) + c * (c * 2 * R)  # rank 0: chunks 0 and 2R-1
        assert ws[0] == brute


@pytest.mark.parametrize("bad", [
    dict(cu=[0], R=1, r=0), dict(cu=[1, 9], R=1, r=0), dict(cu=[0, 8, 8], R=1, r=0),
    dict(cu=[0, 6], R=2, r=0), dict(cu=[0, 8], R=2, r=2), dict(cu=[0, 8], R=0, r=0),
    dict(cu=[0, 8], R=2, r=-1),
])
def test_bad_input_asserts(bad):
    with pytest.raises(AssertionError):
        oracle.metadata_ref(bad["cu"], bad["R"], bad["r"])
