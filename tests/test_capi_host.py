"""libcva host side on the CPU: exports, metadata, schedules, validation.

No GPU is touched: plan creation is host-only C++.  Metadata must equal the
oracle's enumeration bit for bit; the tile schedules must visit exactly the
(Q tile, K/V tile) pairs where the oracle's materialised mask is not all
zero, and call a tile full exactly when every element is visible.
"""
import ctypes
import random
import re
import os

import numpy as np
import pytest

import context_varlen_attention_amd as cva
import oracle
import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "cva.h")


def test_library_exports_every_declared_symbol():
    names = set(re.findall(r"\b(cva_[a-z_]+)\s*\(", open(HEADER).read()))
    assert names, "no declarations parsed"
    lib = ctypes.CDLL(cva.library_path())
    for n in sorted(names):
        assert hasattr(lib, n), f"{n} declared in cva.h but not exported"
    assert names == set(cva.EXPORTS)


def _random_cu(rng, R, n_max=6, c_max=40):
    n = rng.randint(1, n_max)
    return [0] + list(np.cumsum([2 * R * rng.randint(1, c_max) for _ in range(n)]))


@pytest.mark.parametrize("R", [1, 2, 3, 4, 8])
def test_metadata_bit_exact(R):
    rng = random.Random(1234 + R)
    for _ in range(8):
        cu = _random_cu(rng, R)
        for r in range(R):
            md = cva.Plan(cu, R, r, 4, 2, 128, 128, "bf16").metadata
            ref = oracle.metadata_ref(cu, R, r)
            for key in ("local_cu", "actual_seq_qlen", "actual_seq_kvlen", "kv_index",
                        "seg_q_pos0", "workload_per_rank"):
                assert np.array_equal(md[key], ref[key]), (cu, R, r, key)
            assert md["local_tokens"] == ref["local_tokens"]
            assert md["global_tokens"] == ref["global_tokens"]


@pytest.mark.parametrize("name", ["tiny", "gqa16k", "long128k", "mla32k"])
def test_metadata_bit_exact_workloads(name):
    w = synth.make_workload(name)
    md = cva.Plan(w.cu_seqlens, w.cp_size, w.rank, w.hq, w.hkv, w.d_qk, w.d_v, "bf16").metadata
    ref = oracle.metadata_ref(w.cu_seqlens, w.cp_size, w.rank)
    for key in ("local_cu", "actual_seq_qlen", "actual_seq_kvlen", "kv_index", "seg_q_pos0",
                "workload_per_rank"):
        assert np.array_equal(md[key], ref[key]), key


def test_split_helpers_match_oracle():
    rng = random.Random(9)
    for R in (1, 2, 4):
        cu = _random_cu(rng, R)
        for r in range(R):
            assert cva.local_token_ids(cu, R, r).tolist() == oracle.rank_local_positions(cu, R, r)
        assert cva.rank_major_token_ids(cu, R).tolist() == oracle.split.rank_major_order(cu, R)


def _wl(lens, R, r, mask, hq=4, hkv=4, **kw):
    return synth.custom_workload(lens, R, r, hq, hkv, 128, 128, "bf16", mask=mask, **kw)


def _plan(w):
    return cva.Plan(w.cu_seqlens, w.cp_size, w.rank, w.hq, w.hkv, w.d_qk, w.d_v, w.dtype,
                    mask=w.mask, sink=w.sink, window=w.window,
                    branch_bounds=None if w.branch_bounds is None else w.branch_bounds,
                    block=w.block)


MASK_CASES = [
    ([64, 128, 64], 2, 0, "causal", {}),
    ([8, 24, 200, 16, 1000], 4, 3, "causal", {}),
    ([1024, 640], 1, 0, "lambda", dict(sink=64, window=256)),
    ([1200, 400], 2, 1, "lambda", dict(sink=5, window=77)),
    ([640, 832], 2, 0, "lambda", dict(sink=0, window=100)),
    ([1280, 768], 1, 0, "shared_prefix",
     dict(branch_bounds=[[256, 512, 768, 1024, 1280], [128, 288, 448, 608, 768]])),
    ([1280, 768], 2, 1, "shared_prefix",
     dict(branch_bounds=[[200, 300, 300, 900, 1280], [0, 100, 400, 500, 768]])),
    ([2048, 1280], 1, 0, "blockwise", dict(block=256, sink=1, window=2)),
    ([1536, 640, 3072], 2, 1, "blockwise", dict(block=96, sink=2, window=3)),
    ([1200, 400], 2, 0, "blockwise", dict(block=50, sink=1, window=1)),
]


def _oracle_segments(w):
    """(sub-sequence, in-sequence q positions, kv_len) per segment, from the oracle's split."""
    md = oracle.metadata_ref(w.cu_seqlens, w.cp_size, w.rank)
    aq, akv, pos0 = md["actual_seq_qlen"], md["actual_seq_kvlen"], md["seg_q_pos0"]
    out = []
    for s in range(len(pos0)):
        n = aq[s + 1] - aq[s]
        out.append((s // 2, pos0[s] + np.arange(n), akv[s + 1] - akv[s]))
    return out


def _mask_rows(w, i, pos):
    L = int(w.cu_seqlens[i + 1] - w.cu_seqlens[i])
    b = None if w.branch_bounds is None else w.branch_bounds[i]
    return oracle.masks.mask_rows_ref(w.mask, L, pos, w.sink, w.window, b, w.block)


def _q_cuts(w, pos, tq):
    """Row ranges of a segment's Q tiles: every tq rows from the segment's start,
    except under the causal blockwise mask, where the cuts fall on in-sequence
    positions that are multiples of tq (the first cut rounded down to a multiple
    of 32 rows; none if that leaves it at 0 or past the end)."""
    n = len(pos)
    first = tq
    if w.mask == "blockwise":
        f = ((-int(pos[0])) % tq) // 32 * 32
        if 0 < f < n:
            first = f
    cuts, x = [0], min(first, n)
    while cuts[-1] < n:
        cuts.append(x)
        x = min(n, x + tq)
    return list(zip(cuts[:-1], cuts[1:]))


@pytest.mark.parametrize("ci", range(len(MASK_CASES)))
@pytest.mark.parametrize("which", [0, 1, 3])
def test_q_schedule_covers_exactly_nonempty_tiles(ci, which):
    lens, R, r, mask, ex = MASK_CASES[ci]
    w = _wl(lens, R, r, mask, **ex)
    plan = _plan(w)
    tq, tk, tiles, spans = plan.schedule(which)
    segs = _oracle_segments(w)
    cuts = {seg: _q_cuts(w, pos, tq) for seg, (i, pos, kv_len) in enumerate(segs)}
    got = {}
    for seg, q0, rows, s0, ns in tiles:
        assert (q0, q0 + rows) in cuts[seg]
        for a, b, partial, _ in spans[s0: s0 + ns]:
            for t in range(a, b):
                assert (seg, q0, t) not in got
                got[(seg, q0, t)] = bool(partial)
    exp = {}
    for seg, (i, pos, kv_len) in enumerate(segs):
        M = _mask_rows(w, i, pos)
        for q0, q1 in cuts[seg]:
            blk = M[q0: q1, :kv_len]
            for t in range((kv_len + tk - 1) // tk):
                sub = blk[:, t * tk: (t + 1) * tk]
                if sub.any():
                    exp[(seg, q0, t)] = not (sub.all() and sub.shape[1] == tk)
    assert got == exp


@pytest.mark.parametrize("ci", range(len(MASK_CASES)))
def test_kv_schedule_covers_exactly_nonempty_tiles(ci):
    lens, R, r, mask, ex = MASK_CASES[ci]
    w = _wl(lens, R, r, mask, **ex)
    plan = _plan(w)
    tq, tk, tiles, spans = plan.schedule(2)
    segs = _oracle_segments(w)
    got = {}
    seen_tiles = set()
    for seq, k0, keys, s0, ns in tiles:
        assert k0 % tk == 0
        seen_tiles.add((seq, k0 // tk))
        for seg, qa, qb, partial in spans[s0: s0 + ns]:
            assert segs[seg][0] == seq
            for qt in range(qa, qb):
                got[(seg, qt, k0 // tk)] = bool(partial)
    exp = {}
    for seg, (i, pos, kv_len) in enumerate(segs):
        M = _mask_rows(w, i, pos)
        for qt in range((len(pos) + tq - 1) // tq):
            blk = M[qt * tq: (qt + 1) * tq, :kv_len]
            for t in range((kv_len + tk - 1) // tk):
                sub = blk[:, t * tk: (t + 1) * tk]
                if sub.any():
                    # a Q tile cut short by the segment's end also takes the masked path
                    exp[(seg, qt, t)] = not (sub.all() and sub.shape[1] == tk and sub.shape[0] == tq)
    assert got == exp
    # every K/V tile of every sub-sequence's longest prefix has a record
    for seg in range(1, len(segs), 2):
        i, _, kv_len = segs[seg]
        for t in range((kv_len + tk - 1) // tk):
            assert (i, t) in seen_tiles


@pytest.mark.parametrize("ci", range(len(MASK_CASES)))
def test_visible_pairs_match_oracle(ci):
    lens, R, r, mask, ex = MASK_CASES[ci]
    w = _wl(lens, R, r, mask, **ex)
    assert _plan(w).visible_pairs() == oracle.visible_pairs_ref(w)


def test_causal_visible_pairs_closed_form():
    for name in ("gqa16k", "long128k", "mla32k"):
        w = synth.make_workload(name)
        L = w.lengths.astype(np.int64)
        p = cva.Plan(w.cu_seqlens, w.cp_size, w.rank, w.hq, w.hkv, w.d_qk, w.d_v, "bf16")
        assert p.visible_pairs() == int((L * (L + 1)).sum() // (2 * w.cp_size))


def test_sparse_visible_pairs_closed_form():
    w = synth.make_workload("sparse8", mask="lambda")
    p = _plan(w)
    exp = 0
    for L in w.lengths:
        q = np.arange(L)
        exp += int(np.where(q < 4096, q + 1, 4096 + np.minimum(64, q - 4095)).sum())
    assert p.visible_pairs() == exp
    w = synth.make_workload("sparse8", mask="shared_prefix")
    exp = 0
    for b in w.branch_bounds:
        P = int(b[0])
        exp += P * (P + 1) // 2
        for s, e in zip(b[:-1], b[1:]):
            n = int(e - s)
            exp += n * P + n * (n + 1) // 2
    assert _plan(w).visible_pairs() == exp


@pytest.mark.parametrize("kw,status", [
    (dict(cu=[0]), "CVA_E_CU_SEQLENS"),
    (dict(cu=[4, 12]), "CVA_E_CU_SEQLENS"),
    (dict(cu=[0, 8, 8]), "CVA_E_CU_SEQLENS"),
    (dict(cu=[0, 8, 4]), "CVA_E_CU_SEQLENS"),
    (dict(cu=[0, 6], R=2), "CVA_E_ALIGN"),
    (dict(R=0), "CVA_E_RANK"),
    (dict(R=2, r=2), "CVA_E_RANK"),
    (dict(r=-1), "CVA_E_RANK"),
    (dict(hq=6, hkv=4), "CVA_E_HEADS"),
    (dict(hq=0), "CVA_E_HEADS"),
    (dict(d_qk=64, d_v=128), "CVA_E_HEADDIM"),
    (dict(d_qk=96, d_v=96), "CVA_E_HEADDIM"),
    (dict(mask="lambda", window=0), "CVA_E_MASK"),
    (dict(mask="lambda", sink=-1, window=4), "CVA_E_MASK"),
    (dict(mask="shared_prefix", bounds=[[4, 2, 16]]), "CVA_E_MASK"),
    (dict(mask="shared_prefix", bounds=[[4, 8, 15]]), "CVA_E_MASK"),
])
def test_invalid_requests_rejected(kw, status):
    args = dict(cu=[0, 16], R=1, r=0, hq=4, hkv=2, d_qk=128, d_v=128, mask="causal", sink=0,
                window=0, bounds=None)
    args.update(kw)
    with pytest.raises(cva.CvaError) as ei:
        cva.Plan(args["cu"], args["R"], args["r"], args["hq"], args["hkv"], args["d_qk"],
                 args["d_v"], "bf16", mask=args["mask"], sink=args["sink"],
                 window=args["window"], branch_bounds=args["bounds"])
    assert ei.value.status_name == status, str(ei.value)


def test_errors_before_device_work():
    """Calls that need a device copy refuse a plan that has none, without touching HIP."""
    lib = cva.load_library()
    p = cva.Plan([0, 64], 1, 0, 2, 2, 64, 64, "bf16")
    vp = ctypes.c_void_p
    st = lib.cva_fwd(p.handle, vp(16), vp(16), vp(16), vp(16), vp(16), 0.125, None)
    assert cva.STATUS[st] == "CVA_E_NOT_UPLOADED"
    st = lib.cva_bwd(p.handle, *([vp(16)] * 9), vp(16), 1 << 20, 0.125, None)
    assert cva.STATUS[st] == "CVA_E_NOT_UPLOADED"
    assert "cva_plan_upload" in lib.cva_last_error().decode()
    assert lib.cva_plan_upload(p.handle, None, 0, None) == 1


@pytest.mark.parametrize("p", [1.0, -0.25, 1.5, float("nan")])
def test_dropout_probability_rejected(p):
    """Dropout entry points refuse a probability outside [0, 1) before anything
    else (CVA_E_ARG), and a valid one reaches the usual checks."""
    lib = cva.load_library()
    plan = cva.Plan([0, 64], 1, 0, 2, 2, 64, 64, "bf16")
    vp = ctypes.c_void_p
    st = lib.cva_fwd_dropout(plan.handle, *([vp(16)] * 5), 0.125, p, 7, None, 0, None)
    assert cva.STATUS[st] == "CVA_E_ARG"
    assert "dropout" in lib.cva_last_error().decode()
    st = lib.cva_bwd_dropout(plan.handle, *([vp(16)] * 9), vp(16), 1 << 20, 0.125, p, 7, None)
    assert cva.STATUS[st] == "CVA_E_ARG"
    st = lib.cva_fwd_dropout(plan.handle, *([vp(16)] * 5), 0.125, 0.1, 7, None, 0, None)
    assert cva.STATUS[st] == "CVA_E_NOT_UPLOADED"
    st = lib.cva_bwd_dropout(plan.handle, *([vp(16)] * 9), vp(16), 1 << 20, 0.125, 0.1, 7, None)
    assert cva.STATUS[st] == "CVA_E_NOT_UPLOADED"


@pytest.mark.parametrize("seed", [-1, 1 << 64, 0.5, "7"])
def test_dropout_seed_rejected(seed):
    """The binding refuses a dropout seed outside [0, 2**64) before any device work."""
    plan = cva.Plan([0, 64], 1, 0, 2, 2, 64, 64, "bf16")
    with pytest.raises(ValueError):
        cva.fwd(plan, None, None, None, dropout_p=0.1, seed=seed)
    with pytest.raises(ValueError):
        cva.bwd(plan, None, None, None, None, None, None, dropout_p=0.1, seed=seed)


def test_zero_rows_complement_prefixes():
    """Rank-major rows that dK/dV zero-fills are exactly those outside every prefix."""
    for R, r in ((2, 0), (2, 1), (4, 2), (1, 0)):
        cu = [0, 8 * R, 24 * R, 32 * R]
        md = oracle.metadata_ref(cu, R, r)
        covered = np.zeros(cu[-1], bool)
        covered[md["kv_index"]] = True
        # chunks of positions >= (2R - r) c belong to ranks < r (their second chunk)
        assert covered.sum() == sum((2 * R - r) * (cu[i + 1] - cu[i]) // (2 * R) for i in range(3))


def _item_steps(spans, s0, ns):
    return int(sum(b - a for a, b, _, _ in spans[s0: s0 + ns]))


@pytest.mark.parametrize("name,mask", [("gqa16k", None), ("long128k", None), ("mla32k", None),
                                       ("sparse8", "blockwise"), ("sparse8", "lambda")])
def test_fwd_split_pieces(name, mask):
    """Split forward: with A the average K/V tiles per compute unit (at least 8),
    a Q tile is cut only when it walks more than 4/3 A (more than 8 when A is 8),
    into at most 8 pieces of near-equal length; the workspace holds one fp32 row
    (Dv values + LSE) per piece, head and tile row."""
    w = synth.make_workload(name, mask=mask)
    plan = _plan(w)
    tq, tk, t0, s0 = plan.schedule(0)
    _, _, t3, s3 = plan.schedule(3)
    hpt = 4 if (w.hq // w.hkv) % 4 == 0 else (2 if (w.hq // w.hkv) % 2 == 0 else 1)
    steps0 = {(int(t[0]), int(t[1])): _item_steps(s0, t[3], t[4]) for t in t0}
    total = sum(steps0.values()) * (w.hq // hpt)
    cap = max(8, -(-total // 256))
    cut_above = cap * 4 // 3 if cap > 8 else cap
    pieces = {}
    for t in t3:
        pieces.setdefault((int(t[0]), int(t[1])), []).append(_item_steps(s3, t[3], t[4]))
    assert pieces.keys() == steps0.keys()
    n_slots = 0
    for key, pc in pieces.items():
        assert sum(pc) == steps0[key]
        expect = min(8, -(-steps0[key] // cap)) if steps0[key] > cut_above else 1
        assert len(pc) == expect
        assert max(pc) - min(pc) <= 1
        if len(pc) > 1:
            n_slots += len(pc)
    rows = n_slots * w.hq * tq
    expect_bytes = 0 if n_slots == 0 else (-(-rows * w.d_v * 4 // 256)) * 256 + rows * 4
    assert plan.fwd_workspace_bytes() == expect_bytes
    if name == "sparse8" and mask == "blockwise":
        assert n_slots > 0  # its test-example rows walk 1.37x the per-CU average
    if name == "gqa16k":
        assert n_slots == 0  # its longest tile walks 1.25x the per-CU average


@pytest.mark.parametrize("ci", range(len(MASK_CASES)))
def test_visible_pairs_per_rank_match_oracle(ci):
    """Every rank's visible pairs, reported by one rank's plan (the zig-zag split
    balances sum(q_len*kv_len); sparse masks leave the visible pairs unequal)."""
    import dataclasses
    lens, R, r, mask, ex = MASK_CASES[ci]
    w = _wl(lens, R, r, mask, **ex)
    got = _plan(w).metadata["visible_pairs_per_rank"]
    exp = [oracle.visible_pairs_ref(dataclasses.replace(w, rank=s)) for s in range(R)]
    assert list(got) == exp
    assert got[r] == _plan(w).visible_pairs()
    if mask == "causal":
        assert len(set(exp)) == 1


def test_blockwise_ranks_unequal():
    w = _wl([4096, 2048], 4, 0, "blockwise", block=256, sink=1, window=2)
    per = _plan(w).metadata["visible_pairs_per_rank"]
    assert len(set(per.tolist())) > 1


def test_plan_independent_of_planner_threads(monkeypatch):
    """A large batch (>= 32768 local rows, planned on several threads) gives the
    same metadata and schedules as the single-threaded planner."""
    w = synth.make_workload("sparse8", mask="lambda")

    def build():
        p = cva.Plan(w.cu_seqlens, 1, 0, w.hq, w.hkv, w.d_qk, w.d_v, mask="lambda", sink=w.sink,
                     window=w.window)
        return p, [p.schedule(k) for k in range(4)]

    monkeypatch.setenv("CVA_PLAN_THREADS", "1")
    p1, s1 = build()
    monkeypatch.setenv("CVA_PLAN_THREADS", "8")
    p8, s8 = build()
    assert p1.local_tokens >= 32768
    for key in ("kv_index", "actual_seq_qlen", "actual_seq_kvlen", "visible_pairs_per_rank"):
        assert (p1.metadata[key] == p8.metadata[key]).all(), key
    assert p1.metadata["visible_pairs"] == p8.metadata["visible_pairs"]
    for a, b in zip(s1, s8):
        assert a[0] == b[0] and a[1] == b[1]
        assert (a[2] == b[2]).all() and (a[3] == b[3]).all()
