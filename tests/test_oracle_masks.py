"""Pins for the oracle's mask predicates (CPU only).

Small masks are written out by hand from the DCP paper's descriptions (sparse
masks, Fig. 6(b) lambda = attention sink + sliding window; Fig. 6(c) causal
blockwise; Fig. 6(d) shared question); degenerate settings must reduce to the
causal mask; pair counts must match closed forms.
"""
import numpy as np
import pytest

import synth
from oracle.masks import mask_ref, visible_pairs_ref


def _m(rows):
    return np.array([[c == "1" for c in r] for r in rows], dtype=bool)


def test_causal_small():
    exp = _m(["1000", "1100", "1110", "1111"])
    assert (mask_ref("causal", 4) == exp).all()


def test_lambda_small():
    # L=8, sink=2, window=3: row q sees k<2 and q-2<=k<=q.
    exp = _m([
        "10000000",
        "11000000",
        "11100000",
        "11110000",
        "11111000",
        "11011100",
        "11001110",
        "11000111",
    ])
    assert (mask_ref("lambda", 8, sink=2, window=3) == exp).all()


def test_shared_prefix_small():
    # L=10: question 0..3, answer A 4..6, answer B 7..9.
    exp = _m([
        "1000000000",
        "1100000000",
        "1110000000",
        "1111000000",
        "1111100000",
        "1111110000",
        "1111111000",
        "1111000100",
        "1111000110",
        "1111000111",
    ])
    assert (mask_ref("shared_prefix", 10, bounds=[4, 7, 10]) == exp).all()


def test_blockwise_small():
    # L=11, blocks of 2 (the last block, position 10, is the test example),
    # one sink block, a window of 2 blocks (the own block and the one before)
    exp = _m([
        "10000000000",
        "11000000000",
        "11100000000",
        "11110000000",
        "11111000000",
        "11111100000",
        "11001110000",
        "11001111000",
        "11000011100",
        "11000011110",
        "11111111111",
    ])
    assert (mask_ref("blockwise", 11, sink=1, window=2, block=2) == exp).all()


@pytest.mark.parametrize("L", [1, 5, 33, 128])
def test_blockwise_degenerate_reduce_to_causal(L):
    c = mask_ref("causal", L)
    assert (mask_ref("blockwise", L, sink=0, window=L, block=1) == c).all()   # window covers all
    assert (mask_ref("blockwise", L, sink=L, window=1, block=1) == c).all()   # all blocks are sinks
    assert (mask_ref("blockwise", L, sink=0, window=1, block=L) == c).all()   # one block = the test block


def test_blockwise_row_counts_closed_form():
    L, B, S, W = 1000, 64, 1, 2
    M = mask_ref("blockwise", L, sink=S, window=W, block=B)
    last = (L - 1) // B
    for q in range(L):
        b = q // B
        if b == last:
            exp = q + 1
        else:
            sink_end = min(S * B, q + 1)
            ws = max(0, (b - W + 1) * B)
            exp = q + 1 if ws <= sink_end else sink_end + (q + 1 - ws)
        assert M[q].sum() == exp


@pytest.mark.parametrize("L", [1, 5, 33, 128])
def test_degenerate_reduce_to_causal(L):
    c = mask_ref("causal", L)
    assert (mask_ref("lambda", L, sink=0, window=L) == c).all()
    assert (mask_ref("lambda", L, sink=L, window=1) == c).all()
    assert (mask_ref("shared_prefix", L, bounds=[0, L]) == c).all()
    assert (mask_ref("shared_prefix", L, bounds=[L // 2, L]) == c).all()


def test_lambda_row_counts_closed_form():
    L, S, W = 700, 64, 256
    M = mask_ref("lambda", L, sink=S, window=W)
    for q in range(L):
        exp = q + 1 if q < W else W + min(S, q - W + 1)
        assert M[q].sum() == exp


def test_shared_prefix_count_closed_form():
    L = 2048 + 4 * 640
    b = synth.shared_prefix_bounds(L)
    M = mask_ref("shared_prefix", L, bounds=b)
    P = b[0]
    exp = P * (P + 1) // 2
    start = P
    for end in b[1:]:
        n = end - start
        exp += n * P + n * (n + 1) // 2
        start = end
    assert M.sum() == exp


@pytest.mark.parametrize("R", [2, 4])
def test_causal_pairs_equal_per_rank(R):
    lens = [2 * R * c for c in (3, 17, 5, 40)]
    total = sum(L * (L + 1) for L in lens) // (2 * R)
    for r in range(R):
        w = synth.custom_workload(lens, R, r, 1, 1, 8, 8)
        assert visible_pairs_ref(w) == total


def test_shared_prefix_bounds_layout():
    for L in (1024, 1280, 2560, 8192, 65536):
        b = synth.shared_prefix_bounds(L)
        assert b[-1] == L and len(b) == 5
        assert b[0] == (2048 if L >= 2560 else 128 * (L // 640))
        widths = np.diff(b)
        assert (widths == widths[0]).all() and widths[0] % 32 == 0
