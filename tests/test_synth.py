"""The seeded workload generators produce the shapes and structure they promise."""
import numpy as np
import pytest

import synth


@pytest.mark.parametrize("name", list(synth.CONFIG_IDS))
def test_lengths_are_aligned(name):
    w = synth.make_workload(name)
    L = w.lengths
    assert (L > 0).all()
    assert (L % (2 * w.cp_size) == 0).all()
    assert 0 <= w.rank < w.cp_size and w.hq % w.hkv == 0


def test_totals_and_ranges():
    w = synth.make_workload("gqa16k")
    assert w.total_tokens == 16384 and (w.lengths % 8 == 0).all() and w.lengths.max() <= 8192
    assert (w.lengths[:-1] >= 128).all()
    w = synth.make_workload("mla32k")
    assert w.total_tokens == 32768 and (w.lengths[:-1] >= 512).all() and w.lengths.max() <= 16384
    w = synth.make_workload("long128k")
    assert w.total_tokens == 131072 and w.cp_size == 8 and w.rank == 3
    w = synth.make_workload("sparse8")
    assert len(w.lengths) == 8 and (w.lengths % 128 == 0).all()
    assert w.lengths.min() >= 1024 and w.lengths.max() <= 65536
    w2 = synth.make_workload("sparse8", mask="shared_prefix")
    assert (w2.branch_bounds[:, -1] == w2.lengths).all()


def test_generation_is_seeded_and_rounded():
    w = synth.make_workload("tiny", dtype="bf16")
    a = synth.make_tensors(w)
    b = synth.make_tensors(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # bf16 values have their low 16 mantissa bits clear
    assert (a[0].view(np.uint32) & 0xFFFF == 0).all()
    w16 = synth.make_workload("tiny", dtype="fp16")
    q = synth.make_tensors(w16)[0]
    assert np.array_equal(q, q.astype(np.float16).astype(np.float32))


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5], dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.round_to_bf16_bits(x))
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa (1.0) wins;
    # 1+3*2^-8 ties between 1+2^-7 and 1+2^-6: even (1+2^-6) wins.
    assert got.tolist() == [1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5]
