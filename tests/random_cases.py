"""Seeded random batches for the parity sweeps (CPU plan checks and GPU parity).

Each case draws, from its own seed: the CP size R and rank, one to five
sub-sequences (multiples of 2R; about a third under 48 tokens, the rest up
to ~1200, so 1-tile items, items shorter than a tile and ragged tails occur), a head shape (GQA groups of 1, 2 and 4; Q/K head dims 64,
128 and 192), a mask with its parameters (lambda sink and window, shared-prefix
bounds with empty and full branches allowed, blockwise block / sink / window
in blocks) and a 16-bit dtype.
"""
import numpy as np

import synth

N_CASES = 32
SHAPES = [(4, 4, 64, 64), (4, 2, 128, 128), (8, 2, 128, 128), (4, 1, 128, 128), (2, 2, 192, 128),
          (4, 4, 192, 128)]
MASKS = ["causal", "lambda", "shared_prefix", "blockwise"]


def random_case(seed: int):
    """The workload of case ``seed`` (a synth.Workload)."""
    rng = np.random.default_rng([7, int(seed)])
    R = int(rng.integers(1, 5))
    r = int(rng.integers(0, R))
    n = int(rng.integers(1, 6))
    lens = [int(2 * R * rng.integers(1, 1 + (48 if rng.random() < 0.3 else 1200) // (2 * R)))
            for _ in range(n)]
    hq, hkv, dqk, dv = SHAPES[int(rng.integers(0, len(SHAPES)))]
    mask = MASKS[int(rng.integers(0, len(MASKS)))]
    dtype = ["bf16", "fp16"][int(rng.integers(0, 2))]
    kw = {}
    if mask == "lambda":
        kw = dict(sink=int(rng.integers(0, 65)), window=int(rng.integers(1, 513)))
    elif mask == "blockwise":
        kw = dict(block=int(rng.choice([32, 64, 80, 96, 128])), sink=int(rng.integers(0, 3)),
                  window=int(rng.integers(1, 4)))
    elif mask == "shared_prefix":
        nb = int(rng.integers(1, 5))
        bounds = []
        for L in lens:
            cuts = np.sort(rng.integers(0, L + 1, size=nb))
            bounds.append([int(c) for c in cuts] + [L])
        kw = dict(branch_bounds=bounds)
    return synth.custom_workload(lens, R, r, hq, hkv, dqk, dv, dtype, mask=mask, name=f"rand{seed}", **kw)
