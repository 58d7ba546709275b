"""Seeded random batches (tests/random_cases.py) through the forward -- per-item,
with split K/V ranges where the plan cuts, and streamed with a random number of
work-groups -- and the backward, every output element against the fp64 oracle.

Each case mixes CP size and rank, ragged sequence lengths, head shape, mask
parameters and dtype, so shape-dependent mistakes that the hand-picked small
cases miss (an item boundary at an odd place, a tail tile of one row) show up.
"""
import numpy as np
import pytest

import synth
from tests.random_cases import N_CASES, random_case
from tests.test_bwd_gpu import _run as run_bwd
from tests.test_fwd_gpu import _run as run_fwd

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_forward(seed, monkeypatch):
    w = random_case(seed)
    q, k, v = synth.random_tensors(w, 300 + seed, with_dout=False)
    plan = run_fwd(w, q, k, v)
    if plan.fwd_workspace_bytes() > 0:
        run_fwd(w, q, k, v, split=True)
    rng = np.random.default_rng([11, seed])
    monkeypatch.setenv("CVA_FWD_STREAM", "1")
    monkeypatch.setenv("CVA_FWD_STREAM_WGS", str(int(rng.integers(1, 5))))
    run_fwd(w, q, k, v)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_backward(seed):
    w = random_case(seed)
    q, k, v, do = synth.random_tensors(w, 400 + seed)
    run_bwd(w, q, k, v, do)
