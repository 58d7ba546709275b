"""Every device table of every plan the GPU tests and the benchmark launch stays
in bounds (CPU only): the five workloads under every mask, every rank of the
packed GQA batch, forced split cuts, random small batches, and every device's
share of block placements."""
import random

import numpy as np
import pytest

import context_varlen_attention_amd as cva
import synth
from tests.plan_check import check_plan_tables
from tests.gpu_helpers import plan_for

WORKLOADS = [("tiny", None), ("gqa16k", None), ("long128k", None), ("mla32k", None),
             ("sparse8", "lambda"), ("sparse8", "shared_prefix"), ("sparse8", "blockwise"),
             ("sparse8", "causal")]


@pytest.mark.parametrize("name,mask", WORKLOADS)
def test_workload_tables_in_bounds(name, mask):
    w = synth.make_workload(name, mask=mask)
    check_plan_tables(plan_for(w), len(w.lengths), w.total_tokens, w.total_tokens // w.cp_size)


@pytest.mark.parametrize("name,cap", [("gqa16k", "8"), ("long128k", "8"), ("long128k", "256"),
                                      ("mla32k", "8"), ("sparse8", "8")])
def test_forced_split_tables_in_bounds(name, cap, monkeypatch):
    monkeypatch.setenv("CVA_FWD_SPLIT_CAP", cap)
    w = synth.make_workload(name)
    plan = plan_for(w)
    assert plan.tables()["n_split_slots"] > 0
    check_plan_tables(plan, len(w.lengths), w.total_tokens, w.total_tokens // w.cp_size)


def test_every_rank_in_bounds():
    w = synth.make_workload("gqa16k")
    for r in range(w.cp_size):
        w.rank = r
        check_plan_tables(plan_for(w), len(w.lengths), w.total_tokens, w.total_tokens // w.cp_size)


@pytest.mark.parametrize("cap", [None, "2"])
@pytest.mark.parametrize("mask", ["causal", "lambda", "blockwise", "shared_prefix"])
def test_random_small_batches_in_bounds(mask, cap, monkeypatch):
    if cap is not None:  # streamed-forward deals of several items per work-group
        monkeypatch.setenv("CVA_FWD_STREAM_WGS", cap)
    rng = random.Random(11)
    for _ in range(12):
        R = rng.choice([1, 2, 3, 4])
        lens = [2 * R * rng.randint(1, 90) for _ in range(rng.randint(1, 5))]
        G = rng.choice([1, 2, 4])
        hkv = rng.choice([1, 2])
        dqk, dv = rng.choice([(64, 64), (128, 128), (192, 128)])
        bb = None
        if mask == "shared_prefix":
            bb = [synth.shared_prefix_bounds(L, prefix=min(L // 2, 64), n_branches=2) for L in lens]
        w = synth.custom_workload(lens, R, rng.randrange(R), G * hkv, hkv, dqk, dv, "bf16", mask=mask,
                                  sink=2, window=rng.choice([1, 3, 50]), branch_bounds=bb,
                                  block=rng.choice([16, 64]))
        check_plan_tables(plan_for(w), len(lens), w.total_tokens, w.total_tokens // R)


@pytest.mark.parametrize("mask", ["causal", "lambda", "shared_prefix", "blockwise"])
def test_placement_share_tables_in_bounds(mask):
    lens = [1280, 640, 2048, 200]
    bb = None
    if mask == "shared_prefix":
        bb = np.array([synth.shared_prefix_bounds(L, prefix=256) for L in lens])
    for R, B, hq, hkv in [(3, 128, 4, 2), (4, 64, 2, 2), (2, 256, 8, 1)]:
        pl = cva.Placement(np.concatenate([[0], np.cumsum(lens)]), R, B, hq=hq, hkv=hkv, d_qk=128,
                           mask=mask, sink=64, window=300 if mask == "lambda" else 2,
                           branch_bounds=bb, mask_block=128)
        for d in range(R):
            check_plan_tables(pl.device_plan(d), len(lens), sum(lens), sum(lens))


def test_random_sweep_tables_in_bounds(monkeypatch):
    """The plans of the seeded random GPU sweep, per-item and streamed deals."""
    from tests.random_cases import N_CASES, random_case
    for seed in range(N_CASES):
        w = random_case(seed)
        for wgs in (None, "1", "3"):
            if wgs is None:
                monkeypatch.delenv("CVA_FWD_STREAM_WGS", raising=False)
            else:
                monkeypatch.setenv("CVA_FWD_STREAM_WGS", wgs)
            check_plan_tables(plan_for(w), len(w.lengths), w.total_tokens,
                              w.total_tokens // w.cp_size)
