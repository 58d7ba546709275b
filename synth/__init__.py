"""Seeded synthetic inputs for packed variable-length attention.

This module only draws numbers: sub-sequence lengths, mask layouts and
Q/K/V/dO tensors at their full, unsplit packed (THD) shapes.  It holds none of
the attention arithmetic and none of the context-parallel split; both the fp64
oracle and the GPU path receive the same arrays from here and do their own
work on them.

The five workloads are named by what they are:

* ``tiny``      -- cu_seqlens [0,64,192,256], CP rank 0 of R=2, 4/4 heads, D=64, fp32.
* ``gqa16k``    -- 16384 packed tokens, log-uniform lengths in [128, 8192],
                   CP rank 1 of R=4, 32/8 heads, D=128, bf16, causal.
* ``long128k``  -- one 131072-token sequence, CP rank 3 of R=8, 32/8 heads,
                   D=128, bf16, causal.
* ``sparse8``   -- 8 sequences, log-normal lengths (median 8192, sigma 0.8),
                   no CP split, 16/16 heads, D=128, bf16; lambda and
                   shared-prefix masks.
* ``mla32k``    -- 32768 packed tokens, uniform lengths in [512, 16384],
                   CP rank 2 of R=4, 16/16 heads, Dqk=192, Dv=128, fwd+bwd.

The long-tailed length mixes stand in for the long-context datasets the DCP
paper evaluates on (its evaluation section, dataset paragraph), which are not
available here.

Tensors are drawn as float32 N(0,1) and then rounded to the working dtype with
round-to-nearest-even; every consumer sees the rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CONFIG_IDS = {"tiny": 1, "gqa16k": 2, "long128k": 3, "sparse8": 4, "mla32k": 5}


@dataclasses.dataclass
class Workload:
    name: str
    cu_seqlens: np.ndarray          # int64 [n+1], starts at 0
    cp_size: int
    rank: int
    hq: int
    hkv: int
    d_qk: int
    d_v: int
    dtype: str                      # "fp32" | "bf16" | "fp16"
    mask: str = "causal"            # "causal" | "lambda" | "shared_prefix" | "blockwise"
    sink: int = 0                   # lambda: tokens; blockwise: blocks
    window: int = 0                 # lambda: tokens; blockwise: blocks
    block: int = 0                  # blockwise: tokens per block
    # shared-prefix layout: per sequence [prefix_end, branch_end_0, ..., branch_end_{B-1}]
    branch_bounds: Optional[np.ndarray] = None
    backward: bool = False

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens)


# ----------------------------------------------------------------------------
# rounding helpers (input quantisation, not attention arithmetic)
# ----------------------------------------------------------------------------

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bf16 bit patterns, round-to-nearest-even (no NaNs expected)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to ``dtype`` and return them as float32 again."""
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(round_to_bf16_bits(x))
    if dtype == "fp16":
        return x.astype(np.float16).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype}")


# ----------------------------------------------------------------------------
# lengths
# ----------------------------------------------------------------------------

def _cu(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int64)


def _lengths_until(total: int, draw, multiple: int) -> list:
    """Draw lengths until their sum reaches ``total``; trim the last to hit it exactly."""
    out, s = [], 0
    while s < total:
        L = int(draw())
        L = multiple * int(math.ceil(L / multiple))
        if s + L >= total:
            L = total - s
        out.append(L)
        s += L
    return out


def shared_prefix_bounds(L: int, prefix: int = 2048, n_branches: int = 4) -> list:
    """Shared-prefix layout for one sequence of length L (a multiple of 128).

    A shared question of ``prefix`` tokens is followed by ``n_branches`` equal
    answers.  Sequences too short to hold the full prefix use the DCP paper's
    20 %-per-answer shape instead (prefix = 128*floor(L/640)).
    """
    P = prefix if L >= prefix + 512 else 128 * (L // 640)
    rest = L - P
    b = rest // n_branches
    ends = [P + (k + 1) * b for k in range(n_branches)]
    ends[-1] = L
    return [P] + ends


def make_workload(name: str, mask: Optional[str] = None, dtype: Optional[str] = None) -> Workload:
    k = CONFIG_IDS[name]
    rng = np.random.default_rng([k, 0])
    if name == "tiny":
        return Workload(name, _cu([64, 128, 64]), 2, 0, 4, 4, 64, 64, dtype or "fp32")
    if name == "gqa16k":
        lo, hi = math.log(128), math.log(8192)
        lens = _lengths_until(16384, lambda: math.exp(rng.uniform(lo, hi)), 8)
        return Workload(name, _cu(lens), 4, 1, 32, 8, 128, 128, dtype or "bf16")
    if name == "long128k":
        return Workload(name, _cu([131072]), 8, 3, 32, 8, 128, 128, dtype or "bf16")
    if name == "sparse8":
        lens = []
        for _ in range(8):
            x = math.exp(rng.normal(math.log(8192), 0.8))
            L = int(128 * np.rint(x / 128))
            lens.append(min(max(L, 1024), 65536))
        m = mask or "lambda"
        w = Workload(name, _cu(lens), 1, 0, 16, 16, 128, 128, dtype or "bf16", mask=m)
        if m == "lambda":
            w.sink, w.window = 64, 4096
        elif m == "blockwise":
            w.block, w.sink, w.window = 256, 1, 2
        elif m == "shared_prefix":
            w.branch_bounds = np.array([shared_prefix_bounds(L) for L in lens], dtype=np.int64)
        return w
    if name == "mla32k":
        lens = _lengths_until(32768, lambda: rng.integers(512, 16384, endpoint=True), 8)
        return Workload(name, _cu(lens), 4, 2, 16, 16, 192, 128, dtype or "bf16", backward=True)
    raise KeyError(name)


def make_tensors(w: Workload, seed_tag: Optional[int] = None, with_dout: bool = True):
    """Full unsplit Q [T,Hq,Dqk], K [T,Hkv,Dqk], V [T,Hkv,Dv], dO [T,Hq,Dv] as float32.

    Each tensor has its own stream ``default_rng([k, 1, t])`` (t = 0..3 for
    Q, K, V, dO), so one can be drawn without the others.  Values are rounded
    to the workload dtype before they are returned.
    """
    k = CONFIG_IDS.get(w.name, 0) if seed_tag is None else seed_tag
    T = w.total_tokens
    shapes = [(T, w.hq, w.d_qk), (T, w.hkv, w.d_qk), (T, w.hkv, w.d_v), (T, w.hq, w.d_v)]
    out = []
    for t, shp in enumerate(shapes if with_dout else shapes[:3]):
        g = np.random.default_rng([k, 1, t])
        out.append(quantize(g.standard_normal(shp, dtype=np.float32), w.dtype))
    return out


def custom_workload(lengths, cp_size, rank, hq, hkv, d_qk, d_v, dtype="bf16", mask="causal",
                    sink=0, window=0, branch_bounds=None, name="custom", block=0) -> Workload:
    w = Workload(name, _cu(lengths), cp_size, rank, hq, hkv, d_qk, d_v, dtype, mask=mask,
                 sink=sink, window=window, block=block)
    if branch_bounds is not None:
        w.branch_bounds = np.asarray(branch_bounds, dtype=np.int64)
    return w


def random_tensors(w: Workload, seed: int, with_dout: bool = True):
    """Like :func:`make_tensors` but keyed by an explicit integer seed."""
    return make_tensors(w, seed_tag=1000 + int(seed), with_dout=with_dout)
