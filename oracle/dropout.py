"""Attention dropout: the keep mask of every (sequence, head, query, key), fp64 side.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Reading.  MindSpeed RFC section 3.5.2.2 (interface
AttnFuncWithCPAndKVAllGatherForTHDLoadBalanced) takes an attention dropout
probability p in [0, 1) and says nothing more: not the generator, not where
the mask applies.  The plain reading is the usual attention dropout: every
softmax probability P[q, k] is kept with probability 1 - p and scaled by
1 / (1 - p), or set to zero, before it multiplies V; the row normaliser and the
LSE are those of the undropped softmax; the backward uses the same mask, so

    O = (D * P / (1 - p)) V,   dV = (D * P / (1 - p))^T dO,
    dP = D * (dO V^T) / (1 - p),   dS = P * (dP - rowsum(dP * P)),

with D the 0/1 keep mask (the softmax Jacobian of the undropped P, with the
dropped entries' upstream gradient zero).

Random bits.  A counter-based generator, so that any element's decision can be
formed where it is needed, in any order, by both this oracle and the kernels:
Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC 2011, section on the Philox family):
a 128-bit counter (four 32-bit words) and a 64-bit key (two words) go through
ten rounds; each round multiplies words 0 and 2 by the constants 0xD2511F53 and
0xCD9E8D57 into 64-bit products and forms the new words

    (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0)),

and the key is advanced between rounds by the Weyl increments 0x9E3779B9 and
0xBB67AE85.

Element layout (this library's choice).  Key = (seed mod 2^32, seed div 2^32).
Counter = (k div 4, q div 4, head, sequence index), with q and k the in-sequence
positions of the query and the key, so that the mask depends neither on the
context-parallel split nor on how the work is tiled.  One call thus covers a
4 x 4 block of (query, key) pairs: output word q mod 4, byte k mod 4 (bits
8 (k mod 4) ..  + 7) is the element's random byte u, and the element is kept iff
u >= t with t = round(256 p) clamped to [0, 255].  The realised drop
probability is t / 256 and kept values are scaled by 256 / (256 - t) (exactly
unbiased for the realised probability).

Parity: pinned (tests/test_oracle_dropout.py -- published known-answer vectors
of Philox4x32-10; drop fraction, byte uniformity and independence across heads,
sequences and seeds; unbiasedness over many seeds; p = 0 reducing to plain
attention; torch float64 autograd through the defining expression; central
finite differences of the dropped loss; independence of the CP split).
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1, rounds=10):
    """Philox4x32 over arrays of counter words (any broadcastable shapes of
    integers below 2^32) with the 32-bit key (k0, k1); returns four uint64
    arrays holding the 32-bit output words."""
    x = [np.asarray(c, dtype=np.uint64) & np.uint64(MASK32) for c in (c0, c1, c2, c3)]
    x = list(np.broadcast_arrays(*x))
    key0, key1 = int(k0) & MASK32, int(k1) & MASK32
    m0, m1, lo32 = np.uint64(M0), np.uint64(M1), np.uint64(MASK32)
    for r in range(rounds):
        p0 = m0 * x[0]           # < 2^64: no overflow
        p1 = m1 * x[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & lo32
        hi1, lo1 = p1 >> np.uint64(32), p1 & lo32
        x = [hi1 ^ x[1] ^ np.uint64(key0), lo1, hi0 ^ x[3] ^ np.uint64(key1), lo0]
        key0 = (key0 + W0) & MASK32
        key1 = (key1 + W1) & MASK32
    return x


def threshold(p):
    """The byte threshold t for drop probability p in [0, 1): round(256 p) in [0, 255]."""
    p = float(p)
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(255, int(np.floor(256.0 * p + 0.5)))


def keep_scale(p):
    """1 / (1 - realised drop probability) = 256 / (256 - t)."""
    return 256.0 / (256.0 - threshold(p))


def random_bytes(seq, head, qpos, kpos, seed):
    """The random byte of every (query position, key position) pair of one
    sequence and head: array of shape (len(qpos), len(kpos)).  The generator
    runs once per 4 x 4 block that the positions touch."""
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    seed = int(seed)
    qb, qi = np.unique(qpos >> 2, return_inverse=True)
    kb, ki = np.unique(kpos >> 2, return_inverse=True)
    words = np.stack(philox4x32_10(kb[None, :], qb[:, None], head, seq, seed & MASK32, (seed >> 32) & MASK32))
    w = words[(qpos & 3)[:, None], qi[:, None], ki[None, :]]  # word q % 4 of the pair's block
    return (w >> (np.uint64(8) * (kpos & 3).astype(np.uint64))[None, :]) & np.uint64(0xFF)


def keep_mask(seq, head, qpos, kpos, p, seed):
    """Boolean keep mask D[q, k] of one sequence and head (True = kept)."""
    return random_bytes(seq, head, qpos, kpos, seed) >= np.uint64(threshold(p))
