"""Shared helpers for the GPU parity tests.

GPU-side inputs are laid out with libcva's own metadata (local rows of the
rank, rank-major gathered K/V); the oracle splits the same full tensors with its
own enumeration.  Tolerances: MindSpeed RFC section 3.5.1 (fp16 atol = rtol =
5e-3, bf16 atol = rtol = 2.5e-2); fp32 uses 1e-4 (no page value; the kernel
accumulates in fp32 so its error is far below that).
"""
import numpy as np

import context_varlen_attention_amd as cva

TOL = {"bf16": 2.5e-2, "fp16": 5e-3, "fp32": 1e-4}


def torch_dtype(dt):
    import torch
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dt]


def plan_for(w):
    bb = None if w.branch_bounds is None else np.asarray(w.branch_bounds)
    return cva.Plan(w.cu_seqlens, w.cp_size, w.rank, w.hq, w.hkv, w.d_qk, w.d_v, w.dtype,
                    mask=w.mask, sink=w.sink, window=w.window, branch_bounds=bb, block=w.block)


def device_inputs(w, q, k, v, do=None, device="cuda"):
    """Local q / dO rows and rank-major K/V on the GPU, laid out by libcva's metadata."""
    import torch
    dt = torch_dtype(w.dtype)
    loc = cva.local_token_ids(w.cu_seqlens, w.cp_size, w.rank)
    rm = cva.rank_major_token_ids(w.cu_seqlens, w.cp_size)
    out = [torch.from_numpy(np.ascontiguousarray(q[loc])).to(device=device, dtype=dt),
           torch.from_numpy(np.ascontiguousarray(k[rm])).to(device=device, dtype=dt),
           torch.from_numpy(np.ascontiguousarray(v[rm])).to(device=device, dtype=dt)]
    if do is not None:
        out.append(torch.from_numpy(np.ascontiguousarray(do[loc])).to(device=device, dtype=dt))
    return out


def assert_close(got, ref, dtype, what):
    """Element-wise |got - ref| <= tol + tol * |ref| (numpy.allclose semantics)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    tol = TOL[dtype]
    finite = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), finite), f"{what}: non-finite pattern differs"
    err = np.abs(got[finite] - ref[finite])
    bound = tol + tol * np.abs(ref[finite])
    bad = err > bound
    if bad.any():
        idx = np.argmax(err - bound)
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{err.size} elements outside tol {tol}; worst err "
            f"{err[idx]:.3e} (ref {ref[finite][idx]:.4f}); max err {err.max():.3e}")
    return float(err.max()) if err.size else 0.0
