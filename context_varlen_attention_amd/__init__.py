"""Python binding of libcva: one context-parallel rank's share of packed
variable-length attention on MI355X.

This module only marshals arguments to the C ABI declared in ``include/cva.h``
(ctypes); every step of the computation runs in libcva's C++ host code and HIP
kernels.  PyTorch provides device memory and the current stream.  If the
library has not been built the first call raises; there is no fallback path.

Names follow the C ABI:

* :class:`Plan`      -- ``cva_plan_create`` / ``cva_plan_get_metadata`` /
                        ``cva_plan_upload`` / ``cva_plan_get_schedule``
* :func:`fwd`        -- ``cva_fwd``
* :func:`bwd`        -- ``cva_bwd``
  (both with ``dropout_p=``: ``cva_fwd_dropout`` / ``cva_bwd_dropout``)
* :func:`local_token_ids`, :func:`rank_major_token_ids` -- the symmetric split
  and the rank-major order, read from the library's metadata (what a data
  loader and the K/V all-gather would produce).
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

__all__ = ["Plan", "Placement", "PlacedPlan", "fwd", "bwd", "bwd_noalloc", "CvaError", "local_token_ids",
           "rank_major_token_ids", "library_path", "load_library", "timing_enable", "timing_read",
           "timing_select"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# CVA_LIBRARY selects another build of the same library (e.g. the host-sanitized
# one the CPU tests use); by default the in-tree libcva.so next to this file.
_LIB_PATH = os.environ.get("CVA_LIBRARY") or os.path.join(_HERE, "libcva.so")
_lib = None

DTYPES = {"bf16": 0, "fp16": 1, "fp32": 2}
MASKS = {"causal": 0, "lambda": 1, "shared_prefix": 2, "blockwise": 3}
STATUS = {
    0: "CVA_OK", 1: "CVA_E_ARG", 2: "CVA_E_CU_SEQLENS", 3: "CVA_E_ALIGN", 4: "CVA_E_RANK",
    5: "CVA_E_HEADS", 6: "CVA_E_HEADDIM", 7: "CVA_E_DTYPE", 8: "CVA_E_MASK",
    9: "CVA_E_UNSUPPORTED", 10: "CVA_E_WORKLOAD", 11: "CVA_E_HIP", 12: "CVA_E_SCALE",
    13: "CVA_E_WORKSPACE", 14: "CVA_E_NOT_UPLOADED",
}


class CvaError(AssertionError):
    """A libcva call returned an error status (an AssertionError, as the RFC's
    interfaces raise on invalid input)."""

    def __init__(self, status, message):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


class _MaskDesc(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("sink", ctypes.c_int32), ("window", ctypes.c_int32),
                ("n_branches", ctypes.c_int32), ("branch_bounds", ctypes.POINTER(ctypes.c_int32)),
                ("block", ctypes.c_int32)]


_P32 = ctypes.POINTER(ctypes.c_int32)
_P64 = ctypes.POINTER(ctypes.c_int64)


class _Metadata(ctypes.Structure):
    _fields_ = [("local_tokens", ctypes.c_int64), ("global_tokens", ctypes.c_int64),
                ("n_seqs", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("cp_size", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("local_cu", _P32), ("actual_seq_qlen", _P32), ("actual_seq_kvlen", _P32),
                ("kv_index", _P32), ("seg_q_pos0", _P32), ("kv_index_len", ctypes.c_int64),
                ("workload_per_rank", _P64), ("visible_pairs", ctypes.c_int64),
                ("fwd_tiles", ctypes.c_int64), ("visible_pairs_per_rank", _P64)]


class _Schedule(ctypes.Structure):
    _fields_ = [("tile_q", ctypes.c_int32), ("tile_kv", ctypes.c_int32),
                ("n_tiles", ctypes.c_int32), ("n_spans", ctypes.c_int32),
                ("tiles", _P32), ("spans", _P32)]


class _Tables(ctypes.Structure):
    _fields_ = [("n_segs", ctypes.c_int32), ("segs", _P32), ("kv_index_len", ctypes.c_int64),
                ("kv_index", _P32), ("n_rows", ctypes.c_int64), ("row_iv", _P32),
                ("n_zero_ranges", ctypes.c_int32), ("zero_rows", _P32),
                ("n_split_items", ctypes.c_int32), ("split_slot", _P32),
                ("n_combine", ctypes.c_int32), ("split_combine", _P32),
                ("n_split_slots", ctypes.c_int32),
                ("fwd_deal_wgs", ctypes.c_int32), ("fwd_deal_start", _P32),
                ("fwd_deal_items", _P32), ("n_fwd_deal_items", ctypes.c_int32),
                ("split_deal_wgs", ctypes.c_int32), ("split_deal_start", _P32),
                ("split_deal_items", _P32), ("n_split_deal_items", ctypes.c_int32)]


class _PlacementInfo(ctypes.Structure):
    _fields_ = [("n_devices", ctypes.c_int32), ("block", ctypes.c_int32),
                ("n_data_blocks", ctypes.c_int32), ("n_comp_blocks", ctypes.c_int32),
                ("data_blocks", _P32), ("comp_blocks", _P32), ("comp_pairs", _P64),
                ("device_tokens", _P64), ("device_pairs", _P64), ("device_send_bytes", _P64),
                ("device_recv_bytes", _P64), ("total_comm_bytes", ctypes.c_int64),
                ("block_comm_bytes", ctypes.c_int64), ("zigzag_valid", ctypes.c_int32),
                ("zigzag_pairs", _P64), ("zigzag_comm_bytes", ctypes.c_int64)]


EXPORTS = ["cva_last_error", "cva_plan_create", "cva_plan_destroy", "cva_plan_get_metadata",
           "cva_plan_device_bytes", "cva_plan_upload", "cva_fwd", "cva_fwd_workspace_bytes",
           "cva_fwd_split", "cva_bwd_workspace_bytes",
           "cva_bwd", "cva_plan_get_schedule", "cva_timing_enable", "cva_timing_read", "cva_timing_select",
           "cva_placement_create", "cva_placement_get", "cva_placement_destroy",
           "cva_bwd_noalloc_max_bytes", "cva_bwd_noalloc", "cva_placement_plan_create",
           "cva_plan_get_tables", "cva_fwd_dropout", "cva_bwd_dropout"]

# timing ids of cva_timing_read; ids 1 and 2 are reserved (formerly separate
# Delta and zero-fill launches, now part of the dQ kernel)
KERNEL_NAMES = ["fwd", "reserved1", "reserved2", "bwd_dkdv", "bwd_dq", "fwd_merge"]


class _KernelTimes(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * 6), ("total_ms", ctypes.c_double * 6)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libcva.so (raises RuntimeError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m context_varlen_attention_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
    L.cva_last_error.restype = ctypes.c_char_p
    L.cva_last_error.argtypes = []
    L.cva_plan_create.restype = i32
    L.cva_plan_create.argtypes = [_P32, i32, i32, i32, ctypes.POINTER(_MaskDesc), i32, i32, i32,
                                  i32, i32, ctypes.POINTER(vp)]
    L.cva_plan_destroy.restype = None
    L.cva_plan_destroy.argtypes = [vp]
    L.cva_plan_get_metadata.restype = i32
    L.cva_plan_get_metadata.argtypes = [vp, ctypes.POINTER(_Metadata)]
    L.cva_plan_device_bytes.restype = sz
    L.cva_plan_device_bytes.argtypes = [vp]
    L.cva_plan_upload.restype = i32
    L.cva_plan_upload.argtypes = [vp, vp, sz, vp]
    L.cva_fwd.restype = i32
    L.cva_fwd.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp]
    L.cva_fwd_workspace_bytes.restype = sz
    L.cva_fwd_workspace_bytes.argtypes = [vp]
    L.cva_fwd_split.restype = i32
    L.cva_fwd_split.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, sz, vp]
    L.cva_bwd_workspace_bytes.restype = sz
    L.cva_fwd_dropout.restype = i32
    L.cva_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, f32, f32, ctypes.c_uint64, vp, sz, vp]
    L.cva_bwd_dropout.restype = i32
    L.cva_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, f32, f32, ctypes.c_uint64,
                                  vp]
    L.cva_bwd_workspace_bytes.argtypes = [vp]
    L.cva_bwd.restype = i32
    L.cva_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, f32, vp]
    L.cva_bwd_noalloc_max_bytes.restype = sz
    L.cva_bwd_noalloc_max_bytes.argtypes = []
    L.cva_bwd_noalloc.restype = i32
    L.cva_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp]
    L.cva_plan_get_tables.restype = i32
    L.cva_plan_get_tables.argtypes = [vp, ctypes.POINTER(_Tables)]
    L.cva_plan_get_schedule.restype = i32
    L.cva_plan_get_schedule.argtypes = [vp, i32, ctypes.POINTER(_Schedule)]
    L.cva_timing_enable.restype = i32
    L.cva_timing_enable.argtypes = [i32]
    L.cva_timing_read.restype = i32
    L.cva_timing_read.argtypes = [ctypes.POINTER(_KernelTimes)]
    L.cva_timing_select.restype = i32
    L.cva_timing_select.argtypes = [ctypes.c_uint32]
    L.cva_placement_create.restype = i32
    L.cva_placement_create.argtypes = [_P32, i32, ctypes.POINTER(_MaskDesc), i32, i32, i32, i32,
                                       i32, i32, i32, ctypes.c_double, ctypes.POINTER(vp)]
    L.cva_placement_get.restype = i32
    L.cva_placement_get.argtypes = [vp, ctypes.POINTER(_PlacementInfo)]
    L.cva_placement_plan_create.restype = i32
    L.cva_placement_plan_create.argtypes = [vp, i32, ctypes.POINTER(vp)]
    L.cva_placement_destroy.restype = None
    L.cva_placement_destroy.argtypes = [vp]
    _lib = L
    return L


def _check(status):
    if status != 0:
        msg = load_library().cva_last_error().decode(errors="replace")
        raise CvaError(status, msg)


def _arr(ptr, n, dtype):
    if n == 0:
        return np.zeros(0, dtype=dtype)
    return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dtype, copy=True)


class _PlanBase:
    """A libcva plan handle: schedules, device copy (shared by Plan and PlacedPlan)."""

    _h = None
    _dev = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.cva_plan_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def schedule(self, which):
        """(tile_q, tile_kv, tiles [n,5], spans [m,4]) of schedule 0 fwd, 1 dQ, 2 dK/dV,
        3 forward with split K/V ranges."""
        s = _Schedule()
        _check(load_library().cva_plan_get_schedule(self._h, int(which), ctypes.byref(s)))
        tiles = _arr(s.tiles, s.n_tiles * 5, np.int64).reshape(-1, 5)
        spans = _arr(s.spans, s.n_spans * 4, np.int64).reshape(-1, 4)
        return s.tile_q, s.tile_kv, tiles, spans

    def tables(self):
        """``cva_plan_get_tables``: the plan's other device tables as numpy arrays."""
        t = _Tables()
        _check(load_library().cva_plan_get_tables(self._h, ctypes.byref(t)))
        return {
            "segs": _arr(t.segs, t.n_segs * 8, np.int64).reshape(-1, 8),
            "kv_index": _arr(t.kv_index, t.kv_index_len, np.int64),
            "row_iv": _arr(t.row_iv, t.n_rows * 4, np.int64).reshape(-1, 4),
            "zero_rows": _arr(t.zero_rows, t.n_zero_ranges * 2, np.int64).reshape(-1, 2),
            "split_slot": _arr(t.split_slot, t.n_split_items, np.int64),
            "split_combine": _arr(t.split_combine, t.n_combine * 5, np.int64).reshape(-1, 5),
            "n_split_slots": int(t.n_split_slots),
            "fwd_deal": (int(t.fwd_deal_wgs),
                         _arr(t.fwd_deal_start, t.fwd_deal_wgs + 1 if t.fwd_deal_wgs else 0, np.int64),
                         _arr(t.fwd_deal_items, t.n_fwd_deal_items, np.int64)),
            "split_deal": (int(t.split_deal_wgs),
                           _arr(t.split_deal_start, t.split_deal_wgs + 1 if t.split_deal_wgs else 0, np.int64),
                           _arr(t.split_deal_items, t.n_split_deal_items, np.int64)),
        }

    def fwd_workspace_bytes(self):
        """Bytes of the workspace ``cva_fwd_split`` needs (0: the plan splits nothing)."""
        return int(load_library().cva_fwd_workspace_bytes(self._h))

    def device_bytes(self):
        return int(load_library().cva_plan_device_bytes(self._h))

    def upload(self, device=None, stream=None):
        """Copy the plan tables into a torch uint8 buffer on ``device`` and bind them
        (asynchronously, on ``stream``; launches on other streams wait for the copy)."""
        import torch
        dev = torch.device("cuda") if device is None else torch.device(device)
        s = torch.cuda.current_stream(dev) if stream is None else stream
        nbytes = self.device_bytes()
        with torch.cuda.stream(s):
            buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
        off = (-buf.data_ptr()) % 256
        view = buf[off: off + nbytes]
        _check(load_library().cva_plan_upload(self._h, ctypes.c_void_p(view.data_ptr()),
                                              nbytes, ctypes.c_void_p(s.cuda_stream)))
        ready = torch.cuda.Event()
        ready.record(s)
        self._dev = buf  # keep alive while the plan is used
        self._dev_stream, self._dev_ready = s, ready
        return self

    def _bind_stream(self, s):
        """Order a launch on stream ``s`` after the upload, and keep the table buffer
        from being reused while ``s`` may still read it."""
        if s != self._dev_stream:
            s.wait_event(self._dev_ready)
            self._dev.record_stream(s)

    @property
    def uploaded(self):
        return self._dev is not None


class Plan(_PlanBase):
    """Host plan of one rank: metadata + tile schedules (``cva_plan_create``).

    ``branch_bounds``: shared-prefix layout, int [n_seqs][n_branches+1] of
    in-sequence positions {prefix_end, answer ends...}.
    """

    def __init__(self, cu_seqlens, cp_size, rank, hq, hkv, d_qk, d_v=None, dtype="bf16",
                 mask="causal", sink=0, window=0, branch_bounds=None, block=0):
        L = load_library()
        d_v = d_qk if d_v is None else d_v
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        if cu.ndim != 1:
            raise CvaError(1, "cu_seqlens must be 1-D")
        if cu.size and (cu.max() > np.iinfo(np.int32).max or cu.min() < np.iinfo(np.int32).min):
            raise CvaError(1, "cu_seqlens out of int32 range")
        self._cu = np.ascontiguousarray(cu.astype(np.int32))
        if dtype not in DTYPES:
            raise CvaError(7, f"unknown dtype {dtype!r}")
        if mask not in MASKS:
            raise CvaError(8, f"unknown mask {mask!r}")
        self.cp_size, self.rank = int(cp_size), int(rank)
        self.hq, self.hkv, self.d_qk, self.d_v = int(hq), int(hkv), int(d_qk), int(d_v)
        self.dtype, self.mask = dtype, mask
        md = _MaskDesc(MASKS[mask], int(sink), int(window), 0, None, int(block))
        self._bounds = None
        if branch_bounds is not None:
            bb = np.ascontiguousarray(np.asarray(branch_bounds, dtype=np.int32))
            if bb.ndim != 2:
                raise CvaError(8, "branch_bounds must be 2-D [n_seqs][n_branches+1]")
            self._bounds = bb
            md.n_branches = bb.shape[1] - 1
            md.branch_bounds = bb.ctypes.data_as(_P32)
        handle = ctypes.c_void_p()
        n_seqs = max(int(self._cu.size) - 1, 0)
        cu_ptr = self._cu.ctypes.data_as(_P32) if self._cu.size else None
        self._h = None
        _check(L.cva_plan_create(cu_ptr, n_seqs, self.cp_size, self.rank, ctypes.byref(md),
                                 self.hq, self.hkv, self.d_qk, self.d_v, DTYPES[dtype],
                                 ctypes.byref(handle)))
        self._h = handle
        self._dev = None
        m = _Metadata()
        _check(L.cva_plan_get_metadata(self._h, ctypes.byref(m)))
        nseg = m.n_segments
        self.local_tokens = int(m.local_tokens)
        self.global_tokens = int(m.global_tokens)
        self.metadata = {
            "local_tokens": int(m.local_tokens),
            "global_tokens": int(m.global_tokens),
            "local_cu": _arr(m.local_cu, m.n_seqs + 1, np.int64),
            "actual_seq_qlen": _arr(m.actual_seq_qlen, nseg + 1, np.int64),
            "actual_seq_kvlen": _arr(m.actual_seq_kvlen, nseg + 1, np.int64),
            "kv_index": _arr(m.kv_index, m.kv_index_len, np.int64),
            "seg_q_pos0": _arr(m.seg_q_pos0, nseg, np.int64),
            "workload_per_rank": _arr(m.workload_per_rank, m.cp_size, np.int64),
            "visible_pairs": int(m.visible_pairs),
            "fwd_tiles": int(m.fwd_tiles),
            "visible_pairs_per_rank": _arr(m.visible_pairs_per_rank, m.cp_size, np.int64),
        }

    @property
    def cu_seqlens(self):
        return self._cu.astype(np.int64)

    def visible_pairs(self):
        return self.metadata["visible_pairs"]


def _mask_desc(mask, sink, window, branch_bounds, block):
    """(_MaskDesc, bounds array kept alive by the caller)."""
    if mask not in MASKS:
        raise CvaError(8, f"unknown mask {mask!r}")
    md = _MaskDesc(MASKS[mask], int(sink), int(window), 0, None, int(block))
    bb = None
    if branch_bounds is not None:
        bb = np.ascontiguousarray(np.asarray(branch_bounds, dtype=np.int32))
        if bb.ndim != 2:
            raise CvaError(8, "branch_bounds must be 2-D [n_seqs][n_branches+1]")
        md.n_branches = bb.shape[1] - 1
        md.branch_bounds = bb.ctypes.data_as(_P32)
    return md, bb


class Placement:
    """Block placement of a packed batch over ``n_devices`` (``cva_placement_create``).

    Attributes (numpy): ``data_blocks`` [n,4] {sequence, first token, tokens, device},
    ``comp_blocks`` [m,4] {sequence, q block, k/v block, device}, ``comp_pairs`` [m],
    ``device_tokens`` / ``device_pairs`` / ``device_send_bytes`` / ``device_recv_bytes``
    [n_devices], ``total_comm_bytes`` (connectivity volume), ``block_comm_bytes``
    (per-computation-block volume), ``zigzag_pairs`` [n_devices] or None when some
    sequence length does not divide by ``2 * n_devices``, ``zigzag_comm_bytes``.
    ``mask_block`` is the blockwise mask's block size; ``block`` the placement's.
    """

    def __init__(self, cu_seqlens, n_devices, block, hq=1, hkv=1, d_qk=128, d_v=None,
                 dtype="bf16", mask="causal", sink=0, window=0, branch_bounds=None,
                 mask_block=0, epsilon=0.1):
        L = load_library()
        d_v = d_qk if d_v is None else d_v
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        if cu.ndim != 1:
            raise CvaError(1, "cu_seqlens must be 1-D")
        if cu.size and (cu.max() > np.iinfo(np.int32).max or cu.min() < np.iinfo(np.int32).min):
            raise CvaError(1, "cu_seqlens out of int32 range")
        cu32 = np.ascontiguousarray(cu.astype(np.int32))
        if dtype not in DTYPES:
            raise CvaError(7, f"unknown dtype {dtype!r}")
        md, bb = _mask_desc(mask, sink, window, branch_bounds, mask_block)
        n_seqs = max(int(cu32.size) - 1, 0)
        handle = ctypes.c_void_p()
        _check(L.cva_placement_create(cu32.ctypes.data_as(_P32) if cu32.size else None, n_seqs,
                                      ctypes.byref(md), int(n_devices), int(block), int(hq),
                                      int(hkv), int(d_qk), int(d_v), DTYPES[dtype],
                                      float(epsilon), ctypes.byref(handle)))
        del bb
        self._h = handle
        self.hq, self.hkv, self.d_qk, self.d_v, self.dtype = int(hq), int(hkv), int(d_qk), int(d_v), dtype
        self.total_tokens = int(cu32[-1]) if cu32.size else 0
        info = _PlacementInfo()
        _check(L.cva_placement_get(handle, ctypes.byref(info)))
        r = info.n_devices
        self.n_devices, self.block = int(info.n_devices), int(info.block)
        self.data_blocks = _arr(info.data_blocks, info.n_data_blocks * 4, np.int64).reshape(-1, 4)
        self.comp_blocks = _arr(info.comp_blocks, info.n_comp_blocks * 4, np.int64).reshape(-1, 4)
        self.comp_pairs = _arr(info.comp_pairs, info.n_comp_blocks, np.int64)
        self.device_tokens = _arr(info.device_tokens, r, np.int64)
        self.device_pairs = _arr(info.device_pairs, r, np.int64)
        self.device_send_bytes = _arr(info.device_send_bytes, r, np.int64)
        self.device_recv_bytes = _arr(info.device_recv_bytes, r, np.int64)
        self.total_comm_bytes = int(info.total_comm_bytes)
        self.block_comm_bytes = int(info.block_comm_bytes)
        self.zigzag_pairs = _arr(info.zigzag_pairs, r, np.int64) if info.zigzag_valid else None
        self.zigzag_comm_bytes = int(info.zigzag_comm_bytes)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.cva_placement_destroy(h)
            self._h = None

    def device_plan(self, device):
        """``cva_placement_plan_create``: device ``device``'s computation blocks as a
        plan run by :func:`fwd` with ``workspace=True`` on the packed tensors."""
        return PlacedPlan(self, device)


class PlacedPlan(_PlanBase):
    """One device's share of a :class:`Placement` (``cva_placement_plan_create``).

    Runs through ``fwd(plan, q, k, v, workspace=True)`` (``cva_fwd_split``) on the
    packed, unsplit tensors q [T, Hq, Dqk], k/v [T, Hkv, D]; writes o [T, Hq, Dv] and
    lse [Hq, T] at the rows of the O blocks the device contributes to (its partial
    result over its own computation blocks) and leaves the other rows untouched.
    ``blocks`` lists the device's computation blocks (rows of
    ``placement.comp_blocks``).
    """

    def __init__(self, placement, device):
        L = load_library()
        handle = ctypes.c_void_p()
        self._h = None
        self._dev = None
        _check(L.cva_placement_plan_create(placement._h, int(device), ctypes.byref(handle)))
        self._h = handle
        self.device = int(device)
        self.cp_size, self.rank = 1, 0
        self.hq, self.hkv = placement.hq, placement.hkv
        self.d_qk, self.d_v, self.dtype = placement.d_qk, placement.d_v, placement.dtype
        self.global_tokens = self.local_tokens = placement.total_tokens
        self.blocks = placement.comp_blocks[placement.comp_blocks[:, 3] == self.device]


def _launch_stream(plan, stream, device, tensors):
    """The stream a call runs on.  Caller tensors allocated on another stream are
    marked as used by it (record_stream), so that the caching allocator does not
    hand their memory out again while the call may still run; the plan's tables
    are ordered after their upload."""
    import torch
    cur = torch.cuda.current_stream(device)
    s = cur if stream is None else stream
    if s != cur:
        for t in tensors:
            if t is not None:
                t.record_stream(s)
    plan._bind_stream(s)
    return s


_TORCH_DT = {"bf16": "bfloat16", "fp16": "float16", "fp32": "float32"}


def _expect(t, name, shape, dtype, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise CvaError(1, f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise CvaError(1, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != getattr(torch, dtype):
        raise CvaError(7, f"{name} has dtype {t.dtype}, expected torch.{dtype}")
    if not t.is_cuda or t.device != device:
        raise CvaError(1, f"{name} must live on {device}")
    if not t.is_contiguous():
        raise CvaError(1, f"{name} must be contiguous")


def _scale(plan, softmax_scale):
    if softmax_scale is None:
        return 1.0 / math.sqrt(plan.d_qk)
    return float(softmax_scale)


def _check_seed(dropout_p, seed):
    """The dropout seed is the generator's 64-bit key: an integer in [0, 2**64)."""
    if dropout_p is not None and not (isinstance(seed, (int, np.integer)) and 0 <= int(seed) < (1 << 64)):
        raise ValueError(f"dropout seed must be an integer in [0, 2**64), got {seed!r}")


def fwd(plan: Plan, q, k_rm, v_rm, softmax_scale=None, out=None, lse=None, stream=None,
        workspace=None, dropout_p=None, seed=0):
    """``cva_fwd``: returns (o [T_loc, Hq, Dv], lse [Hq, T_loc] float32).

    With ``workspace`` (a device uint8 tensor of at least
    ``plan.fwd_workspace_bytes()`` bytes, or ``True`` to allocate one) this calls
    ``cva_fwd_split`` instead: the long K/V ranges are split and merged.
    With ``dropout_p`` (a probability in [0, 1)) it calls ``cva_fwd_dropout``
    with ``seed`` (an integer below 2**64), with or without that workspace.
    """
    _check_seed(dropout_p, seed)
    import torch
    if not plan.uploaded:
        plan.upload(q.device)
    dev = q.device
    dt = _TORCH_DT[plan.dtype]
    T, Tl = plan.global_tokens, plan.local_tokens
    _expect(q, "q", (Tl, plan.hq, plan.d_qk), dt, dev)
    _expect(k_rm, "k_rm", (T, plan.hkv, plan.d_qk), dt, dev)
    _expect(v_rm, "v_rm", (T, plan.hkv, plan.d_v), dt, dev)
    s = _launch_stream(plan, stream, dev, (q, k_rm, v_rm, out, lse))
    with torch.cuda.stream(s):  # outputs made here belong to the launch stream
        if out is None:
            out = torch.empty((Tl, plan.hq, plan.d_v), dtype=q.dtype, device=dev)
        if lse is None:
            lse = torch.empty((plan.hq, Tl), dtype=torch.float32, device=dev)
    _expect(out, "out", (Tl, plan.hq, plan.d_v), dt, dev)
    _expect(lse, "lse", (plan.hq, Tl), "float32", dev)
    vp = ctypes.c_void_p
    L = load_library()
    if workspace is True:
        with torch.cuda.stream(s):
            workspace = torch.empty(max(plan.fwd_workspace_bytes(), 256), dtype=torch.uint8, device=dev)
    elif workspace is not None and s != torch.cuda.current_stream(dev):
        workspace.record_stream(s)
    if dropout_p is not None:
        ws, wsb = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                       workspace.numel() * workspace.element_size())
        _check(L.cva_fwd_dropout(plan.handle, vp(q.data_ptr()), vp(k_rm.data_ptr()), vp(v_rm.data_ptr()),
                                 vp(out.data_ptr()), vp(lse.data_ptr()), _scale(plan, softmax_scale),
                                 float(dropout_p), int(seed), vp(ws), wsb, vp(s.cuda_stream)))
        return out, lse
    if workspace is None:
        _check(L.cva_fwd(plan.handle, vp(q.data_ptr()), vp(k_rm.data_ptr()), vp(v_rm.data_ptr()),
                         vp(out.data_ptr()), vp(lse.data_ptr()), _scale(plan, softmax_scale),
                         vp(s.cuda_stream)))
        return out, lse
    _check(L.cva_fwd_split(plan.handle, vp(q.data_ptr()), vp(k_rm.data_ptr()), vp(v_rm.data_ptr()),
                           vp(out.data_ptr()), vp(lse.data_ptr()), _scale(plan, softmax_scale),
                           vp(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
                           vp(s.cuda_stream)))
    return out, lse


def bwd(plan: Plan, q, k_rm, v_rm, o, lse, dout, softmax_scale=None, dq=None, dk_rm=None,
        dv_rm=None, workspace=None, stream=None, dropout_p=None, seed=0):
    """``cva_bwd``: returns (dq [T_loc,Hq,Dqk], dk_rm [T,Hkv,Dqk], dv_rm [T,Hkv,Dv]).

    With ``dropout_p`` it calls ``cva_bwd_dropout`` (the backward of
    ``fwd(..., dropout_p=p, seed=seed)``; pass the same p and seed)."""
    _check_seed(dropout_p, seed)
    import torch
    if not plan.uploaded:
        plan.upload(q.device)
    dev = q.device
    dt = _TORCH_DT[plan.dtype]
    T, Tl = plan.global_tokens, plan.local_tokens
    _expect(q, "q", (Tl, plan.hq, plan.d_qk), dt, dev)
    _expect(k_rm, "k_rm", (T, plan.hkv, plan.d_qk), dt, dev)
    _expect(v_rm, "v_rm", (T, plan.hkv, plan.d_v), dt, dev)
    _expect(o, "o", (Tl, plan.hq, plan.d_v), dt, dev)
    _expect(lse, "lse", (plan.hq, Tl), "float32", dev)
    _expect(dout, "dout", (Tl, plan.hq, plan.d_v), dt, dev)
    s = _launch_stream(plan, stream, dev, (q, k_rm, v_rm, o, lse, dout, dq, dk_rm, dv_rm, workspace))
    L = load_library()
    ws_bytes = int(L.cva_bwd_workspace_bytes(plan.handle))
    with torch.cuda.stream(s):  # outputs and workspace made here belong to the launch stream
        if dq is None:
            dq = torch.empty_like(q)
        if dk_rm is None:
            dk_rm = torch.empty_like(k_rm)
        if dv_rm is None:
            dv_rm = torch.empty_like(v_rm)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device=dev)
    _expect(dq, "dq", (Tl, plan.hq, plan.d_qk), dt, dev)
    _expect(dk_rm, "dk_rm", (T, plan.hkv, plan.d_qk), dt, dev)
    _expect(dv_rm, "dv_rm", (T, plan.hkv, plan.d_v), dt, dev)
    vp = ctypes.c_void_p
    if dropout_p is not None:
        _check(L.cva_bwd_dropout(plan.handle, vp(q.data_ptr()), vp(k_rm.data_ptr()), vp(v_rm.data_ptr()),
                                 vp(o.data_ptr()), vp(lse.data_ptr()), vp(dout.data_ptr()), vp(dq.data_ptr()),
                                 vp(dk_rm.data_ptr()), vp(dv_rm.data_ptr()), vp(workspace.data_ptr()),
                                 workspace.numel() * workspace.element_size(), _scale(plan, softmax_scale),
                                 float(dropout_p), int(seed), vp(s.cuda_stream)))
        return dq, dk_rm, dv_rm
    _check(L.cva_bwd(plan.handle, vp(q.data_ptr()), vp(k_rm.data_ptr()), vp(v_rm.data_ptr()),
                     vp(o.data_ptr()), vp(lse.data_ptr()), vp(dout.data_ptr()), vp(dq.data_ptr()),
                     vp(dk_rm.data_ptr()), vp(dv_rm.data_ptr()), vp(workspace.data_ptr()),
                     workspace.numel() * workspace.element_size(), _scale(plan, softmax_scale),
                     vp(s.cuda_stream)))
    return dq, dk_rm, dv_rm


def bwd_noalloc(plan: Plan, q, k_rm, v_rm, o, lse, dout, dq, dk_rm, dv_rm, softmax_scale=None,
                stream=None):
    """``cva_bwd_noalloc``: ``bwd`` into caller-given dq / dk_rm / dv_rm with no
    device allocation (the row statistics live in the library's own array)."""
    dev = q.device
    dt = _TORCH_DT[plan.dtype]
    T, Tl = plan.global_tokens, plan.local_tokens
    for t, name, shape in ((q, "q", (Tl, plan.hq, plan.d_qk)), (k_rm, "k_rm", (T, plan.hkv, plan.d_qk)),
                           (v_rm, "v_rm", (T, plan.hkv, plan.d_v)), (o, "o", (Tl, plan.hq, plan.d_v)),
                           (dout, "dout", (Tl, plan.hq, plan.d_v)), (dq, "dq", (Tl, plan.hq, plan.d_qk)),
                           (dk_rm, "dk_rm", (T, plan.hkv, plan.d_qk)),
                           (dv_rm, "dv_rm", (T, plan.hkv, plan.d_v))):
        _expect(t, name, shape, dt, dev)
    _expect(lse, "lse", (plan.hq, Tl), "float32", dev)
    s = _launch_stream(plan, stream, dev, (q, k_rm, v_rm, o, lse, dout, dq, dk_rm, dv_rm))
    vp = ctypes.c_void_p
    _check(load_library().cva_bwd_noalloc(
        plan.handle, vp(q.data_ptr()), vp(k_rm.data_ptr()), vp(v_rm.data_ptr()), vp(o.data_ptr()),
        vp(lse.data_ptr()), vp(dout.data_ptr()), vp(dq.data_ptr()), vp(dk_rm.data_ptr()),
        vp(dv_rm.data_ptr()), _scale(plan, softmax_scale), vp(s.cuda_stream)))
    return dq, dk_rm, dv_rm


def timing_enable(on=True):
    """``cva_timing_enable``: start (and reset) or stop per-kernel event timing."""
    _check(load_library().cva_timing_enable(1 if on else 0))


def timing_select(kernels=None):
    """Time only the named kernels (KERNEL_NAMES entries); None = all."""
    mask = 0xFFFFFFFF if kernels is None else sum(1 << KERNEL_NAMES.index(k) for k in kernels)
    _check(load_library().cva_timing_select(mask))


def timing_read():
    """``cva_timing_read``: {kernel name: (launches, total ms)} since timing_enable(True)."""
    t = _KernelTimes()
    _check(load_library().cva_timing_read(ctypes.byref(t)))
    return {n: (int(t.launches[i]), float(t.total_ms[i])) for i, n in enumerate(KERNEL_NAMES)}


def local_token_ids(cu_seqlens, cp_size, rank):
    """Packed token ids rank ``rank`` holds, in local order, from libcva's metadata."""
    p = Plan(cu_seqlens, cp_size, rank, 1, 1, 64, 64, "bf16")
    md = p.metadata
    cu = p.cu_seqlens
    aq, pos0 = md["actual_seq_qlen"], md["seg_q_pos0"]
    out = np.empty(p.local_tokens, dtype=np.int64)
    for s in range(len(pos0)):
        i = s // 2
        n = aq[s + 1] - aq[s]
        out[aq[s]: aq[s + 1]] = cu[i] + pos0[s] + np.arange(n)
    return out


def rank_major_token_ids(cu_seqlens, cp_size):
    """Packed token id at every row of the rank-major all-gathered K/V."""
    return np.concatenate([local_token_ids(cu_seqlens, cp_size, s) for s in range(cp_size)])
