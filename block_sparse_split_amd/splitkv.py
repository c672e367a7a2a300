"""Python binding of libsplitkv (argument marshalling only).

Each function has the name of the C entry point it calls and does nothing
but check shapes/dtypes, take pointers and forward the call; every step of
the attention path runs in the HIP kernels of ``libsplitkv.so``.  PyTorch is
used for device memory and streams.  If the library is not built, every call
raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import threading
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SKV_LIBRARY") or os.path.join(_HERE, "libsplitkv.so")

SKV_F32 = 0
SKV_BF16 = 1
XCDS = 8          # XCDs of the device (per-XCD speeds are given per XCD)
SKV_OK = 0
STATUS_NAMES = {0: "SKV_OK", -1: "SKV_ERR_INVALID_ARG", -2: "SKV_ERR_UNSUPPORTED",
                -3: "SKV_ERR_HIP", -4: "SKV_ERR_WORKSPACE"}

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


class SplitKVError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class SkvProblem(ctypes.Structure):
    _fields_ = [("nb", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("anchors", _i32p), ("lo", _i32p), ("n_chunks", ctypes.c_int32),
                ("chunk_pos", _i32p), ("chunk_off", _i32p), ("with_draft", ctypes.c_int32)]


class SkvScheduleInfo(ctypes.Structure):
    _fields_ = [("words", ctypes.c_int64), ("n_workgroups", ctypes.c_int32),
                ("n_tiles", ctypes.c_int32), ("n_qtiles", ctypes.c_int32),
                ("n_items", ctypes.c_int32), ("n_split_qtiles", ctypes.c_int32),
                ("n_partial_slots", ctypes.c_int32), ("n_kv_items", ctypes.c_int32),
                ("xcd_mode", ctypes.c_int32),
                ("fwd_workspace_bytes", ctypes.c_int64), ("bwd_workspace_bytes", ctypes.c_int64),
                ("item_cost_total", ctypes.c_int64), ("item_cost_max_bin", ctypes.c_int64),
                ("kv_cost_total", ctypes.c_int64), ("kv_cost_max_bin", ctypes.c_int64),
                ("nb", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("n_local", ctypes.c_int32), ("with_draft", ctypes.c_int32),
                ("n_dq_items", ctypes.c_int32), ("n_dq_split_qtiles", ctypes.c_int32),
                ("n_dq_partial_slots", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("dq_cost_total", ctypes.c_int64), ("dq_cost_max_bin", ctypes.c_int64)]


_lib = None


def lib():
    """Load libsplitkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run "
                           "`python -m block_sparse_split_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.skv_last_error.restype = ctypes.c_char_p
    L.skv_last_error.argtypes = []
    L.skv_abi_version.restype = ctypes.c_int32
    L.skv_chunk_costs.argtypes = [_i32p, _i32p, ctypes.c_int32, _i32p, _i32p, ctypes.c_int32,
                                  ctypes.c_int32, _i64p]
    L.skv_plan_lpt_costs.argtypes = [_i64p, ctypes.c_int32, ctypes.c_int32, _i32p, _i64p]
    L.skv_plan_lpt.argtypes = [_i32p, _i32p, ctypes.c_int32, _i32p, _i32p, ctypes.c_int32,
                               ctypes.c_int32, ctypes.c_int32, _i32p, _i64p, _i64p]
    L.skv_plan_lpt_split.argtypes = [_i64p, _i32p, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_int32, _i32p, _i64p, _i32p, _i64p, _i64p]
    L.skv_schedule_build.argtypes = [ctypes.POINTER(SkvProblem), ctypes.c_int32, _i32p,
                                     ctypes.c_int64, ctypes.POINTER(SkvScheduleInfo)]
    L.skv_schedule_build_xcd.argtypes = [ctypes.POINTER(SkvProblem), ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_float),
                                         ctypes.POINTER(ctypes.c_float), _i32p, ctypes.c_int64,
                                         ctypes.POINTER(SkvScheduleInfo)]
    L.skv_attn_fwd_partial.argtypes = [ctypes.POINTER(SkvProblem),
                                       ctypes.POINTER(SkvScheduleInfo), _vp, _vp, _vp, _vp,
                                       _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, ctypes.c_int64,
                                       _vp]
    L.skv_attn_fwd_partial_noalloc.argtypes = [ctypes.POINTER(SkvProblem),
                                               ctypes.POINTER(SkvScheduleInfo), _vp, _vp,
                                               _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp,
                                               _vp]
    L.skv_dq_finalize.argtypes = [ctypes.c_int32, ctypes.c_int64, _vp, ctypes.c_int64, _vp,
                                  ctypes.c_int32, _vp]
    L.skv_merge_lse.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _vp,
                                ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp, _vp]
    L.skv_attn_bwd.argtypes = [ctypes.POINTER(SkvProblem), ctypes.POINTER(SkvScheduleInfo),
                               _vp,                                  # schedule
                               _vp, _vp, _vp, _vp, _vp,              # Q K V Kd Vd
                               _vp, _vp, _vp,                        # O dO LSE
                               _vp, _vp, _vp, _vp, _vp,              # dQ dK dV dKd dVd
                               ctypes.c_int32, _vp, ctypes.c_int64, _vp]
    L.skv_timing_enable.argtypes = [ctypes.c_int32]
    L.skv_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    L.skv_timing_result.argtypes = [ctypes.c_int32, ctypes.c_char_p, ctypes.c_int32, _i64p,
                                    ctypes.POINTER(ctypes.c_double)]
    L.skv_timing_wg_clock.argtypes = [_vp, ctypes.c_int64]
    for name in ("skv_chunk_costs", "skv_plan_lpt_costs", "skv_plan_lpt", "skv_plan_lpt_split",
                 "skv_schedule_build", "skv_schedule_build_xcd", "skv_attn_fwd_partial",
                 "skv_attn_fwd_partial_noalloc",
                 "skv_merge_lse", "skv_dq_finalize", "skv_attn_bwd", "skv_timing_enable",
                 "skv_timing_collect",
                 "skv_timing_result", "skv_timing_wg_clock"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(fn, status):
    if status != SKV_OK:
        raise SplitKVError(fn, status, lib().skv_last_error().decode())


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


def _i64(a):
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a, a.ctypes.data_as(_i64p)


# ---------------------------------------------------------------- planner

def skv_chunk_costs(anchors, lo, chunk_pos, chunk_len, tile_k):
    a, ap = _i32(anchors)
    l, lp = _i32(lo)
    p, pp = _i32(chunk_pos)
    n, np_ = _i32(chunk_len)
    out = np.zeros(len(p), np.int64)
    _check("skv_chunk_costs", lib().skv_chunk_costs(ap, lp, len(a), pp, np_, len(p), tile_k,
                                                   out.ctypes.data_as(_i64p)))
    return out


def skv_plan_lpt_costs(costs, n_bins):
    c, cp = _i64(costs)
    bins = np.zeros(len(c), np.int32)
    load = np.zeros(n_bins, np.int64)
    _check("skv_plan_lpt_costs", lib().skv_plan_lpt_costs(
        cp, len(c), n_bins, bins.ctypes.data_as(_i32p), load.ctypes.data_as(_i64p)))
    return bins, load


NO_CUT = 2 ** 63 - 1  # skv_plan_lpt_split target that never cuts


def skv_plan_lpt_split(extra, steps, item_cost, step_cost, n_bins, target=0):
    """LPT with splitting; returns (pieces [n, 4] = (unit, k0, k1, bin) in
    placement order, cost [n], target used, load [n_bins])."""
    e, ep = _i64(extra)
    st, sp = _i32(steps)
    if len(e) != len(st):
        raise ValueError("extra and steps must have the same length")
    cap = len(st) + n_bins
    pieces = np.zeros((cap, 4), np.int32)
    cost = np.zeros(cap, np.int64)
    n = ctypes.c_int32(0)
    t = ctypes.c_int64(0)
    load = np.zeros(n_bins, np.int64)
    _check("skv_plan_lpt_split", lib().skv_plan_lpt_split(
        ep, sp, len(st), int(item_cost), int(step_cost), int(n_bins), int(target), cap,
        pieces.ctypes.data_as(_i32p), cost.ctypes.data_as(_i64p), ctypes.byref(n),
        ctypes.byref(t), load.ctypes.data_as(_i64p)))
    return pieces[:n.value], cost[:n.value], t.value, load


def skv_plan_lpt(anchors, lo, chunk_pos, chunk_len, tile_k, n_bins):
    a, ap = _i32(anchors)
    l, lp = _i32(lo)
    p, pp = _i32(chunk_pos)
    n, np_ = _i32(chunk_len)
    bins = np.zeros(len(p), np.int32)
    cost = np.zeros(len(p), np.int64)
    load = np.zeros(n_bins, np.int64)
    _check("skv_plan_lpt", lib().skv_plan_lpt(
        ap, lp, len(a), pp, np_, len(p), tile_k, n_bins, bins.ctypes.data_as(_i32p),
        cost.ctypes.data_as(_i64p), load.ctypes.data_as(_i64p)))
    return bins, cost, load


# ---------------------------------------------------------------- problem

class Problem:
    """Host description of one shard's attention problem (skv_problem)."""

    def __init__(self, nb, hq, hkv, d, scale, dtype, anchors, lo, chunk_pos=(),
                 chunk_off=(0,), with_draft=True):
        self.anchors, ap = _i32(anchors)
        self.lo, lp = _i32(lo)
        self.chunk_pos, cp = _i32(chunk_pos)
        self.chunk_off, co = _i32(chunk_off)
        self.dtype = dtype
        self.c = SkvProblem(nb, hq, hkv, d, scale, dtype, ap, lp, len(self.chunk_pos), cp, co,
                            int(bool(with_draft)))

    @property
    def nq(self):
        return self.c.nb * 16

    @property
    def n_local(self):
        return int(self.chunk_off[-1]) if len(self.chunk_off) else 0

    @property
    def qt_per_head(self):
        """256-row query tiles per kv head."""
        return -(-self.nq * (self.c.hq // self.c.hkv) // 256)


def skv_schedule_build(problem: Problem, n_workgroups: int = 0):
    info = SkvScheduleInfo()
    L = lib()
    _check("skv_schedule_build", L.skv_schedule_build(ctypes.byref(problem.c), n_workgroups,
                                                      None, 0, ctypes.byref(info)))
    image = np.zeros(info.words, np.int32)
    # build with the workgroup count resolved by the size query
    _check("skv_schedule_build", L.skv_schedule_build(
        ctypes.byref(problem.c), info.n_workgroups, image.ctypes.data_as(_i32p), len(image),
        ctypes.byref(info)))
    return image, info


def skv_schedule_build_xcd(problem: Problem, n_workgroups: int, xcd_speed, cost_scale=None):
    """Schedule planned for per-XCD speeds: xcd_speed is [3, 8] (forward,
    dQ, dK/dV kernels x XCD), relative work per unit time; cost_scale, if
    given, is [2, hkv, qt_per_head] (forward, dQ): measured multipliers of
    the cost of each kv head's query tiles."""
    sp = np.ascontiguousarray(np.asarray(xcd_speed, np.float32).reshape(-1))
    if sp.size != 3 * XCDS:
        raise ValueError(f"xcd_speed must hold 3 x {XCDS} values, got {sp.size}")
    fp = sp.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    cp = None
    if cost_scale is not None:
        cs = np.ascontiguousarray(np.asarray(cost_scale, np.float32).reshape(-1))
        want = 2 * problem.c.hkv * problem.qt_per_head
        if cs.size != want:
            raise ValueError(f"cost_scale must hold 2 x hkv x qt_per_head = {want} values, "
                             f"got {cs.size}")
        cp = cs.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    info = SkvScheduleInfo()
    L = lib()
    _check("skv_schedule_build_xcd", L.skv_schedule_build_xcd(
        ctypes.byref(problem.c), n_workgroups, fp, cp, None, 0, ctypes.byref(info)))
    image = np.zeros(info.words, np.int32)
    _check("skv_schedule_build_xcd", L.skv_schedule_build_xcd(
        ctypes.byref(problem.c), info.n_workgroups, fp, cp, image.ctypes.data_as(_i32p),
        len(image), ctypes.byref(info)))
    return image, info


# ---------------------------------------------------------------- device calls

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SKV_BF16
    if t.dtype == torch.float32:
        return SKV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t, name, dtype=None, shape=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} must not be None")
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _tdtype(code):
    torch = _torch()
    return torch.bfloat16 if code == SKV_BF16 else torch.float32


def skv_attn_fwd_partial(problem: Problem, info, schedule, Q, K, V, Kd, Vd, O, LSE,
                         workspace=None, stream=None):
    torch = _torch()
    p = problem.c
    dt = _tdtype(problem.dtype)
    nq, nl = problem.nq, problem.n_local
    args = [ctypes.byref(p), ctypes.byref(info),
            _ptr(schedule, "schedule", torch.int32, (info.words,)),
            _ptr(Q, "Q", dt, (nq, p.hq, p.d)),
            _ptr(K, "K", dt, (nl, p.hkv, p.d), allow_none=nl == 0),
            _ptr(V, "V", dt, (nl, p.hkv, p.d), allow_none=nl == 0),
            _ptr(Kd, "Kd", dt, (nq, p.hkv, p.d), allow_none=not p.with_draft),
            _ptr(Vd, "Vd", dt, (nq, p.hkv, p.d), allow_none=not p.with_draft),
            _ptr(O, "O", None, (nq, p.hq, p.d)), _dtype_code(O),
            _ptr(LSE, "LSE", torch.float32, (nq, p.hq)),
            _ptr(workspace, "workspace", None, None, allow_none=True),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream(stream)]
    if not p.with_draft:
        args[6] = args[7] = None
    _check("skv_attn_fwd_partial", lib().skv_attn_fwd_partial(*args))


def skv_attn_fwd_partial_noalloc(problem: Problem, info, schedule, Q, K, V, Kd, Vd, O, LSE,
                                 stream=None):
    torch = _torch()
    p = problem.c
    dt = _tdtype(problem.dtype)
    nq, nl = problem.nq, problem.n_local
    nd = not p.with_draft
    _check("skv_attn_fwd_partial_noalloc", lib().skv_attn_fwd_partial_noalloc(
        ctypes.byref(p), ctypes.byref(info),
        _ptr(schedule, "schedule", torch.int32, (info.words,)),
        _ptr(Q, "Q", dt, (nq, p.hq, p.d)),
        _ptr(K, "K", dt, (nl, p.hkv, p.d), allow_none=nl == 0),
        _ptr(V, "V", dt, (nl, p.hkv, p.d), allow_none=nl == 0),
        None if nd else _ptr(Kd, "Kd", dt, (nq, p.hkv, p.d)),
        None if nd else _ptr(Vd, "Vd", dt, (nq, p.hkv, p.d)),
        _ptr(O, "O", None, (nq, p.hq, p.d)), _dtype_code(O),
        _ptr(LSE, "LSE", torch.float32, (nq, p.hq)), _stream(stream)))


def skv_merge_lse(O_parts, LSE_parts, O_out, LSE_out, stream=None):
    torch = _torch()
    k = O_parts.shape[0]
    d = O_parts.shape[-1]
    rows = O_parts[0].numel() // d
    _check("skv_merge_lse", lib().skv_merge_lse(
        k, rows, d, _ptr(O_parts, "O_parts"), _dtype_code(O_parts),
        _ptr(LSE_parts, "LSE_parts", torch.float32, (k,) + tuple(O_parts.shape[1:-1])),
        _ptr(O_out, "O_out", None, tuple(O_parts.shape[1:])), _dtype_code(O_out),
        _ptr(LSE_out, "LSE_out", torch.float32, tuple(O_parts.shape[1:-1])), _stream(stream)))


def skv_dq_finalize(parts, dq_out, stream=None):
    """Sum fp32 dQ shares parts[0..n-1] (a [n, ...] fp32 device tensor whose
    shares are contiguous; dim 0 may be padded, e.g. a slice of a longer
    buffer) into dq_out ([...], fp32 or bf16)."""
    torch = _torch()
    if not parts.is_cuda or parts.dtype != torch.float32:
        raise ValueError("parts must be a float32 device tensor")
    if parts.dim() < 1 or parts.shape[0] < 1:
        raise ValueError("parts must be [n, ...] with n >= 1")
    if not parts[0].is_contiguous():
        raise ValueError("each share must be contiguous")
    elems = parts[0].numel()
    stride = parts.stride(0) if parts.shape[0] > 1 else elems
    out = _ptr(dq_out, "dq_out", None, tuple(parts.shape[1:]))
    _check("skv_dq_finalize", lib().skv_dq_finalize(
        parts.shape[0], elems, ctypes.c_void_p(parts.data_ptr()) if elems else None, stride,
        out, _dtype_code(dq_out), _stream(stream)))


def skv_attn_bwd(problem: Problem, info, schedule, Q, K, V, Kd, Vd, O, dO, LSE, dQ, dK, dV,
                 dKd, dVd, grad_dtype=SKV_F32, workspace=None, stream=None):
    torch = _torch()
    p = problem.c
    dt = _tdtype(problem.dtype)
    gt = _tdtype(grad_dtype)
    nq, nl = problem.nq, problem.n_local
    nd = not p.with_draft
    _check("skv_attn_bwd", lib().skv_attn_bwd(
        ctypes.byref(p), ctypes.byref(info),
        _ptr(schedule, "schedule", torch.int32, (info.words,)),
        _ptr(Q, "Q", dt, (nq, p.hq, p.d)),
        _ptr(K, "K", dt, (nl, p.hkv, p.d), allow_none=nl == 0),
        _ptr(V, "V", dt, (nl, p.hkv, p.d), allow_none=nl == 0),
        None if nd else _ptr(Kd, "Kd", dt, (nq, p.hkv, p.d)),
        None if nd else _ptr(Vd, "Vd", dt, (nq, p.hkv, p.d)),
        _ptr(O, "O", dt, (nq, p.hq, p.d)), _ptr(dO, "dO", dt, (nq, p.hq, p.d)),
        _ptr(LSE, "LSE", torch.float32, (nq, p.hq)),
        _ptr(dQ, "dQ", torch.float32, (nq, p.hq, p.d)),
        _ptr(dK, "dK", gt, (nl, p.hkv, p.d), allow_none=nl == 0),
        _ptr(dV, "dV", gt, (nl, p.hkv, p.d), allow_none=nl == 0),
        None if nd else _ptr(dKd, "dKd", gt, (nq, p.hkv, p.d)),
        None if nd else _ptr(dVd, "dVd", gt, (nq, p.hkv, p.d)),
        grad_dtype, _ptr(workspace, "workspace", None, None, allow_none=True),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))


class Shard:
    """A problem with its schedule uploaded and workspaces allocated.

    Convenience wrapper for repeated calls (one schedule per batch serves
    every layer).  Allocation happens here, never inside the calls."""

    def __init__(self, problem: Problem, device="cuda", n_workgroups: int = 0,
                 xcd_speed=None, cost_scale=None):
        torch = _torch()
        self.problem = problem
        self.cost_scale = cost_scale
        if xcd_speed is None:
            if cost_scale is not None:
                raise ValueError("cost_scale needs xcd_speed")
            self.image, self.info = skv_schedule_build(problem, n_workgroups)
        else:
            self.image, self.info = skv_schedule_build_xcd(problem, n_workgroups, xcd_speed,
                                                           cost_scale)
        self.schedule = torch.from_numpy(self.image).to(device)
        nbytes = max(self.info.fwd_workspace_bytes, self.info.bwd_workspace_bytes, 256)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def fwd(self, Q, K, V, Kd, Vd, O, LSE, stream=None):
        skv_attn_fwd_partial(self.problem, self.info, self.schedule, Q, K, V, Kd, Vd, O, LSE,
                             self.workspace, stream)

    def fwd_noalloc(self, Q, K, V, Kd, Vd, O, LSE, stream=None):
        skv_attn_fwd_partial_noalloc(self.problem, self.info, self.schedule, Q, K, V, Kd, Vd, O,
                                     LSE, stream)

    def bwd(self, Q, K, V, Kd, Vd, O, dO, LSE, dQ, dK, dV, dKd, dVd, grad_dtype=SKV_F32,
            stream=None):
        skv_attn_bwd(self.problem, self.info, self.schedule, Q, K, V, Kd, Vd, O, dO, LSE, dQ,
                     dK, dV, dKd, dVd, grad_dtype, self.workspace, stream)


def queue_loads(image):
    """Planned load (item costs) of every queue of a schedule image, per
    kernel: array [3, n_wg] for the forward, dQ and dK/dV queues (dQ's are
    the forward's unless the image gives dQ sections of its own)."""
    from .csrc_layout import H, I, K, K_WORDS, I_WORDS
    img = np.asarray(image)
    h = {k: int(img[v]) for k, v in H.items()}
    n = h["NWG"]

    out = np.zeros((3, n), np.int64)
    plans = ((h["OFF_ITEMS"], h["OFF_QOFF"], h["OFF_QUEUE"], I_WORDS, I["COST"]),
             (h["OFF_DQ_ITEMS"], h["OFF_DQ_QOFF"], h["OFF_DQ_QUEUE"], I_WORDS, I["COST"]),
             (h["OFF_KV"], h["OFF_KVQOFF"], h["OFF_KVQUEUE"], K_WORDS, K["COST"]))
    for k, (oi, qo, qq, words, cw) in enumerate(plans):
        off = img[qo: qo + n + 1]
        q = img[qq: qq + off[-1]]
        n_items = int(q.max()) + 1 if len(q) else 0
        cost = img[oi: oi + n_items * words].reshape(-1, words)[:, cw].astype(np.int64)
        for v in range(n):
            out[k, v] = cost[q[off[v]: off[v + 1]]].sum()
    return out


def xcd_speeds_from_stamps(image, runs):
    """Relative speed of each XCD in each kernel, from per-workgroup clock
    stamps (skv_timing_wg_clock) of launches with this schedule: runs is a
    list of [3, n_wg, 4] arrays (start, end, XCC_ID, HW_ID per queue).
    speed[k, x] = planned load run on XCD x / time spent on XCD x, scaled
    to mean 1 over the XCDs; a kernel without stamps gets 1."""
    loads = queue_loads(image)
    n = loads.shape[1]
    work = np.zeros((3, XCDS))
    time = np.zeros((3, XCDS))
    for r in runs:
        r = np.asarray(r).reshape(3, n, 4)
        for k in range(3):
            dur = (r[k, :, 1] - r[k, :, 0]).astype(np.float64)
            ok = (r[k, :, 1] > 0) & (dur > 0)
            x = (r[k, :, 2] & 0xF).astype(np.int64) % XCDS
            np.add.at(work[k], x[ok], loads[k][ok])
            np.add.at(time[k], x[ok], dur[ok])
    speed = np.ones((3, XCDS))
    for k in range(3):
        if np.all(time[k] > 0) and np.all(work[k] > 0):
            v = work[k] / time[k]
            speed[k] = v / v.mean()
    return speed


def _plan_sections(image):
    """(items, queue offsets, queue) of the forward and dQ plans."""
    from .csrc_layout import H, I_WORDS
    img = np.asarray(image)
    h = {k: int(img[v]) for k, v in H.items()}
    n = h["NWG"]
    out = []
    for oi, qo, qq in ((h["OFF_ITEMS"], h["OFF_QOFF"], h["OFF_QUEUE"]),
                       (h["OFF_DQ_ITEMS"], h["OFF_DQ_QOFF"], h["OFF_DQ_QUEUE"])):
        off = img[qo: qo + n + 1]
        q = img[qq: qq + off[-1]]
        n_items = int(q.max()) + 1 if len(q) else 0
        out.append((img[oi: oi + n_items * I_WORDS].reshape(-1, I_WORDS), off, q))
    return h, out


def calibrate_from_stamps(datasets, groups_per_head: int = 8, ridge: float = 0.05,
                          iters: int = 4):
    """Per-XCD speeds and measured cost scales from per-workgroup stamps.

    datasets: list of (image, runs, cost_scale) -- a schedule image, the
    stamps of launches with it (as for xcd_speeds_from_stamps) and the cost
    scales it was built with (None for none).  Returns (speed [3, 8],
    cost_scale [2, hkv, qt_per_head]) for skv_schedule_build_xcd.

    Model, per forward or dQ launch: queue v on XCD x takes
    sum over its items i of tau * s_g(i) * c_i / speed_x, with c_i the
    item's cost before any scale and g(i) its (kv head, group of
    consecutive query tiles).  Speeds (with the scales fixed) and scales
    (with the speeds fixed, least squares with a ridge pull towards 1)
    are fitted in turn, the scales normalised to a cost-weighted mean of 1.
    Where the stamps cannot tell a kv head's overall cost from the speed of
    the XCDs that ran it (each head always ran on the same XCDs), the
    ridge leaves that factor with the speeds.  dK/dV gets the dQ kernel's
    speeds: its workgroups take items of other queues once their own is
    done, so its stamps time more than the queue each was planned, and the
    XCDs that run it are the same."""
    from .csrc_layout import I
    speed = np.ones((3, XCDS))
    first = None
    eqs = {0: [], 1: []}
    for image, runs, used in datasets:
        h, plans = _plan_sections(image)
        hkv, qtph, n = h["HKV"], h["QT_PER_HEAD"], h["NWG"]
        if first is None:
            first = (hkv, qtph)
        elif first != (hkv, qtph):
            raise ValueError("datasets of different problems")
        per = -(-qtph // groups_per_head)
        ng = -(-qtph // per)
        for k, (items, off, q) in enumerate(plans):
            head, qt = items[:, I["HEAD"]], items[:, I["QT"]]
            cost = items[:, I["COST"]].astype(np.float64)
            if used is not None:
                cost = cost / np.asarray(used, np.float64).reshape(2, hkv, qtph)[k, head, qt]
            grp = head * ng + qt // per
            A = np.zeros((n, hkv * ng))
            for v in range(n):
                ii = q[off[v]: off[v + 1]]
                np.add.at(A[v], grp[ii], cost[ii])
            for r in runs:
                r = np.asarray(r).reshape(3, n, 4)
                dur = (r[k, :, 1] - r[k, :, 0]).astype(np.float64)
                ok = (r[k, :, 1] > 0) & (dur > 0)
                if not ok.any():   # a kernel that did not run (forward-only steps)
                    continue
                x = (r[k, :, 2] & 0xF).astype(np.int64) % XCDS
                eqs[k].append((A[ok], dur[ok], x[ok]))
    hkv, qtph = first
    per = -(-qtph // groups_per_head)
    ng = -(-qtph // per)
    scale = np.ones((2, hkv, qtph))
    for k in (0, 1):
        if not eqs[k]:
            continue
        sig = np.ones(hkv * ng)
        wsum = sum(A.sum(0) for A, _, _ in eqs[k])
        for _ in range(iters):
            work, time = np.zeros(XCDS), np.zeros(XCDS)
            for A, dur, x in eqs[k]:
                np.add.at(work, x, A @ sig)
                np.add.at(time, x, dur)
            if np.all(time > 0) and np.all(work > 0):
                v = work / time
                speed[k] = v / v.mean()
            M = np.vstack([A for A, _, _ in eqs[k]])
            y = np.concatenate([dur * speed[k][x] for _, dur, x in eqs[k]])
            tau = y.sum() / M.sum()
            MtM = M.T @ M
            lam = ridge * float(np.mean(np.diag(MtM))) + 1e-30
            beta = np.linalg.solve(MtM + lam * np.eye(len(sig)), M.T @ y + lam * tau)
            sig = np.clip(beta / tau, 0.5, 2.0)
            sig /= (sig * wsum).sum() / wsum.sum()
        scale[k] = np.repeat(sig.reshape(hkv, ng), per, axis=1)[:, :qtph]
    speed[2] = speed[1]
    return speed, scale


def measure_xcd_speed(shard, step, steps: int = 4):
    """Run `step` (a callable doing one forward + backward with `shard`)
    `steps` times with per-workgroup stamps and return the per-XCD speeds
    ([3, 8]) of its schedule's queues."""
    torch = _torch()
    n = shard.info.n_workgroups
    clk = torch.zeros(3 * n * 4, dtype=torch.int64, device=shard.schedule.device)
    runs = []
    skv_timing_wg_clock(clk)
    try:
        for _ in range(steps):
            clk.zero_()
            step()
            torch.cuda.synchronize()
            runs.append(clk.view(3, n, 4).cpu().numpy().copy())
    finally:
        skv_timing_wg_clock(None)
    return xcd_speeds_from_stamps(shard.image, runs)


# ---------------------------------------------------------------- timing

_wg_clock_keep = threading.local()


def skv_timing_wg_clock(buffer=None):
    """Set (a uint64/int64 device tensor) or clear (None) the per-workgroup
    clock stamp buffer of the calling thread.  The tensor is kept alive
    here while it is set, since the library holds only its pointer."""
    if buffer is None:
        _check("skv_timing_wg_clock", lib().skv_timing_wg_clock(None, 0))
        _wg_clock_keep.buf = None
        return
    torch = _torch()
    if buffer.dtype not in (torch.int64, torch.uint64):
        raise ValueError(f"buffer must be int64 or uint64, got {buffer.dtype}")
    ptr = _ptr(buffer, "buffer")  # device tensor, contiguous
    if ptr is None:
        raise ValueError("buffer must not be empty")
    _check("skv_timing_wg_clock", lib().skv_timing_wg_clock(
        ptr, buffer.numel() * buffer.element_size()))
    _wg_clock_keep.buf = buffer


def skv_timing_enable(on: bool = True):
    _check("skv_timing_enable", lib().skv_timing_enable(int(bool(on))))


def skv_timing_collect():
    """{kernel name: (launches, total ms)} of the events recorded so far."""
    n = ctypes.c_int32(0)
    _check("skv_timing_collect", lib().skv_timing_collect(ctypes.byref(n)))
    out = {}
    buf = ctypes.create_string_buffer(64)
    for k in range(n.value):
        cnt = ctypes.c_int64(0)
        ms = ctypes.c_double(0)
        _check("skv_timing_result", lib().skv_timing_result(k, buf, 64, ctypes.byref(cnt),
                                                            ctypes.byref(ms)))
        out[buf.value.decode()] = (cnt.value, ms.value)
    return out
