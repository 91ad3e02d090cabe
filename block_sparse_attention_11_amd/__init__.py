"""Python binding of libkpage.so: KPage-style block-sparse attention on MI355X (gfx950).

Thin ctypes marshalling over the C ABI declared in include/kpage.h; every step of
the computation runs in the library's HIP kernels.  The functions keep the C
names.  Tensors are torch tensors on the GPU (device memory and streams only).

The library must have been built (``python -m block_sparse_attention_11_amd.build``
or ``__graft_entry__.build()``); importing works without it, but every call
raises ``KpageError`` when the shared object is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KPAGE_LIB names another build of the same library (the host-sanitizer build of the CPU tests)
LIB_PATH = os.environ.get("KPAGE_LIB") or os.path.join(_HERE, "libkpage.so")

KPAGE_OK, KPAGE_ERR_INVALID, KPAGE_ERR_UNSUPPORTED, KPAGE_ERR_OOM, KPAGE_ERR_HIP = range(5)
STATUS_NAMES = {0: "OK", 1: "INVALID", 2: "UNSUPPORTED", 3: "OOM", 4: "HIP"}

TABLES = {
    "fwd_route": (0, np.int32), "fwd_walk_ptr": (1, np.int64), "fwd_walk": (2, np.int32),
    "fwd_nfull": (3, np.int32), "fwd_valid": (4, np.uint32), "q64_queue": (5, np.int32),
    "q128_queue": (6, np.int32), "owner_ptr": (7, np.int64), "owners": (8, np.int32),
    "owner_aligned": (9, np.uint8), "revq_ptr": (10, np.int64), "revq": (11, np.int32),
    "qwalk_ptr": (12, np.int64), "qwalk": (13, np.int32), "adj": (14, np.uint64),
    "bwd_queue": (15, np.int32), "uncovered_ptr": (16, np.int64), "uncovered": (17, np.int32),
    "group_ptr": (18, np.int64), "group_members": (19, np.int32), "group_walk_ptr": (20, np.int64),
    "group_walk": (21, np.int32), "group_nfull": (22, np.int32), "group_valid": (23, np.uint32),
}

EXPORTED_SYMBOLS = (
    "kpage_plan", "kpage_plan_device", "kpage_plan_upload", "kpage_attn_fwd", "kpage_bwd_workspace_size", "kpage_attn_bwd",
    "kpage_attn_bwd_noalloc",
    "kpage_plan_stats", "kpage_plan_export", "kpage_plan_destroy", "kpage_timing_enable", "kpage_timing_read",
    "kpage_last_error", "kpage_select_workspace_size", "kpage_select_topk", "kpage_select_top_p_workspace_size",
    "kpage_select_top_p",
)

KERNELS = {"fwd": 0, "fwd_exact": 1, "bwd_pre": 2, "bwd_zero": 3, "bwd_kv": 4, "bwd_dq": 5, "bwd_reduce": 6,
           "fwd_q64": 7, "bwd_dq_q64": 8}


class KpageError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kpage {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class KpageProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_q_blocks", ctypes.c_int32), ("n_kv_blocks", ctypes.c_int32),
        ("seq_q", ctypes.c_int64), ("seq_kv", ctypes.c_int64), ("per_head", ctypes.c_int32),
        ("q_valid", ctypes.c_void_p), ("kv_valid", ctypes.c_void_p), ("kv_offset", ctypes.c_void_p),
        ("q2k_ptr", ctypes.c_void_p), ("q2k_idx", ctypes.c_void_p),
    ]


class KpagePlanOpts(ctypes.Structure):
    _fields_ = [("q_group", ctypes.c_int32), ("align_q128", ctypes.c_int32), ("align_q64", ctypes.c_int32),
                ("ungrouped", ctypes.c_int32)]


class KpageSelectLayout(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_q_blocks", ctypes.c_int32), ("n_kv_blocks", ctypes.c_int32),
        ("seq_q", ctypes.c_int64), ("seq_kv", ctypes.c_int64),
        ("q_valid", ctypes.c_void_p), ("kv_valid", ctypes.c_void_p), ("kv_offset", ctypes.c_void_p),
    ]


class KpageSelectClusters(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_q_clusters", ctypes.c_int32), ("n_kv_clusters", ctypes.c_int32),
        ("n_q_blocks", ctypes.c_int32), ("n_kv_blocks", ctypes.c_int32),
        ("q_centroids", ctypes.c_void_p), ("kv_centroids", ctypes.c_void_p),
        ("q_cluster_size", ctypes.c_void_p), ("kv_cluster_size", ctypes.c_void_p),
        ("q_block_cluster", ctypes.c_void_p), ("kv_block_cluster", ctypes.c_void_p),
    ]


class KpagePairStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("useful", "whole_block", "paged_m128", "nominal", "scheduled", "bwd_physical", "bwd_useful_check")]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded shared library; raises KpageError when it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise KpageError(KPAGE_ERR_HIP, f"{LIB_PATH} is missing: build the HIP library first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.kpage_plan.argtypes = [ctypes.POINTER(KpageProblem), ctypes.POINTER(KpagePlanOpts), ctypes.POINTER(vp)]
        L.kpage_plan_device.argtypes = [ctypes.POINTER(KpageProblem), ctypes.c_int64, ctypes.POINTER(KpagePlanOpts), vp,
                                        ctypes.POINTER(vp)]
        L.kpage_plan_upload.argtypes = [vp, vp]
        L.kpage_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp]
        L.kpage_bwd_workspace_size.argtypes = [vp, ctypes.POINTER(sz)]
        L.kpage_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, f32, vp]
        L.kpage_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp]
        L.kpage_plan_stats.argtypes = [vp, ctypes.POINTER(KpagePairStats)]
        L.kpage_plan_export.argtypes = [vp, i32, vp, ctypes.POINTER(sz)]
        L.kpage_timing_enable.argtypes = [vp, i32]
        L.kpage_timing_read.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        L.kpage_select_workspace_size.argtypes = [ctypes.POINTER(KpageSelectLayout), ctypes.POINTER(sz)]
        L.kpage_select_topk.argtypes = [ctypes.POINTER(KpageSelectLayout), vp, vp, ctypes.c_int32, vp, vp, vp, sz, vp]
        L.kpage_select_top_p_workspace_size.argtypes = [ctypes.POINTER(KpageSelectClusters), ctypes.POINTER(sz)]
        L.kpage_select_top_p.argtypes = [ctypes.POINTER(KpageSelectClusters), ctypes.c_double, ctypes.c_double, vp, vp,
                                         vp, sz, vp]
        L.kpage_plan_destroy.argtypes = [vp]
        L.kpage_plan_destroy.restype = None
        L.kpage_last_error.restype = ctypes.c_char_p
        for name in EXPORTED_SYMBOLS:
            if name not in ("kpage_plan_destroy", "kpage_last_error"):
                getattr(L, name).restype = ctypes.c_int
        _lib_handle = L
    return _lib_handle


def kpage_last_error() -> str:
    return lib().kpage_last_error().decode()


def _check(status: int):
    if status != KPAGE_OK:
        raise KpageError(status, kpage_last_error())


class Plan:
    """Owns a kpage_plan_t handle plus the shape facts the binding checks tensors against."""

    def __init__(self, handle, batch, heads, head_dim, seq_q, seq_kv):
        self.handle = handle
        self.batch, self.heads, self.head_dim = batch, heads, head_dim
        self.seq_q, self.seq_kv = seq_q, seq_kv

    def close(self):
        if self.handle:
            lib().kpage_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _arr(x, dtype):
    return np.ascontiguousarray(np.asarray(x, dtype=dtype))


def kpage_plan(problem, align_q64: int = 0, align_q128: int = 0, q_group: int = 0, grouped: bool = True) -> Plan:
    """Plan for ``problem`` (any object with the workloads.Workload descriptor attributes).
    grouped=False runs every query block as its own work item (kpage_plan_opts.ungrouped)."""
    qv = _arr(problem.q_valid, np.int32)
    kvv = _arr(problem.kv_valid, np.int32)
    ko = None if problem.kv_offset is None else _arr(problem.kv_offset, np.int64)
    ptr = _arr(problem.q2k_ptr, np.int64)
    idx = _arr(problem.q2k_idx, np.int32)
    if idx.size == 0:
        idx = np.zeros(1, dtype=np.int32)
    p = KpageProblem(
        batch=problem.batch, heads=problem.heads, head_dim=problem.head_dim,
        n_q_blocks=problem.n_q, n_kv_blocks=problem.n_kv, seq_q=problem.seq_q, seq_kv=problem.seq_kv,
        per_head=1 if problem.per_head else 0,
        q_valid=qv.ctypes.data, kv_valid=kvv.ctypes.data, kv_offset=0 if ko is None else ko.ctypes.data,
        q2k_ptr=ptr.ctypes.data, q2k_idx=idx.ctypes.data)
    opts = KpagePlanOpts(q_group=q_group, align_q128=align_q128, align_q64=align_q64, ungrouped=0 if grouped else 1)
    h = ctypes.c_void_p()
    _check(lib().kpage_plan(ctypes.byref(p), ctypes.byref(opts), ctypes.byref(h)))
    return Plan(h, problem.batch, problem.heads, problem.head_dim, problem.seq_q, problem.seq_kv)


def kpage_plan_device(problem, align_q64: int = 0, align_q128: int = 0, q_group: int = 0, stream=None,
                      grouped: bool = True) -> Plan:
    """Plan for ``problem`` built on the GPU from device copies of its descriptor arrays
    (kpage_plan_device).  The arrays may be numpy arrays (copied to the current device
    here) or CUDA tensors of the right dtypes."""
    import torch

    def dev(x, dtype):
        if isinstance(x, torch.Tensor) and x.is_cuda:
            t = x.contiguous()
            if t.dtype != dtype:
                raise KpageError(KPAGE_ERR_INVALID, f"descriptor array of dtype {t.dtype}, need {dtype}")
            return t
        return torch.from_numpy(np.ascontiguousarray(np.asarray(x))).to(dtype).cuda()

    qv = dev(problem.q_valid, torch.int32)
    kvv = dev(problem.kv_valid, torch.int32)
    ko = None if problem.kv_offset is None else dev(problem.kv_offset, torch.int64)
    ptr = dev(problem.q2k_ptr, torch.int64)
    idx = dev(problem.q2k_idx, torch.int32)
    nnz = int(idx.numel())
    if nnz == 0:
        idx = torch.zeros(1, dtype=torch.int32, device=qv.device)
    p = KpageProblem(
        batch=problem.batch, heads=problem.heads, head_dim=problem.head_dim,
        n_q_blocks=problem.n_q, n_kv_blocks=problem.n_kv, seq_q=problem.seq_q, seq_kv=problem.seq_kv,
        per_head=1 if problem.per_head else 0,
        q_valid=qv.data_ptr(), kv_valid=kvv.data_ptr(), kv_offset=0 if ko is None else ko.data_ptr(),
        q2k_ptr=ptr.data_ptr(), q2k_idx=idx.data_ptr())
    opts = KpagePlanOpts(q_group=q_group, align_q128=align_q128, align_q64=align_q64, ungrouped=0 if grouped else 1)
    h = ctypes.c_void_p()
    _check(lib().kpage_plan_device(ctypes.byref(p), nnz, ctypes.byref(opts), _stream_ptr(stream), ctypes.byref(h)))
    return Plan(h, problem.batch, problem.heads, problem.head_dim, problem.seq_q, problem.seq_kv)


def kpage_plan_stats(plan: Plan) -> dict:
    s = KpagePairStats()
    _check(lib().kpage_plan_stats(plan.handle, ctypes.byref(s)))
    return {n: int(getattr(s, n)) for n, _ in KpagePairStats._fields_}


def kpage_plan_export(plan: Plan, table: str) -> np.ndarray:
    tid, dtype = TABLES[table]
    n = ctypes.c_size_t(0)
    _check(lib().kpage_plan_export(plan.handle, tid, None, ctypes.byref(n)))
    out = np.zeros(n.value // np.dtype(dtype).itemsize, dtype=dtype)
    if n.value:
        _check(lib().kpage_plan_export(plan.handle, tid, out.ctypes.data, ctypes.byref(n)))
    return out


def kpage_timing_enable(plan: Plan, enable=True):
    """enable: False/0 off, True/1 on, 2 on with the forward and dQ launches split by route."""
    _check(lib().kpage_timing_enable(plan.handle, int(enable)))


def kpage_timing_read(plan: Plan, kernel: str):
    """(total milliseconds, launches) of one kernel since the last read (waits for its events)."""
    ms, n = ctypes.c_double(0), ctypes.c_int64(0)
    _check(lib().kpage_timing_read(plan.handle, KERNELS[kernel], ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


def kpage_bwd_workspace_size(plan: Plan) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().kpage_bwd_workspace_size(plan.handle, ctypes.byref(n)))
    return int(n.value)


def _stream_ptr(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev(t, rows, plan: Plan, name, dtype):
    import torch
    want = (plan.batch, plan.heads, rows) + ((plan.head_dim,) if dtype == torch.bfloat16 else ())
    if not t.is_cuda or t.dtype != dtype or tuple(t.shape) != want or not t.is_contiguous():
        raise KpageError(KPAGE_ERR_INVALID, f"{name}: need a contiguous {dtype} CUDA tensor of shape {want}, "
                                            f"got {tuple(t.shape)} {t.dtype} on {t.device}")
    return t.data_ptr()


def kpage_plan_upload(plan: Plan, stream=None):
    _check(lib().kpage_plan_upload(plan.handle, _stream_ptr(stream)))


def kpage_attn_fwd(plan: Plan, q, k, v, o, lse, softmax_scale: float, stream=None):
    import torch
    bf = torch.bfloat16
    args = (_dev(q, plan.seq_q, plan, "q", bf), _dev(k, plan.seq_kv, plan, "k", bf),
            _dev(v, plan.seq_kv, plan, "v", bf), _dev(o, plan.seq_q, plan, "o", bf),
            _dev(lse, plan.seq_q, plan, "lse", torch.float32))
    _check(lib().kpage_attn_fwd(plan.handle, *args, ctypes.c_float(softmax_scale), _stream_ptr(stream)))


def kpage_attn_bwd(plan: Plan, q, k, v, o, lse, do, dq, dk, dv, workspace, softmax_scale: float, stream=None):
    import torch
    bf = torch.bfloat16
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise KpageError(KPAGE_ERR_INVALID, "workspace must be a contiguous CUDA tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    args = (_dev(q, plan.seq_q, plan, "q", bf), _dev(k, plan.seq_kv, plan, "k", bf),
            _dev(v, plan.seq_kv, plan, "v", bf), _dev(o, plan.seq_q, plan, "o", bf),
            _dev(lse, plan.seq_q, plan, "lse", torch.float32), _dev(do, plan.seq_q, plan, "do", bf),
            _dev(dq, plan.seq_q, plan, "dq", bf), _dev(dk, plan.seq_kv, plan, "dk", bf),
            _dev(dv, plan.seq_kv, plan, "dv", bf))
    _check(lib().kpage_attn_bwd(plan.handle, *args, workspace.data_ptr(), ctypes.c_size_t(ws_bytes),
                                ctypes.c_float(softmax_scale), _stream_ptr(stream)))


# the static scratch of kpage_attn_bwd_noalloc (KPAGE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20


def kpage_attn_bwd_noalloc(plan: Plan, q, k, v, o, lse, do, dq, dk, dv, softmax_scale: float, stream=None):
    """kpage_attn_bwd with the library's static device scratch as workspace: no allocation."""
    import torch
    bf = torch.bfloat16
    args = (_dev(q, plan.seq_q, plan, "q", bf), _dev(k, plan.seq_kv, plan, "k", bf),
            _dev(v, plan.seq_kv, plan, "v", bf), _dev(o, plan.seq_q, plan, "o", bf),
            _dev(lse, plan.seq_q, plan, "lse", torch.float32), _dev(do, plan.seq_q, plan, "do", bf),
            _dev(dq, plan.seq_q, plan, "dq", bf), _dev(dk, plan.seq_kv, plan, "dk", bf),
            _dev(dv, plan.seq_kv, plan, "dv", bf))
    _check(lib().kpage_attn_bwd_noalloc(plan.handle, *args, ctypes.c_float(softmax_scale), _stream_ptr(stream)))


# ---- convenience wrappers (allocation of outputs only) ----

def attn_fwd(plan: Plan, q, k, v, softmax_scale: float, stream=None):
    import torch
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    kpage_attn_fwd(plan, q, k, v, o, lse, softmax_scale, stream)
    return o, lse


def attn_bwd(plan: Plan, q, k, v, o, lse, do, softmax_scale: float, stream=None, workspace=None):
    import torch
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty(kpage_bwd_workspace_size(plan), dtype=torch.uint8, device=q.device)
    kpage_attn_bwd(plan, q, k, v, o, lse, do, dq, dk, dv, workspace, softmax_scale, stream)
    return dq, dk, dv


# ---- block selection prelude (device graph for kpage_plan_device) ----

def _select_layout(q, k, q_valid, kv_valid, kv_offset):
    import torch
    for name, t, dt in (("q_valid", q_valid, torch.int32), ("kv_valid", kv_valid, torch.int32)):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dt and t.is_contiguous() and t.dim() == 1):
            raise KpageError(KPAGE_ERR_INVALID, f"{name}: need a contiguous 1-D int32 CUDA tensor")
    if kv_offset is not None and not (isinstance(kv_offset, torch.Tensor) and kv_offset.is_cuda
                                      and kv_offset.dtype == torch.int64 and kv_offset.is_contiguous()):
        raise KpageError(KPAGE_ERR_INVALID, "kv_offset: need a contiguous int64 CUDA tensor or None")
    for name, t in (("q", q), ("k", k)):
        if not (t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous() and t.dim() == 4):
            raise KpageError(KPAGE_ERR_INVALID, f"{name}: need a contiguous bf16 CUDA tensor [B, H, S, d]")
    B, H, Sq, d = q.shape
    if tuple(k.shape[:2]) != (B, H) or k.shape[3] != d:
        raise KpageError(KPAGE_ERR_INVALID, "q and k must agree in batch, heads and head_dim")
    return KpageSelectLayout(batch=B, heads=H, head_dim=d, n_q_blocks=int(q_valid.numel()),
                             n_kv_blocks=int(kv_valid.numel()), seq_q=Sq, seq_kv=k.shape[2],
                             q_valid=q_valid.data_ptr(), kv_valid=kv_valid.data_ptr(),
                             kv_offset=0 if kv_offset is None else kv_offset.data_ptr())


def kpage_select_workspace_size(q, k, q_valid, kv_valid, kv_offset=None) -> int:
    lay = _select_layout(q, k, q_valid, kv_valid, kv_offset)
    n = ctypes.c_size_t(0)
    _check(lib().kpage_select_workspace_size(ctypes.byref(lay), ctypes.byref(n)))
    return int(n.value)


def select_topk(q, k, q_valid, kv_valid, kv_offset, top_k: int, stream=None, workspace=None):
    """Top-k block selection on the GPU (kpage_select_topk): returns the device CSR graph
    (q2k_ptr int64 [B*H, n_q + 1], q2k_idx int32 [B*H*n_q*top_k] capacity)."""
    import torch
    lay = _select_layout(q, k, q_valid, kv_valid, kv_offset)
    BH, n_q = lay.batch * lay.heads, lay.n_q_blocks
    ptr = torch.empty((BH, n_q + 1), dtype=torch.int64, device=q.device)
    idx = torch.empty(max(BH * n_q * top_k, 1), dtype=torch.int32, device=q.device)
    if workspace is None:
        n = ctypes.c_size_t(0)
        _check(lib().kpage_select_workspace_size(ctypes.byref(lay), ctypes.byref(n)))
        workspace = torch.empty(n.value, dtype=torch.uint8, device=q.device)
    _check(lib().kpage_select_topk(ctypes.byref(lay), q.data_ptr(), k.data_ptr(), int(top_k), ptr.data_ptr(),
                                   idx.data_ptr(), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream_ptr(stream)))
    return ptr, idx


class SelectedProblem:
    """A kpage problem whose descriptor arrays are device tensors: one block layout
    shared by all heads (repeated per slot) and a per-(b, h) selected graph."""

    def __init__(self, q, k, q_valid, kv_valid, kv_offset, q2k_ptr, q2k_idx):
        import torch
        B, H, Sq, d = q.shape
        G = B * H
        self.batch, self.heads, self.head_dim = B, H, d
        self.n_q, self.n_kv = int(q_valid.numel()), int(kv_valid.numel())
        self.seq_q, self.seq_kv = Sq, k.shape[2]
        self.per_head = True
        self.q_valid = q_valid.repeat(G).view(G, -1)
        self.kv_valid = kv_valid.repeat(G).view(G, -1)
        off = kv_offset if kv_offset is not None else \
            torch.arange(self.n_kv, dtype=torch.int64, device=q.device) * 128
        self.kv_offset = off.repeat(G).view(G, -1)
        self.q2k_ptr, self.q2k_idx = q2k_ptr, q2k_idx


def plan_topk(q, k, q_valid, kv_valid, kv_offset, top_k: int, stream=None, **opts) -> Plan:
    """Selection, then planning, both on the GPU: the plan of the top-k graph of (q, k)."""
    ptr, idx = select_topk(q, k, q_valid, kv_valid, kv_offset, top_k, stream)
    return kpage_plan_device(SelectedProblem(q, k, q_valid, kv_valid, kv_offset, ptr, idx), stream=stream, **opts)


def select_top_p(batch: int, heads: int, q_cent, k_cent, q_size, k_size, q_block_cluster, k_block_cluster,
                 top_p: float, scale: float, stream=None, workspace=None):
    """Cluster top-p selection on the GPU (kpage_select_top_p).  Arrays are CUDA tensors:
    q_cent / k_cent fp32 [B*H, n_clusters, d]; q_size / k_size int32 [B*H, n_clusters];
    q_block_cluster / k_block_cluster int32 [B*H, n_blocks].  Returns the device CSR graph
    (q2k_ptr int64 [B*H, n_q + 1], q2k_idx int32 with capacity B*H*n_q*n_kv)."""
    import torch
    arrs = dict(q_cent=(q_cent, torch.float32, 3), k_cent=(k_cent, torch.float32, 3),
                q_size=(q_size, torch.int32, 2), k_size=(k_size, torch.int32, 2),
                q_block_cluster=(q_block_cluster, torch.int32, 2), k_block_cluster=(k_block_cluster, torch.int32, 2))
    for name, (t, dt, nd) in arrs.items():
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dt and t.is_contiguous() and t.dim() == nd
                and t.shape[0] == batch * heads):
            raise KpageError(KPAGE_ERR_INVALID, f"{name}: need a contiguous {dt} CUDA tensor of rank {nd}, "
                                                f"first dimension batch * heads")
    G, n_qc, d = q_cent.shape
    n_kc = k_cent.shape[1]
    n_q, n_kv = q_block_cluster.shape[1], k_block_cluster.shape[1]
    desc = KpageSelectClusters(batch=batch, heads=heads, head_dim=d, n_q_clusters=n_qc, n_kv_clusters=n_kc,
                               n_q_blocks=n_q, n_kv_blocks=n_kv, q_centroids=q_cent.data_ptr(),
                               kv_centroids=k_cent.data_ptr(), q_cluster_size=q_size.data_ptr(),
                               kv_cluster_size=k_size.data_ptr(), q_block_cluster=q_block_cluster.data_ptr(),
                               kv_block_cluster=k_block_cluster.data_ptr())
    if workspace is None:
        n = ctypes.c_size_t(0)
        _check(lib().kpage_select_top_p_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
        workspace = torch.empty(n.value, dtype=torch.uint8, device=q_cent.device)
    ptr = torch.empty((G, n_q + 1), dtype=torch.int64, device=q_cent.device)
    idx = torch.empty(max(G * n_q * n_kv, 1), dtype=torch.int32, device=q_cent.device)
    _check(lib().kpage_select_top_p(ctypes.byref(desc), float(top_p), float(scale), ptr.data_ptr(), idx.data_ptr(),
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    _stream_ptr(stream)))
    return ptr, idx
