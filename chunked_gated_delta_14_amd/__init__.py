"""Python binding of libgdr (chunked gated delta-rule training on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgdr.so``; PyTorch tensors provide device memory and streams.
The names mirror the C ABI in ``include/gdr.h``.  There is no CPU fallback:
if the library is missing or the device is not gfx950 the calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

from . import _build

__all__ = [
    "GDR_KDA", "GDR_GDN", "GDR_FWD_SAVE", "GDR_FWD_SKIP_OUTPUT", "GDR_IN_QK_L2NORM", "GDR_IN_BETA_SIGMOID", "GDR_WALK_AUTO", "GDR_WALK_SLICES", "GDR_WALK_RINGS", "GDR_PLAN_BALANCED", "GDR_PLAN_EQUAL", "GdrError", "lib", "plan_chunks", "max_doc_chunks", "workspace_bytes",
    "Problem", "kda_fwd", "kda_bwd", "gdn_fwd", "gdn_bwd", "kda_ckpt", "gdn_ckpt", "kda_ckpt_noalloc",
    "GDR_NOALLOC_SCRATCH_BYTES", "status_string",
    "check_device", "walk_layout_chosen", "timing_enable", "timing_read", "EXPORTED_SYMBOLS",
]

GDR_KDA = 0
GDR_GDN = 1
GDR_FWD_SAVE = 1
GDR_FWD_SKIP_OUTPUT = 2  # forward without the output (o may be None): the recompute of a ckpt step
GDR_IN_QK_L2NORM = 1     # Problem input flag: q, k rows scaled to unit L2 norm inside the kernels
GDR_IN_BETA_SIGMOID = 2  # Problem input flag: beta holds logits, sigmoid applied inside the kernels
GDR_WALK_AUTO, GDR_WALK_SLICES, GDR_WALK_RINGS = 0, 1, 2  # Problem walk_layout
GDR_PLAN_BALANCED, GDR_PLAN_EQUAL = 0, 1  # Problem walk_plan: segments shared by length, or equally

EXPORTED_SYMBOLS = (
    "gdr_plan_chunks", "gdr_workspace_bytes", "gdr_kda_fwd", "gdr_kda_bwd", "gdr_gdn_fwd",
    "gdr_gdn_bwd", "gdr_kda_ckpt", "gdr_gdn_ckpt", "gdr_check_device", "gdr_status_string",
    "gdr_last_error", "gdr_timing_enable", "gdr_timing_read", "gdr_walk_layout_chosen",
    "gdr_kda_ckpt_noalloc",
)
GDR_NOALLOC_SCRATCH_BYTES = 64 << 20  # the static workspace of gdr_kda_ckpt_noalloc


class GdrError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__("libgdr: %s (%d): %s" % (status_string(status), status, detail))


class _CProblem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("N", ctypes.c_int32), ("H_qk", ctypes.c_int32),
        ("H_v", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
        ("chunk_table", ctypes.c_void_p), ("n_chunks", ctypes.c_int32), ("h0", ctypes.c_void_p),
        ("scale", ctypes.c_float), ("input_flags", ctypes.c_uint32), ("walk_segments", ctypes.c_int32),
        ("max_doc_chunks", ctypes.c_int32), ("walk_layout", ctypes.c_int32), ("walk_plan", ctypes.c_int32),
    ]


_lib = None
_lock = threading.Lock()


def lib():
    """Load libgdr.so (built in-tree by ``_build.build``); raise if it is absent."""
    global _lib
    with _lock:
        if _lib is None:
            path = _build.LIB_PATH
            if not os.path.exists(path):
                raise RuntimeError("libgdr.so is not built (run __graft_entry__.build() or "
                                   "python -m chunked_gated_delta_14_amd._build)")
            L = ctypes.CDLL(path)
            i32, i64, u32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p
            P = ctypes.POINTER(_CProblem)
            L.gdr_plan_chunks.argtypes = [ctypes.POINTER(i32), i32, ctypes.POINTER(i32), i64,
                                          ctypes.POINTER(i32), ctypes.POINTER(i64)]
            L.gdr_plan_chunks.restype = i32
            L.gdr_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, u32]
            L.gdr_workspace_bytes.restype = i64
            for name in ("gdr_kda_fwd", "gdr_gdn_fwd"):
                fn = getattr(L, name)
                fn.argtypes = [P, vp, vp, vp, i64, u32, vp]
                fn.restype = i32
            for name in ("gdr_kda_bwd", "gdr_gdn_bwd"):
                fn = getattr(L, name)
                fn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]
                fn.restype = i32
            for name in ("gdr_kda_ckpt", "gdr_gdn_ckpt"):
                fn = getattr(L, name)
                fn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]
                fn.restype = i32
            L.gdr_kda_ckpt_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
            L.gdr_kda_ckpt_noalloc.restype = i32
            L.gdr_timing_enable.argtypes = [i32]
            L.gdr_timing_enable.restype = i32
            L.gdr_timing_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(i64), i32, ctypes.POINTER(i32), i32]
            L.gdr_timing_read.restype = i32
            L.gdr_walk_layout_chosen.argtypes = [i32, P, i32, ctypes.POINTER(i32)]
            L.gdr_walk_layout_chosen.restype = i32
            L.gdr_check_device.argtypes = []
            L.gdr_check_device.restype = i32
            L.gdr_status_string.argtypes = [i32]
            L.gdr_status_string.restype = ctypes.c_char_p
            L.gdr_last_error.argtypes = []
            L.gdr_last_error.restype = ctypes.c_char_p
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gdr_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != 0:
        raise GdrError(status, lib().gdr_last_error().decode())


def check_device() -> None:
    _check(lib().gdr_check_device())


def walk_layout_chosen(variant, problem, compute_units=0) -> int:
    """GDR_WALK_SLICES or GDR_WALK_RINGS: the walks' launch layout for `problem`
    (a Problem or a _CProblem) on a device with `compute_units` CUs (0: current)."""
    code = variant if isinstance(variant, int) else (GDR_KDA if variant == "kda" else GDR_GDN)
    c = problem.cstruct if hasattr(problem, "cstruct") else ctypes.byref(problem)
    out = ctypes.c_int32()
    _check(lib().gdr_walk_layout_chosen(code, c, int(compute_units), ctypes.byref(out)))
    return out.value


def timing_enable(on: bool = True) -> None:
    """Per-kernel event timing inside the library (see gdr_timing_enable)."""
    _check(lib().gdr_timing_enable(1 if on else 0))


def timing_read(reset: bool = True) -> dict:
    """{kernel name: (total ms, launches)} of the timed launches so far."""
    names = (ctypes.c_char_p * 4)()
    ms = (ctypes.c_double * 4)()
    n_l = (ctypes.c_int64 * 4)()
    cnt = ctypes.c_int32()
    _check(lib().gdr_timing_read(names, ms, n_l, 4, ctypes.byref(cnt), 1 if reset else 0))
    return {names[i].decode(): (float(ms[i]), int(n_l[i])) for i in range(cnt.value)}


def plan_chunks(cu_seqlens):
    """Host chunk planner.  Returns (table: np.int32 array, n_chunks)."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    N = len(cu) - 1
    nc = ctypes.c_int32()
    tl = ctypes.c_int64()
    ip = ctypes.POINTER(ctypes.c_int32)
    _check(lib().gdr_plan_chunks(cu.ctypes.data_as(ip), N, None, 0, ctypes.byref(nc), ctypes.byref(tl)))
    table = np.zeros(max(int(tl.value), 1), dtype=np.int32)
    _check(lib().gdr_plan_chunks(cu.ctypes.data_as(ip), N, table.ctypes.data_as(ip), table.size,
                                 ctypes.byref(nc), ctypes.byref(tl)))
    return table[: tl.value], int(nc.value)


def workspace_bytes(variant, T, N, n_chunks, H_qk, H_v, K=128, V=128, flags=0) -> int:
    r = lib().gdr_workspace_bytes(variant, T, N, n_chunks, H_qk, H_v, K, V, flags)
    if r < 0:
        _check(-r)
    return int(r)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch

        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def max_doc_chunks(table, N, n_chunks) -> int:
    """Chunks of the longest document, from the planner's per-document first-chunk section."""
    if N == 0 or n_chunks == 0:
        return 0
    doc_ptr = np.asarray(table[3 * n_chunks:3 * n_chunks + N + 1], dtype=np.int64)
    return int(np.max(np.diff(doc_ptr)))


class Problem:
    """A packed problem: the input tensors (device), cu_seqlens and its chunk table.

    q, k: bf16 [T, H_qk, 128]; v: bf16 [T, H_v, 128]; g: fp32 [T, H_v, 128] (KDA)
    or [T, H_v] (GDN); beta: bf16 [T, H_v] (KDA) or fp32 [T, H_v] (GDN);
    cu_seqlens: host sequence or tensor of N+1 ints; h0: fp32 [N, H_v, 128, 128] or None.
    input_flags: GDR_IN_QK_L2NORM and/or GDR_IN_BETA_SIGMOID (activations applied in the kernels).
    walk_segments: 0 = automatic segmentation of the state walks, n >= 1 = at most n segments.
    walk_layout: GDR_WALK_AUTO, GDR_WALK_SLICES or GDR_WALK_RINGS (launch layout of the walks).
    walk_plan: GDR_PLAN_BALANCED or GDR_PLAN_EQUAL (segments of segmented walks per document).
    """

    def __init__(self, variant, q, k, v, g, beta, cu_seqlens, h0=None, scale=None, input_flags=0, walk_segments=0,
                 walk_layout=GDR_WALK_AUTO, walk_plan=GDR_PLAN_BALANCED):
        import torch

        self.variant = variant
        self.q, self.k, self.v, self.g, self.beta, self.h0 = q, k, v, g, beta, h0
        cu_host = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int32)
        self.cu_host = cu_host
        table, nc = plan_chunks(cu_host)
        dev = q.device
        self.cu = torch.from_numpy(cu_host.copy()).to(dev)
        self.table = torch.from_numpy(table.copy()).to(dev)
        self.table_host = table
        self.n_chunks = nc
        self.T, self.H_qk = int(q.shape[0]), int(q.shape[1])
        self.H_v = int(v.shape[1])
        self.N = len(cu_host) - 1
        self.K, self.V = int(q.shape[2]), int(v.shape[2])
        self.scale = float(self.K ** -0.5 if scale is None else scale)
        self._c = _CProblem(self.T, self.N, self.H_qk, self.H_v, self.K, self.V,
                            q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
                            self.cu.data_ptr(), self.table.data_ptr(), nc,
                            h0.data_ptr() if h0 is not None else None, self.scale, int(input_flags),
                            int(walk_segments), max_doc_chunks(table, self.N, nc), int(walk_layout),
                            int(walk_plan))
        self.input_flags = int(input_flags)

    def workspace_bytes(self, flags=GDR_FWD_SAVE) -> int:
        return workspace_bytes(self.variant, self.T, self.N, self.n_chunks, self.H_qk, self.H_v,
                               self.K, self.V, flags)

    def alloc_workspace(self, flags=GDR_FWD_SAVE):
        import torch

        nbytes = max(self.workspace_bytes(flags), 256)
        return torch.empty(nbytes, dtype=torch.uint8, device=self.q.device)

    @property
    def cstruct(self):
        return ctypes.byref(self._c)


def _fwd(name, prob, o, ht, workspace, flags, stream):
    _check(getattr(lib(), name)(prob.cstruct, _ptr(o), _ptr(ht), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), flags, _stream(stream)))


def _bwd(name, prob, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, stream):
    _check(getattr(lib(), name)(prob.cstruct, _ptr(dout), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                _ptr(dbeta), _ptr(dh0), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))


def _ckpt(name, prob, o, ht, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, stream):
    _check(getattr(lib(), name)(prob.cstruct, _ptr(o), _ptr(ht), _ptr(dout), _ptr(dht), _ptr(dq), _ptr(dk),
                                _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))


def kda_fwd(prob, o, ht, workspace, flags=0, stream=None):
    _fwd("gdr_kda_fwd", prob, o, ht, workspace, flags, stream)


def gdn_fwd(prob, o, ht, workspace, flags=0, stream=None):
    _fwd("gdr_gdn_fwd", prob, o, ht, workspace, flags, stream)


def kda_bwd(prob, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, stream=None):
    _bwd("gdr_kda_bwd", prob, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, stream)


def gdn_bwd(prob, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, stream=None):
    _bwd("gdr_gdn_bwd", prob, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, stream)


def kda_ckpt(prob, o, ht, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, stream=None):
    _ckpt("gdr_kda_ckpt", prob, o, ht, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, stream)


def gdn_ckpt(prob, o, ht, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, stream=None):
    _ckpt("gdr_gdn_ckpt", prob, o, ht, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, stream)


def kda_ckpt_noalloc(prob, o, ht, dout, dht, dq, dk, dv, dg, dbeta, dh0, stream=None):
    """gdr_kda_ckpt on the library's static per-device workspace (no workspace argument)."""
    _check(lib().gdr_kda_ckpt_noalloc(prob.cstruct, _ptr(o), _ptr(ht), _ptr(dout), _ptr(dht), _ptr(dq), _ptr(dk),
                                      _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), _stream(stream)))
