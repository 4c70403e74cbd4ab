"""Plain fp64 CPU oracle for gated delta-rule attention (KDA / GDN).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and it
shares no code with that path.

Two independent evaluations live here:

* ``forward`` / ``backward``: the token-by-token recurrence and its
  hand-derived reverse mode, in C (``gdr_oracle.c``), fp64, OpenMP over
  (document, Q/K head) units.  This is the definition the GPU path is held to.
* ``oracle.chunked``: a separate NumPy fp64 evaluation of the same quantities
  through the 64-token chunk algebra (WY factors, state walk, adjoint walk).
  It is used only to cross-check the token form and to inspect intermediates.

Inputs are upcast exactly from their stored bits (bf16 / fp32 -> fp64).
Shapes: q, k [T, Hqk, K]; v, dout [T, Hv, V]; g [T, Hv, K] (per-channel, KDA)
or [T, Hv] (scalar, GDN); beta [T, Hv]; h0, dht [N, Hv, K, V];
cu_seqlens [N+1] (int).  Value head j reads Q/K head j // (Hv // Hqk).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            ip = ctypes.POINTER(ctypes.c_int32)
            i = ctypes.c_int
            lib.gdr_oracle_forward.argtypes = [i, i, i, i, i, i, i, dp, dp, dp, dp, dp, ip, dp,
                                               ctypes.c_double, dp, dp, i]
            lib.gdr_oracle_forward.restype = ctypes.c_int
            lib.gdr_oracle_backward.argtypes = [i, i, i, i, i, i, i, dp, dp, dp, dp, dp, ip, dp,
                                                ctypes.c_double, dp, dp, dp, dp, dp, dp, dp, dp, i]
            lib.gdr_oracle_backward.restype = ctypes.c_int
            _lib = lib
    return _lib


def default_threads() -> int:
    """Threads = the CPUs this process may run on (not the host's total)."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def as_f64(x):
    """Exact upcast of a torch tensor or array (bf16 / fp16 / fp32 / fp64) to fp64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        import torch

        x = x.detach().to("cpu")
        if x.dtype != torch.float64:
            x = x.to(torch.float64)
        return np.ascontiguousarray(x.numpy())
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _shapes(q, v, g, cu):
    T, Hqk, K = q.shape
    Hv, V = v.shape[1], v.shape[2]
    per_channel = 1 if g.ndim == 3 else 0
    N = len(cu) - 1
    return T, N, Hqk, Hv, K, V, per_channel


def forward(q, k, v, g, beta, cu_seqlens, h0=None, scale=None, threads=None):
    """Token-recurrence forward.  Returns (o [T,Hv,V], ht [N,Hv,K,V]) in fp64."""
    lib = _load()
    q, k, v, g, beta, h0 = (as_f64(x) for x in (q, k, v, g, beta, h0))
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T, N, Hqk, Hv, K, V, pc = _shapes(q, v, g, cu)
    if scale is None:
        scale = K ** -0.5
    o = np.zeros((T, Hv, V))
    ht = np.zeros((N, Hv, K, V))
    rc = lib.gdr_oracle_forward(T, N, Hqk, Hv, K, V, pc, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta), _ptr(cu, ctypes.c_int32), _ptr(h0), float(scale),
                                _ptr(o), _ptr(ht), threads or default_threads())
    if rc:
        raise ValueError("oracle forward rejected the problem (code %d)" % rc)
    return o, ht


def backward(q, k, v, g, beta, cu_seqlens, dout, h0=None, dht=None, scale=None, threads=None):
    """Hand-derived reverse mode of the recurrence.

    Returns a dict with dq, dk [T,Hqk,K]; dv [T,Hv,V]; dg (g's shape);
    dbeta [T,Hv]; dh0 [N,Hv,K,V]; all fp64.
    """
    lib = _load()
    q, k, v, g, beta, h0, dout, dht = (as_f64(x) for x in (q, k, v, g, beta, h0, dout, dht))
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T, N, Hqk, Hv, K, V, pc = _shapes(q, v, g, cu)
    if scale is None:
        scale = K ** -0.5
    dq = np.zeros((T, Hqk, K))
    dk = np.zeros((T, Hqk, K))
    dv = np.zeros((T, Hv, V))
    dg = np.zeros(g.shape)
    dbeta = np.zeros((T, Hv))
    dh0 = np.zeros((N, Hv, K, V))
    rc = lib.gdr_oracle_backward(T, N, Hqk, Hv, K, V, pc, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                 _ptr(beta), _ptr(cu, ctypes.c_int32), _ptr(h0), float(scale),
                                 _ptr(dout), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                 _ptr(dbeta), _ptr(dh0), threads or default_threads())
    if rc:
        raise ValueError("oracle backward failed (code %d)" % rc)
    return {"dq": dq, "dk": dk, "dv": dv, "dg": dg, "dbeta": dbeta, "dh0": dh0}


# ---------------------------------------------------------------------------
# Input activations (optional, applied before the recurrence)
#
# The GDN shapes of PR #8638 (benchmark shapes paragraph) normalise q and k
# inside the kernel, the inverse norm kept for the backward (its review notes
# on qk_rstd); PR #8218 (baselines paragraph) names the L2 norm and the beta
# sigmoid together as in-kernel steps.  No page gives the epsilon, so the
# plainest reading is
# taken: q_hat = q * (sum_c q_c^2 + EPS)^(-1/2) with EPS = 1e-6 per (token,
# head) row, and beta = 1 / (1 + exp(-b)).  The backward is the chain rule
# through these maps:
#   d q = rstd * (d q_hat - q_hat * <q_hat, d q_hat>)      (per row)
#   d b = d beta * beta * (1 - beta)
# ---------------------------------------------------------------------------
L2NORM_EPS = 1e-6


def l2norm_rows(x):
    """Rows of x (last axis) scaled to unit L2 norm: returns (x_hat, rstd), fp64."""
    x = as_f64(x)
    rstd = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2NORM_EPS)
    return x * rstd, rstd


def l2norm_rows_backward(x_hat, rstd, dx_hat):
    """Gradient through l2norm_rows, from the normalised rows and their rstd."""
    dot = np.sum(x_hat * dx_hat, axis=-1, keepdims=True)
    return rstd * (dx_hat - x_hat * dot)


def sigmoid(b):
    b = as_f64(b)
    return 1.0 / (1.0 + np.exp(-b))


def _activate(q, k, beta, qk_l2norm, beta_sigmoid):
    q, k, beta = as_f64(q), as_f64(k), as_f64(beta)
    rq = rk = None
    if qk_l2norm:
        q, rq = l2norm_rows(q)
        k, rk = l2norm_rows(k)
    if beta_sigmoid:
        beta = sigmoid(beta)
    return q, k, beta, rq, rk


def forward_act(q, k, v, g, beta, cu_seqlens, h0=None, scale=None, threads=None, qk_l2norm=False,
                beta_sigmoid=False):
    """``forward`` with the input activations applied first."""
    qa, ka, ba, _, _ = _activate(q, k, beta, qk_l2norm, beta_sigmoid)
    return forward(qa, ka, v, g, ba, cu_seqlens, h0, scale, threads)


def backward_act(q, k, v, g, beta, cu_seqlens, dout, h0=None, dht=None, scale=None, threads=None,
                 qk_l2norm=False, beta_sigmoid=False):
    """``backward`` with respect to the raw inputs of ``forward_act``."""
    qa, ka, ba, rq, rk = _activate(q, k, beta, qk_l2norm, beta_sigmoid)
    grads = backward(qa, ka, v, g, ba, cu_seqlens, dout, h0, dht, scale, threads)
    if qk_l2norm:
        grads["dq"] = l2norm_rows_backward(qa, rq, grads["dq"])
        grads["dk"] = l2norm_rows_backward(ka, rk, grads["dk"])
    if beta_sigmoid:
        grads["dbeta"] = grads["dbeta"] * ba * (1.0 - ba)
    return grads


def loss(o, ht, dout, dht=None):
    """The scalar whose gradient ``backward`` returns: sum(o*dout) + sum(ht*dht)."""
    val = float(np.sum(o * as_f64(dout)))
    if dht is not None:
        val += float(np.sum(ht * as_f64(dht)))
    return val
