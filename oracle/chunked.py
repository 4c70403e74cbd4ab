"""fp64 NumPy evaluation of the gated delta rule through its 64-token chunk algebra.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  This is a second,
independent way to reach the token recurrence's result: the per-chunk WY form,
a sequential walk over chunk states and an adjoint walk.  It exists to
cross-check the token-form oracle (the two share no code) and to give
per-chunk intermediates for debugging.

The pages describe the chunked training pipeline only by its stages (FlashInfer
PR #8638 description: a prep program, a state walk that writes per-chunk
tapes, an output program; PR #7723: the adjoint walk over chunks).  The
algebra below is derived from the recurrence; for a chunk of L <= 64 tokens
with entering state S:

    G_r    = sum_{j<=r} g_j                      (in-chunk, per channel)
    E_rs   = sum_c k_rc k_sc exp(G_rc - G_sc)     (s < r)
    A      = diag(beta) E ;   T = (I + A)^-1
    W      = T (beta * k * exp(G)) ;   U = T (beta * v)
    Vn     = U - W S                              (the "new values", beta * r_t)
    Kbar_r = k_r * exp(G_last - G_r) ;  gamma = exp(G_last)
    S_next = diag(gamma) S + Kbar^T Vn
    M_rs   = sum_c q_rc k_sc exp(G_rc - G_sc)     (s <= r)
    O      = scale [ (q * exp(G)) S + M Vn ]

and the backward is the reverse mode of those lines (chain rule through T,
the exponentials and the in-chunk cumulative sum).
"""
from __future__ import annotations

import numpy as np

from . import as_f64

CHUNK = 64


def _chunk_factors(qc, kc, vc, gc, bc, per_channel):
    L, K = kc.shape
    if per_channel:
        G = np.cumsum(gc, axis=0)
    else:
        G = np.repeat(np.cumsum(gc)[:, None], K, axis=1)
    low_eq = np.tril(np.ones((L, L), dtype=bool))
    low = np.tril(np.ones((L, L), dtype=bool), -1)
    diff = G[:, None, :] - G[None, :, :]
    D = np.where(low_eq[:, :, None], np.exp(np.where(low_eq[:, :, None], diff, 0.0)), 0.0)
    E = np.einsum("rc,sc,rsc->rs", kc, kc, D) * low
    A = bc[:, None] * E
    T = np.linalg.inv(np.eye(L) + A)
    Gam = np.exp(G)
    Kt = kc * Gam
    W = T @ (bc[:, None] * Kt)
    U = T @ (bc[:, None] * vc)
    Kbar = kc * np.exp(G[-1][None, :] - G)
    gamma = np.exp(G[-1])
    M = np.einsum("rc,sc,rsc->rs", qc, kc, D) * low_eq
    Qt = qc * Gam
    return dict(G=G, D=D, E=E, A=A, T=T, Gam=Gam, Kt=Kt, W=W, U=U, Kbar=Kbar,
                gamma=gamma, M=M, Qt=Qt, low=low, low_eq=low_eq)


def _arrays(q, k, v, g, beta, cu_seqlens, h0, dout=None, dht=None):
    q, k, v, g, beta, h0, dout, dht = (as_f64(x) for x in (q, k, v, g, beta, h0, dout, dht))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return q, k, v, g, beta, h0, dout, dht, cu


def chunked_forward(q, k, v, g, beta, cu_seqlens, h0=None, scale=None, keep=False):
    """Returns (o, ht) and, with keep=True, a list of per-chunk records."""
    q, k, v, g, beta, h0, _, _, cu = _arrays(q, k, v, g, beta, cu_seqlens, h0)
    T, Hqk, K = q.shape
    Hv, V = v.shape[1:]
    grp = Hv // Hqk
    pc = g.ndim == 3
    scale = K ** -0.5 if scale is None else scale
    o = np.zeros((T, Hv, V))
    ht = np.zeros((len(cu) - 1, Hv, K, V))
    records = []
    for n in range(len(cu) - 1):
        for j in range(Hv):
            i = j // grp
            S = h0[n, j].copy() if h0 is not None else np.zeros((K, V))
            for t0 in range(cu[n], cu[n + 1], CHUNK):
                t1 = min(t0 + CHUNK, cu[n + 1])
                f = _chunk_factors(q[t0:t1, i], k[t0:t1, i], v[t0:t1, j],
                                   g[t0:t1, j], beta[t0:t1, j], pc)
                Vn = f["U"] - f["W"] @ S
                o[t0:t1, j] = scale * (f["Qt"] @ S + f["M"] @ Vn)
                if keep:
                    records.append(dict(doc=n, head=j, t0=t0, t1=t1, S=S.copy(), Vn=Vn, **f))
                S = f["gamma"][:, None] * S + f["Kbar"].T @ Vn
            ht[n, j] = S
    return (o, ht, records) if keep else (o, ht)


def chunked_backward(q, k, v, g, beta, cu_seqlens, dout, h0=None, dht=None, scale=None):
    """Chunk-algebra reverse mode; same outputs as ``oracle.backward``."""
    q, k, v, g, beta, h0, dout, dht, cu = _arrays(q, k, v, g, beta, cu_seqlens, h0, dout, dht)
    T, Hqk, K = q.shape
    Hv, V = v.shape[1:]
    grp = Hv // Hqk
    pc = g.ndim == 3
    scale = K ** -0.5 if scale is None else scale
    dq = np.zeros((T, Hqk, K))
    dk = np.zeros((T, Hqk, K))
    dv = np.zeros((T, Hv, V))
    dg = np.zeros(g.shape)
    dbeta = np.zeros((T, Hv))
    dh0 = np.zeros((len(cu) - 1, Hv, K, V))
    for n in range(len(cu) - 1):
        for j in range(Hv):
            i = j // grp
            S = h0[n, j].copy() if h0 is not None else np.zeros((K, V))
            starts = list(range(cu[n], cu[n + 1], CHUNK))
            states = []
            for t0 in starts:
                t1 = min(t0 + CHUNK, cu[n + 1])
                f = _chunk_factors(q[t0:t1, i], k[t0:t1, i], v[t0:t1, j],
                                   g[t0:t1, j], beta[t0:t1, j], pc)
                states.append(S)
                S = f["gamma"][:, None] * S + f["Kbar"].T @ (f["U"] - f["W"] @ S)
            dS = dht[n, j].copy() if dht is not None else np.zeros((K, V))
            for t0, S in zip(reversed(starts), reversed(states)):
                t1 = min(t0 + CHUNK, cu[n + 1])
                qc, kc, vc, bc = q[t0:t1, i], k[t0:t1, i], v[t0:t1, j], beta[t0:t1, j]
                f = _chunk_factors(qc, kc, vc, g[t0:t1, j], bc, pc)
                D, T_, W, M = f["D"], f["T"], f["W"], f["M"]
                Vn = f["U"] - W @ S
                dOp = scale * dout[t0:t1, j]
                # state and output adjoints
                dVn = M.T @ dOp + f["Kbar"] @ dS
                dS_prev = f["gamma"][:, None] * dS + f["Qt"].T @ dOp - W.T @ dVn
                dM = (dOp @ Vn.T) * f["low_eq"]
                dW = -dVn @ S.T
                dKbar = Vn @ dS.T
                dQt = dOp @ S.T
                # through the WY factors and the triangular inverse
                TdU = T_.T @ dVn
                TdW = T_.T @ dW
                dv[t0:t1, j] = bc[:, None] * TdU
                dKt = bc[:, None] * TdW
                dT = dVn @ (bc[:, None] * vc).T + dW @ (bc[:, None] * f["Kt"]).T
                dA = -(T_.T @ dT @ T_.T) * f["low"]
                dbeta[t0:t1, j] = (np.sum(TdU * vc, 1) + np.sum(TdW * f["Kt"], 1)
                                   + np.sum(dA * f["E"], 1))
                # gated products: row-side and column-side sums
                qM_row = np.einsum("rs,sc,rsc->rc", dM, kc, D)
                kM_col = np.einsum("rs,rc,rsc->sc", dM, qc, D)
                kA_row = bc[:, None] * np.einsum("rs,sc,rsc->rc", dA, kc, D)
                kA_col = np.einsum("rs,r,rc,rsc->sc", dA, bc, kc, D)
                Gam = f["Gam"]
                decay_last = np.exp(f["G"][-1][None, :] - f["G"])
                dq[t0:t1, i] += Gam * dQt + qM_row
                dk[t0:t1, i] += Gam * dKt + decay_last * dKbar + kM_col + kA_row + kA_col
                dG = (f["Qt"] * dQt + qc * qM_row - kc * kM_col + kc * kA_row - kc * kA_col
                      + f["Kt"] * dKt - f["Kbar"] * dKbar)
                dG[-1] += np.sum(f["Kbar"] * dKbar, 0) + f["gamma"] * np.sum(dS * S, 1)
                dgc = np.cumsum(dG[::-1], axis=0)[::-1]
                if pc:
                    dg[t0:t1, j] = dgc
                else:
                    dg[t0:t1, j] = dgc.sum(1)
                dS = dS_prev
            dh0[n, j] = dS
    return {"dq": dq, "dk": dk, "dv": dv, "dg": dg, "dbeta": dbeta, "dh0": dh0}
