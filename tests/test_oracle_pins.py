"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test fixes the oracle to something independent: central finite
differences, closed forms of special cases (derived from the recurrence by
hand), a second algorithm (the chunk algebra), and invariants (document reset,
KDA/GDN equivalences).  A dropped term, a sign or index error, or a transposed
operand anywhere in the forward or the hand-derived backward fails at least
one of them.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.chunked import chunked_backward, chunked_forward

from helpers import max_abs, random_problem, rel_rms


def _fwd(p, **kw):
    return oracle.forward(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu"], p.get("h0"), **kw)


def _bwd(p, **kw):
    return oracle.backward(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu"], p["dout"],
                           p.get("h0"), p.get("dht"), **kw)


def _loss(p):
    o, ht = _fwd(p, threads=1)
    return oracle.loss(o, ht, p["dout"], p.get("dht"))


# --------------------------------------------------------------------------
# Pin 1: central finite differences of the loss sum(o*dout) + sum(ht*dht)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["kda", "gdn"])
def test_finite_differences_every_entry(variant):
    rng = np.random.default_rng(11 if variant == "kda" else 12)
    if variant == "kda":
        p = random_problem(rng, [23, 41], 1, 1, 8, 8, per_channel=True)
    else:
        p = random_problem(rng, [23, 41], 1, 3, 8, 8, per_channel=False)
    grads = _bwd(p, threads=1)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}
    eps = 1e-6
    for name, gname in names.items():
        x = p[name]
        fd = np.zeros_like(x)
        flat = x.reshape(-1)
        for idx in range(flat.size):
            keep = flat[idx]
            flat[idx] = keep + eps
            lp = _loss(p)
            flat[idx] = keep - eps
            lm = _loss(p)
            flat[idx] = keep
            fd.reshape(-1)[idx] = (lp - lm) / (2 * eps)
        an = grads[gname]
        scale = max(1.0, np.abs(an).max())
        assert np.abs(fd - an).max() <= 1e-6 * scale, (name, np.abs(fd - an).max())


@pytest.mark.parametrize("variant", ["kda", "gdn"])
def test_finite_differences_directional_head_dim_128(variant):
    rng = np.random.default_rng(21 if variant == "kda" else 22)
    if variant == "kda":
        p = random_problem(rng, [23, 41], 1, 1, 128, 128, per_channel=True)
    else:
        p = random_problem(rng, [23, 41], 1, 3, 128, 128, per_channel=False)
    grads = _bwd(p, threads=4)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}
    eps = 1e-6
    for trial in range(16):
        dirs = {n: rng.standard_normal(p[n].shape) for n in names}
        analytic = sum(float(np.sum(grads[names[n]] * dirs[n])) for n in names)
        for n in names:
            p[n] += eps * dirs[n]
        lp = _loss(p)
        for n in names:
            p[n] -= 2 * eps * dirs[n]
        lm = _loss(p)
        for n in names:
            p[n] += eps * dirs[n]
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - analytic) <= 1e-6 * max(1.0, abs(analytic)), (trial, fd, analytic)


# --------------------------------------------------------------------------
# Pin 2a: beta = 0, g = 0, h0 = 0 -> the state never moves; dq, dk, dv and
# dg vanish, dh0 = scale sum_t q_t dout_t^T, and dbeta is causal linear
# attention:  dbeta_s = scale * sum_{t >= s, same doc} (q_t . k_s)(dout_t . v_s)
# --------------------------------------------------------------------------
def test_beta_zero_linear_attention_gradient():
    rng = np.random.default_rng(3)
    p = random_problem(rng, [50, 17, 90], 2, 2, 32, 24, per_channel=True, h0=False, dht=False)
    p["beta"][:] = 0.0
    p["g"][:] = 0.0
    o, ht = _fwd(p)
    gr = _bwd(p)
    assert np.all(o == 0) and np.all(ht == 0)
    for name in ("dq", "dk", "dv", "dg"):
        assert np.all(gr[name] == 0), name
    scale = 32 ** -0.5
    cu = p["cu"]
    # the initial state's gradient: dh0 = scale * sum_t q_t dout_t^T over the document
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        for h in range(2):
            ref_h0 = scale * p["q"][a:b, h].T @ p["dout"][a:b, h]
            assert max_abs(gr["dh0"][n, h], ref_h0) <= 1e-12
    ref = np.zeros_like(p["beta"])
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        for h in range(2):
            qk = p["q"][a:b, h] @ p["k"][a:b, h].T          # [t, s]
            dv_ = p["dout"][a:b, h] @ p["v"][a:b, h].T      # [t, s]
            causal = np.triu(np.ones((b - a, b - a)))        # s <= t  -> [s, t]
            ref[a:b, h] = scale * np.sum(causal * (qk * dv_).T, axis=1)
    assert max_abs(gr["dbeta"], ref) <= 1e-12 * max(1.0, np.abs(ref).max())


# --------------------------------------------------------------------------
# Pin 2b: g = 0, h0 = 0, orthonormal keys within a document, any beta:
#   S_t = sum_{s<=t} beta_s k_s v_s^T  ->  o_t = scale sum_{s<=t} beta_s (q_t.k_s) v_s
# The closed form is exact for every q, v, beta on that key set, so its
# autograd also pins dq, dv and dbeta.
# --------------------------------------------------------------------------
def test_orthonormal_keys_closed_form():
    rng = np.random.default_rng(4)
    K = V = 128
    docs = [100, 60]
    p = random_problem(rng, docs, 1, 1, K, V, per_channel=True, h0=False, dht=False)
    p["g"][:] = 0.0
    cu = p["cu"]
    for n in range(len(docs)):
        Q, _ = np.linalg.qr(rng.standard_normal((K, K)))
        p["k"][cu[n]:cu[n + 1], 0] = Q[:, : docs[n]].T
    scale = K ** -0.5
    o, _ = _fwd(p)
    gr = _bwd(p)

    q = torch.tensor(p["q"][:, 0], requires_grad=True)
    v = torch.tensor(p["v"][:, 0], requires_grad=True)
    b = torch.tensor(p["beta"][:, 0], requires_grad=True)
    k = torch.tensor(p["k"][:, 0])
    outs = []
    for n in range(len(docs)):
        a, e = cu[n], cu[n + 1]
        qk = q[a:e] @ k[a:e].T
        causal = torch.tril(torch.ones(e - a, e - a, dtype=torch.float64))
        outs.append(scale * (qk * causal * b[a:e][None, :]) @ v[a:e])
    ref = torch.cat(outs)
    assert max_abs(o[:, 0], ref.detach().numpy()) <= 1e-13
    (ref * torch.tensor(p["dout"][:, 0])).sum().backward()
    assert max_abs(gr["dq"][:, 0], q.grad.numpy()) <= 1e-12
    assert max_abs(gr["dv"][:, 0], v.grad.numpy()) <= 1e-12
    assert max_abs(gr["dbeta"][:, 0], b.grad.numpy()) <= 1e-12


# --------------------------------------------------------------------------
# Pin 3: axis-aligned keys k_t = e_{pi(t)}: every state row is its own
# exponential moving average,
#   row_c(S_t) = a_tc (1 - beta_t [pi(t)=c]) row_c(S_{t-1}) + beta_t [pi(t)=c] v_t
#   o_t = scale sum_c q_tc row_c(S_t)
# pi(t) = t mod 8 repeats keys inside a 64-token chunk.  Autograd of this
# form pins dq, dv, dg, dbeta and dh0 at head dim 128 (dk is off the key set).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("per_channel", [True, False])
def test_axis_aligned_keys_ema(per_channel):
    rng = np.random.default_rng(5)
    K = V = 128
    docs = [77, 0, 150]
    p = random_problem(rng, docs, 1, 1, K, V, per_channel=per_channel)
    T = sum(docs)
    cu = p["cu"]
    pi = np.zeros(T, dtype=np.int64)
    for n in range(len(docs)):
        idx = np.arange(docs[n])
        pi[cu[n]:cu[n + 1]] = idx % 8
    p["k"][:] = 0.0
    p["k"][np.arange(T), 0, pi] = 1.0
    scale = K ** -0.5
    o, ht = _fwd(p)
    gr = _bwd(p)

    q = torch.tensor(p["q"][:, 0], requires_grad=True)
    v = torch.tensor(p["v"][:, 0], requires_grad=True)
    g = torch.tensor(p["g"][:, 0], requires_grad=True)
    b = torch.tensor(p["beta"][:, 0], requires_grad=True)
    h0 = torch.tensor(p["h0"][:, 0], requires_grad=True)
    outs, finals = [], []
    for n in range(len(docs)):
        S = h0[n]
        for t in range(cu[n], cu[n + 1]):
            a = torch.exp(g[t]) if per_channel else torch.exp(g[t]).expand(K)
            onehot = torch.zeros(K, dtype=torch.float64)
            onehot[pi[t]] = 1.0
            keep = a * (1.0 - b[t] * onehot)
            S = keep[:, None] * S + (b[t] * onehot)[:, None] * v[t][None, :]
            outs.append(scale * (q[t][:, None] * S).sum(0))
        finals.append(S)
    ref_o = torch.stack(outs)
    ref_ht = torch.stack(finals)
    assert max_abs(o[:, 0], ref_o.detach().numpy()) <= 1e-12
    assert max_abs(ht[:, 0], ref_ht.detach().numpy()) <= 1e-12
    loss = (ref_o * torch.tensor(p["dout"][:, 0])).sum() + (ref_ht * torch.tensor(p["dht"][:, 0])).sum()
    loss.backward()
    for name, t in (("dq", q), ("dv", v), ("dg", g), ("dbeta", b), ("dh0", h0)):
        assert max_abs(gr[name][:, 0], t.grad.numpy()) <= 1e-11 * max(1.0, np.abs(t.grad.numpy()).max()), name


# --------------------------------------------------------------------------
# Pin 4: overwrite property.  k_t = e_1, beta = 1, g = 0 -> the state is
# e_1 v_t^T after every token, so o_t = scale q_t1 v_t.
# --------------------------------------------------------------------------
def test_overwrite_property():
    rng = np.random.default_rng(6)
    p = random_problem(rng, [33, 70], 1, 1, 16, 16, per_channel=True, h0=False, dht=False)
    p["k"][:] = 0.0
    p["k"][:, 0, 0] = 1.0
    p["beta"][:] = 1.0
    p["g"][:] = 0.0
    o, ht = _fwd(p)
    ref = 16 ** -0.5 * p["q"][:, 0, 0][:, None] * p["v"][:, 0]
    assert max_abs(o[:, 0], ref) <= 1e-14
    last = p["cu"][1:] - 1
    for n, t in enumerate(last):
        expect = np.zeros((16, 16))
        expect[0] = p["v"][t, 0]
        assert max_abs(ht[n, 0], expect) <= 1e-14


# --------------------------------------------------------------------------
# Pin 5: beta = 0 (no writes), any g, h0 != 0, dht = 0:
#   o_t   = scale (exp(G_t) * q_t)^T h0,    G_t = sum_{j<=t in doc} g_j
#   dh0   = scale sum_t (exp(G_t) * q_t) dout_t^T
#   dg_tc = scale sum_{t'>=t} q_t'c exp(G_t'c) (h0 dout_t')_c
# (GDN: G is a scalar per token and dg_t sums the channel terms.)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("per_channel", [True, False])
def test_gate_and_initial_state_closed_form(per_channel):
    rng = np.random.default_rng(7)
    K, V = 32, 16
    p = random_problem(rng, [40, 90], 1, 1, K, V, per_channel=per_channel, dht=False)
    p["beta"][:] = 0.0
    scale = K ** -0.5
    o, ht = _fwd(p)
    gr = _bwd(p)
    cu = p["cu"]
    for n in range(2):
        a, e = cu[n], cu[n + 1]
        gg = p["g"][a:e, 0]
        G = np.cumsum(gg, axis=0) if per_channel else np.cumsum(gg)[:, None] * np.ones((1, K))
        qg = np.exp(G) * p["q"][a:e, 0]                     # [t, K]
        h = p["h0"][n, 0]
        assert max_abs(o[a:e, 0], scale * qg @ h) <= 1e-13
        do = p["dout"][a:e, 0]
        assert max_abs(gr["dh0"][n, 0], scale * qg.T @ do) <= 1e-12
        term = scale * qg * (do @ h.T)                        # [t', c]
        dg_ref = np.cumsum(term[::-1], axis=0)[::-1]
        if not per_channel:
            dg_ref = dg_ref.sum(1)
        assert max_abs(gr["dg"][a:e, 0], dg_ref) <= 1e-12 * max(1.0, np.abs(dg_ref).max())
        G_last = G[-1]
        assert max_abs(ht[n, 0], np.exp(G_last)[:, None] * h) <= 1e-13


# --------------------------------------------------------------------------
# Pin 6: an independent algorithm -- the chunk algebra -- agrees with the
# token recurrence (forward and backward) on ragged packs with partial chunks.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["kda", "gdn"])
def test_chunked_form_matches_token_form(variant):
    rng = np.random.default_rng(8)
    docs = [130, 1, 64, 200, 0, 65]
    if variant == "kda":
        p = random_problem(rng, docs, 2, 2, 128, 128, per_channel=True)
    else:
        p = random_problem(rng, docs, 2, 6, 128, 128, per_channel=False)
    o, ht = _fwd(p)
    gr = _bwd(p)
    o2, ht2 = chunked_forward(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu"], p["h0"])
    gr2 = chunked_backward(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu"], p["dout"], p["h0"], p["dht"])
    assert rel_rms(o2, o) <= 1e-9 and rel_rms(ht2, ht) <= 1e-9
    for key in gr:
        assert rel_rms(gr2[key], gr[key]) <= 1e-9, key


# --------------------------------------------------------------------------
# Pin 7: document reset.  A packed batch equals its documents run one at a
# time, and perturbing one document leaves every other document's outputs
# and gradients bitwise unchanged.
# --------------------------------------------------------------------------
def test_document_reset_invariant():
    rng = np.random.default_rng(9)
    docs = [37, 64, 0, 99]
    p = random_problem(rng, docs, 2, 2, 16, 16, per_channel=True)
    o, ht = _fwd(p, threads=3)
    gr = _bwd(p, threads=3)
    cu = p["cu"]
    for n in range(len(docs)):
        a, e = cu[n], cu[n + 1]
        sub = {key: p[key][a:e] for key in ("q", "k", "v", "g", "beta", "dout")}
        sub["cu"] = np.array([0, e - a], dtype=np.int32)
        sub["h0"] = p["h0"][n:n + 1]
        sub["dht"] = p["dht"][n:n + 1]
        o1, ht1 = _fwd(sub, threads=1)
        gr1 = _bwd(sub, threads=1)
        assert np.array_equal(o1, o[a:e]) and np.array_equal(ht1, ht[n:n + 1])
        for key in ("dq", "dk", "dv", "dg", "dbeta"):
            assert np.array_equal(gr1[key], gr[key][a:e]), key
        assert np.array_equal(gr1["dh0"], gr["dh0"][n:n + 1])
        if e - a == 0:  # empty document: ht = h0, dh0 = dht
            assert np.array_equal(ht1[0], p["h0"][n]) and np.array_equal(gr1["dh0"][0], p["dht"][n])
    # perturb document 1 and check the others
    q2 = dict(p)
    q2 = {key: (val.copy() if isinstance(val, np.ndarray) else val) for key, val in p.items()}
    a, e = cu[1], cu[2]
    for key in ("q", "k", "v", "g", "beta", "dout"):
        q2[key][a:e] += 0.1 * rng.standard_normal(q2[key][a:e].shape)
    o2, ht2 = _fwd(q2, threads=3)
    gr2 = _bwd(q2, threads=3)
    mask = np.ones(cu[-1], dtype=bool)
    mask[a:e] = False
    assert np.array_equal(o2[mask], o[mask])
    assert not np.array_equal(o2[a:e], o[a:e])
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.array_equal(gr2[key][mask], gr[key][mask]), key


# --------------------------------------------------------------------------
# Pin 8: KDA <-> GDN.  GDN with one value head per Q/K head is KDA with the
# scalar gate broadcast over channels (dg = channel sum of KDA's dg); GDN with
# three value heads per group is KDA on replicated q, k with dq, dk summed
# over the group.
# --------------------------------------------------------------------------
def test_gdn_equals_kda_with_broadcast_gate():
    rng = np.random.default_rng(10)
    docs = [70, 130]
    p = random_problem(rng, docs, 2, 2, 32, 32, per_channel=False)
    kda = dict(p)
    kda["g"] = np.repeat(p["g"][:, :, None], 32, axis=2)
    o1, ht1 = _fwd(p)
    o2, ht2 = _fwd(kda)
    assert rel_rms(o1, o2) <= 1e-14 and rel_rms(ht1, ht2) <= 1e-14
    g1 = _bwd(p)
    g2 = _bwd(kda)
    for key in ("dq", "dk", "dv", "dbeta", "dh0"):
        assert rel_rms(g1[key], g2[key]) <= 1e-13, key
    assert rel_rms(g1["dg"], g2["dg"].sum(-1)) <= 1e-13


def test_gdn_groups_equal_replicated_kda():
    rng = np.random.default_rng(13)
    docs = [90, 45]
    G = 3
    p = random_problem(rng, docs, 2, 2 * G, 32, 32, per_channel=False)
    kda = dict(p)
    kda["q"] = np.repeat(p["q"], G, axis=1)
    kda["k"] = np.repeat(p["k"], G, axis=1)
    o1, _ = _fwd(p)
    o2, _ = _fwd(kda)
    assert rel_rms(o1, o2) <= 1e-14
    g1 = _bwd(p)
    g2 = _bwd(kda)
    T = sum(docs)
    for key in ("dq", "dk"):
        summed = g2[key].reshape(T, 2, G, 32).sum(2)
        assert rel_rms(g1[key], summed) <= 1e-13, key
    for key in ("dv", "dg", "dbeta", "dh0"):
        assert rel_rms(g1[key], g2[key]) <= 1e-13, key


def test_oracle_rejects_bad_problem():
    rng = np.random.default_rng(14)
    p = random_problem(rng, [10, 10], 2, 3, 8, 8, per_channel=False)  # 3 % 2 != 0
    with pytest.raises(ValueError):
        _fwd(p)


# --------------------------------------------------------------------------
# Input activations: in-kernel q/k L2 norm and beta sigmoid
# --------------------------------------------------------------------------
def _loss_act(p, **act):
    o, ht = oracle.forward_act(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu"], p.get("h0"), threads=1, **act)
    return oracle.loss(o, ht, p["dout"], p.get("dht"))


@pytest.mark.parametrize("variant", ["kda", "gdn"])
def test_activations_finite_differences(variant):
    """d/dq, d/dk, d/dbeta through the L2 norm and the sigmoid, entry by entry."""
    rng = np.random.default_rng(31 if variant == "kda" else 32)
    if variant == "kda":
        p = random_problem(rng, [19, 30], 1, 1, 8, 8, per_channel=True)
    else:
        p = random_problem(rng, [19, 30], 1, 3, 8, 8, per_channel=False)
    p["beta"] = rng.normal(size=p["beta"].shape)  # logits
    act = dict(qk_l2norm=True, beta_sigmoid=True)
    grads = oracle.backward_act(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu"], p["dout"], p.get("h0"),
                                p.get("dht"), threads=1, **act)
    eps = 1e-6
    for name, gname in {"q": "dq", "k": "dk", "beta": "dbeta"}.items():
        x = p[name]
        flat = x.reshape(-1)
        fd = np.zeros_like(x)
        for idx in range(flat.size):
            keep = flat[idx]
            flat[idx] = keep + eps
            lp = _loss_act(p, **act)
            flat[idx] = keep - eps
            lm = _loss_act(p, **act)
            flat[idx] = keep
            fd.reshape(-1)[idx] = (lp - lm) / (2 * eps)
        an = grads[gname]
        assert np.abs(an - fd).max() <= 1e-6 * max(1.0, np.abs(an).max()), name


def test_l2norm_scale_invariance_and_orthogonal_gradient():
    """q -> c q (c > 0) leaves the normalised forward unchanged (up to the epsilon),
    and each row's gradient is orthogonal to the row: sum_c dq_c q_c equals
    <q_hat, dq_hat> EPS / (|q|^2 + EPS), which is zero but for the epsilon."""
    rng = np.random.default_rng(33)
    p = random_problem(rng, [37, 20], 2, 2, 16, 16, per_channel=True)
    p["q"] *= 3.0  # rows well away from zero norm
    p["k"] *= 3.0
    o1, h1 = oracle.forward_act(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu"], p.get("h0"), qk_l2norm=True)
    o2, h2 = oracle.forward_act(2.5 * p["q"], 0.4 * p["k"], p["v"], p["g"], p["beta"], p["cu"], p.get("h0"),
                                qk_l2norm=True)
    assert np.abs(o1 - o2).max() <= 1e-6 * np.abs(o1).max()
    assert np.abs(h1 - h2).max() <= 1e-6 * np.abs(h1).max()
    gr = oracle.backward_act(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu"], p["dout"], p.get("h0"),
                             p.get("dht"), qk_l2norm=True)
    for x, d in ((p["q"], gr["dq"]), (p["k"], gr["dk"])):
        radial = np.sum(x * d, axis=-1)
        assert np.abs(radial).max() <= 1e-6 * np.abs(d).max() * np.abs(x).max() * x.shape[-1]
    # unit rows pass through the norm unchanged (to the epsilon)
    qu = p["q"] / np.linalg.norm(p["q"], axis=-1, keepdims=True)
    ku = p["k"] / np.linalg.norm(p["k"], axis=-1, keepdims=True)
    oa, _ = oracle.forward_act(qu, ku, p["v"], p["g"], p["beta"], p["cu"], p.get("h0"), qk_l2norm=True)
    ob, _ = oracle.forward(qu, ku, p["v"], p["g"], p["beta"], p["cu"], p.get("h0"))
    assert np.abs(oa - ob).max() <= 1e-5 * np.abs(ob).max()
