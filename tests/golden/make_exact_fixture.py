"""Writes the exact-arithmetic fixtures of tests/test_golden_exact.py.

The gated delta rule read from the pages (FlashInfer PR #8218 and PR #7723
descriptions: per-token decay, erase and write of the state, output from the
updated state, state restarted at every document boundary) is evaluated here in
exact rational arithmetic (``fractions.Fraction``) on tiny problems:

    S'_t = Diag(a_t) S_{t-1}          a_t = exp(g_t): per channel (KDA) or per head (GDN)
    S_t  = S'_t + beta_t k_t (v_t - S'_t^T k_t)^T
    o_t  = scale * S_t^T q_t,         ht = S at the end of each document

The decay factors a are exact dyadic rationals and g = log(a) is stored
rounded to fp64.  Gradients of the loss sum(o * dout) + sum(ht * dht) come from
forward-mode differentiation with dual numbers over the same exact arithmetic,
one input element at a time (dg = a * dL/da), so they share nothing with the
oracle's hand-derived reverse mode.  This script imports neither the oracle nor
the library; run it from the repository root to regenerate the JSON files.
"""
import json
import math
import os
import random
from fractions import Fraction as F

HERE = os.path.dirname(os.path.abspath(__file__))


class D:
    """Dual number over exact rationals: value + eps * derivative."""
    __slots__ = ("v", "d")

    def __init__(self, v, d=F(0)):
        self.v, self.d = F(v), F(d)

    def __add__(self, o):
        return D(self.v + o.v, self.d + o.d)

    def __sub__(self, o):
        return D(self.v - o.v, self.d - o.d)

    def __mul__(self, o):
        return D(self.v * o.v, self.v * o.d + self.d * o.v)


def run(prob, seed_name=None, seed_index=None):
    """Forward pass in dual numbers; returns (o, ht, loss) with the derivative
    along the unit direction of input element prob[seed_name][seed_index]."""
    def inp(name, idx):
        x = prob[name]
        for i in idx:
            x = x[i]
        return D(x, 1 if (name == seed_name and tuple(idx) == seed_index) else 0)

    T, N, Hqk, Hv, K, V = (prob[n] for n in ("T", "N", "Hqk", "Hv", "K", "V"))
    cu, scale, per_channel = prob["cu"], D(prob["scale"]), prob["per_channel"]
    o = [[[None] * V for _ in range(Hv)] for _ in range(T)]
    ht = [[[[None] * V for _ in range(K)] for _ in range(Hv)] for _ in range(N)]
    loss = D(0)
    for n in range(N):
        for j in range(Hv):
            i = j // (Hv // Hqk)
            S = [[inp("h0", (n, j, c, e)) for e in range(V)] for c in range(K)]
            for t in range(cu[n], cu[n + 1]):
                a = [inp("a", (t, j, c)) if per_channel else inp("a", (t, j)) for c in range(K)]
                S = [[a[c] * S[c][e] for e in range(V)] for c in range(K)]
                kt = [inp("k", (t, i, c)) for c in range(K)]
                r = []
                for e in range(V):
                    acc = inp("v", (t, j, e))
                    for c in range(K):
                        acc = acc - S[c][e] * kt[c]
                    r.append(acc)
                b = inp("beta", (t, j))
                S = [[S[c][e] + b * kt[c] * r[e] for e in range(V)] for c in range(K)]
                for e in range(V):
                    acc = D(0)
                    for c in range(K):
                        acc = acc + S[c][e] * inp("q", (t, i, c))
                    o[t][j][e] = scale * acc
                    loss = loss + o[t][j][e] * D(prob["dout"][t][j][e])
            for c in range(K):
                for e in range(V):
                    ht[n][j][c][e] = S[c][e]
                    loss = loss + S[c][e] * D(prob["dht"][n][j][c][e])
    return o, ht, loss


def shape_of(x):
    s = []
    while isinstance(x, list):
        s.append(len(x))
        x = x[0]
    return tuple(s)


def indices(shape):
    if not shape:
        yield ()
        return
    for i in range(shape[0]):
        for rest in indices(shape[1:]):
            yield (i,) + rest


def tensor(shape, draw):
    if not shape:
        return draw()
    return [tensor(shape[1:], draw) for _ in range(shape[0])]


def make(name, docs, Hqk, Hv, K, V, per_channel, seed):
    rnd = random.Random(seed)
    dy = lambda den: (lambda: F(rnd.randint(-den, den), den))          # dyadic in [-1, 1]
    decay = lambda: F(rnd.choice([1, 2, 3, 4, 5, 6, 7, 8]), 8)          # a in (0, 1]
    beta = lambda: F(rnd.randint(0, 8), 8)
    T, N = sum(docs), len(docs)
    cu = [0]
    for d in docs:
        cu.append(cu[-1] + d)
    prob = dict(T=T, N=N, Hqk=Hqk, Hv=Hv, K=K, V=V, cu=cu, scale=F(1, 2), per_channel=per_channel,
                q=tensor((T, Hqk, K), dy(4)), k=tensor((T, Hqk, K), dy(4)), v=tensor((T, Hv, V), dy(4)),
                a=tensor((T, Hv, K) if per_channel else (T, Hv), decay), beta=tensor((T, Hv), beta),
                h0=tensor((N, Hv, K, V), dy(8)), dout=tensor((T, Hv, V), dy(4)), dht=tensor((N, Hv, K, V), dy(4)))
    o, ht, _ = run(prob)
    grads = {}
    for src, dst in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("a", "dg"), ("beta", "dbeta"), ("h0", "dh0")):
        shp = shape_of(prob[src])
        flat = []
        for idx in indices(shp):
            _, _, L = run(prob, src, idx)
            d = L.d
            if src == "a":  # dL/dg = a dL/da
                x = prob["a"]
                for i in idx:
                    x = x[i]
                d = d * x
            flat.append(float(d))
        grads[dst] = (list(shp), flat)

    def floats(x):
        return [floats(y) for y in x] if isinstance(x, list) else float(x.v if isinstance(x, D) else x)

    g = [[math.log(x) for x in row] if not per_channel else [[math.log(x) for x in col] for col in row]
         for row in prob["a"]]
    out = dict(name=name, citation="gated delta rule read from FlashInfer PR #8218 / PR #7723 descriptions; "
                                   "exact rational evaluation with forward-mode dual numbers",
               variant="kda" if per_channel else "gdn", cu_seqlens=cu, scale=0.5,
               q=floats(prob["q"]), k=floats(prob["k"]), v=floats(prob["v"]), g=g, beta=floats(prob["beta"]),
               h0=floats(prob["h0"]), dout=floats(prob["dout"]), dht=floats(prob["dht"]),
               o=floats(o), ht=floats(ht), grads=grads)
    with open(os.path.join(HERE, name + ".json"), "w") as f:
        json.dump(out, f)
    print("wrote", name)


if __name__ == "__main__":
    make("exact_kda_tiny", (3, 2), 2, 2, 3, 2, True, 1)
    make("exact_gdn_tiny", (2, 3), 1, 2, 3, 2, False, 2)
