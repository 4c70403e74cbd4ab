"""Oracle against exact rational arithmetic on tiny problems (tests/golden/).

The fixtures hold the outputs and gradients of the gated delta rule evaluated
in exact rationals by tests/golden/make_exact_fixture.py (gradients by
forward-mode dual numbers, one input element at a time), which imports neither
the oracle nor the library.  K = 3 and V = 2 differ, so a transposed state or
operand cannot pass; two documents per pack check the reset, h0 and dht enter.
The only inexact step on the oracle's side is fp64 rounding (exp of the stored
log-decay included), so the bound is a few hundred units in the last place.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CASES = ["exact_kda_tiny", "exact_gdn_tiny"]


def load(name):
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        d = json.load(f)
    arr = {k: np.asarray(d[k], dtype=np.float64) for k in ("q", "k", "v", "g", "beta", "h0", "dout", "dht", "o", "ht")}
    grads = {k: np.asarray(flat, dtype=np.float64).reshape(shape) for k, (shape, flat) in d["grads"].items()}
    return d, arr, grads


def close(x, ref, what):
    err = np.max(np.abs(x - ref))
    bound = 1e-13 * max(1.0, float(np.max(np.abs(ref))))
    assert err <= bound, "%s: max |oracle - exact| = %.3g > %.3g" % (what, err, bound)


@pytest.mark.parametrize("name", CASES)
def test_oracle_matches_exact_rationals(name):
    d, a, grads = load(name)
    cu = np.asarray(d["cu_seqlens"], dtype=np.int32)
    o, ht = oracle.forward(a["q"], a["k"], a["v"], a["g"], a["beta"], cu, a["h0"], scale=d["scale"])
    close(o, a["o"], name + " o")
    close(ht, a["ht"], name + " ht")
    g = oracle.backward(a["q"], a["k"], a["v"], a["g"], a["beta"], cu, a["dout"], a["h0"], a["dht"], scale=d["scale"])
    for key in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        close(g[key], grads[key], "%s %s" % (name, key))
