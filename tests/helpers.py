"""Small shared helpers for the test-suite (error metrics, tiny input builders)."""
import numpy as np


def rel_rms(x, ref):
    """||x - ref||_2 / ||ref||_2 over the whole tensor, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.sqrt(np.sum(ref * ref))
    num = np.sqrt(np.sum((x - ref) ** 2))
    if den == 0.0:
        return float(num)
    return float(num / den)


def max_abs(x, ref):
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64)))) if np.size(ref) else 0.0


def random_problem(rng, docs, Hqk, Hv, K, V, per_channel, h0=True, dht=True, gmin=-5.0):
    """fp64 inputs with the pages' distributions: q, k unit-norm rows, v ~ N(0,1),
    g ~ U(gmin, 0), beta = sigmoid(N(0,1))."""
    T = int(sum(docs))
    q = rng.standard_normal((T, Hqk, K))
    k = rng.standard_normal((T, Hqk, K))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Hv, V))
    g = gmin * rng.random((T, Hv, K) if per_channel else (T, Hv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, Hv))))
    cu = np.concatenate([[0], np.cumsum(docs)]).astype(np.int32)
    N = len(docs)
    h = 0.1 * rng.standard_normal((N, Hv, K, V)) if h0 else None
    dout = rng.standard_normal((T, Hv, V))
    dh = rng.standard_normal((N, Hv, K, V)) if dht else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu=cu, h0=h, dout=dout, dht=dh)
