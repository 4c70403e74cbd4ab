"""GPU parity: libgdr (through its C ABI) against the fp64 oracle, element by element.

Small packs span several 64-token chunks, partial last chunks, single-token
and empty documents, initial states and final-state gradients; the pages'
workloads 0 and 1 run whole.  Larger workloads are in test_gpu_workloads.py.
"""
import numpy as np
import pytest
import torch

from chunked_gated_delta_14_amd import workloads
from gpu_runner import compare, oracle_all, run_gdr
from helpers import rel_rms

pytestmark = pytest.mark.gpu

SMALL = [
    # (variant, docs, H_qk, H_v, h0, dht)
    ("kda", (64,), 1, 1, False, False),
    ("kda", (200, 312), 2, 2, False, False),
    ("kda", (1, 63, 64, 65, 130, 7), 2, 2, True, True),
    ("kda", (0, 100, 0, 257), 3, 3, True, True),
    ("gdn", (64,), 1, 1, False, False),
    ("gdn", (130, 1, 200), 1, 3, True, True),
    ("gdn", (77, 64, 129), 2, 6, False, True),
    ("gdn", (70, 190), 2, 4, True, True),   # groups of 2 value heads
    ("gdn", (130, 65), 1, 4, False, True),  # one group of 4
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "%s_%s_h%d_%d" % (c[0], "-".join(map(str, c[1])), c[2], c[3]))
def test_small_pack_parity(case):
    variant, docs, hqk, hv, h0, dht = case
    w = workloads.custom(variant, docs, hqk, hv, with_h0=h0, seed=sum(docs) + hv)
    inp = workloads.make_inputs(w, device="cpu", dht=dht)
    print("[case]", w.name, flush=True)
    got = run_gdr(variant, inp, dht=inp["dht"])
    ref = oracle_all(variant, inp, dht=inp["dht"])
    compare(got, ref, label=w.name)


ACT = [
    # (variant, docs, H_qk, H_v): raw q, k rows of varying norm, beta as logits
    ("kda", (1, 63, 64, 65, 130, 7), 2, 2),
    ("gdn", (130, 1, 200), 1, 3),
    ("gdn", (77, 64, 129), 2, 6),
]


@pytest.mark.parametrize("case", ACT, ids=lambda c: "%s_%s_h%d_%d" % (c[0], "-".join(map(str, c[1])), c[2], c[3]))
def test_input_activations_parity(case):
    """In-kernel q/k L2 norm and beta sigmoid (GDR_IN_QK_L2NORM | GDR_IN_BETA_SIGMOID)
    against the oracle with the same activations, forward and backward."""
    import chunked_gated_delta_14_amd as gdr

    variant, docs, hqk, hv = case
    w = workloads.custom(variant, docs, hqk, hv, with_h0=True, seed=sum(docs) + 7 * hv)
    inp = workloads.make_inputs(w, device="cpu", dht=True)
    gen = torch.Generator().manual_seed(sum(docs))
    T = w.T
    for name in ("q", "k"):
        x = inp[name].float()
        inp[name] = (x * (0.25 + 4.0 * torch.rand((T, hqk, 1), generator=gen))).to(torch.bfloat16)
    inp["beta"] = torch.randn(tuple(inp["beta"].shape), generator=gen).to(inp["beta"].dtype)
    print("[case]", w.name, "activations", flush=True)
    got = run_gdr(variant, inp, dht=inp["dht"], input_flags=gdr.GDR_IN_QK_L2NORM | gdr.GDR_IN_BETA_SIGMOID)
    ref = oracle_all(variant, inp, dht=inp["dht"], qk_l2norm=True, beta_sigmoid=True)
    compare(got, ref, label=w.name + "_act")


SEGMENTED = [
    # (variant, docs, H_qk, H_v): few wavefronts, so the walks cut documents into
    # segments; documents shorter than the segment count and empty ones included
    ("kda", (1000, 130, 0, 1, 257), 1, 1),
    ("gdn", (700, 64, 3), 1, 3),
]


@pytest.mark.parametrize("case", SEGMENTED, ids=lambda c: "%s_%s_h%d_%d" % (c[0], "-".join(map(str, c[1])), c[2], c[3]))
def test_segmented_walks(case):
    """Walks split into 2, 3 and 4 segments per document (carry and transfer
    walks, composed at the segment starts) against the oracle, and against the
    unsegmented walk: the two differ only by fp32 rounding of the composition,
    which reaches the bf16 outputs and tapes as rare last-place flips."""
    variant, docs, hqk, hv = case
    w = workloads.custom(variant, docs, hqk, hv, with_h0=True, seed=sum(docs) + 11 * hv)
    inp = workloads.make_inputs(w, device="cpu", dht=True)
    ref = oracle_all(variant, inp, dht=inp["dht"])
    base = None
    for P in (1, 2, 3, 4):
        print("[case]", w.name, "walk_segments", P, flush=True)
        got = run_gdr(variant, inp, dht=inp["dht"], walk_segments=P)
        compare(got, ref, label="%s_P%d" % (w.name, P))
        if base is None:
            base = got
            continue
        for name, x in got.items():
            r = rel_rms(x.double().numpy(), base[name].double().numpy())
            assert r <= 1e-3, "%s P=%d vs P=1: rel-RMS %.3g" % (name, P, r)


LAYOUTS = [
    # (variant, docs, H_qk, H_v, walk_segments): ragged packs, segmented and not
    ("kda", (1, 63, 64, 65, 130, 7), 2, 2, 1),
    ("kda", (1000, 130, 0, 1, 257), 1, 1, 3),
    ("gdn", (77, 64, 129), 2, 6, 1),
    ("gdn", (700, 64, 3), 1, 3, 4),
]


@pytest.mark.parametrize("case", LAYOUTS, ids=lambda c: "%s_%s_h%d_%d_P%d" % (c[0], "-".join(map(str, c[1])), c[2], c[3], c[4]))
def test_walk_layouts_agree(case):
    """The two launch layouts of the walks (one wavefront per slice; slice
    wavefronts in workgroups sharing the chain's operands through LDS) run the
    same products in the same order: every output is bitwise equal, and the
    ring layout matches the oracle."""
    import chunked_gated_delta_14_amd as gdr

    variant, docs, hqk, hv, P = case
    w = workloads.custom(variant, docs, hqk, hv, with_h0=True, seed=sum(docs) + 13 * hv)
    inp = workloads.make_inputs(w, device="cpu", dht=True)
    print("[case]", w.name, "walk layouts, segments", P, flush=True)
    slices = run_gdr(variant, inp, dht=inp["dht"], walk_segments=P, walk_layout=gdr.GDR_WALK_SLICES)
    rings = run_gdr(variant, inp, dht=inp["dht"], walk_segments=P, walk_layout=gdr.GDR_WALK_RINGS)
    for name in slices:
        assert torch.equal(slices[name], rings[name]), "%s differs between walk layouts" % name
    fwd_only = run_gdr(variant, inp, backward=False, walk_segments=P, walk_layout=gdr.GDR_WALK_RINGS)
    assert torch.equal(fwd_only["o"], rings["o"]) and torch.equal(fwd_only["ht"], rings["ht"])
    compare(rings, oracle_all(variant, inp, dht=inp["dht"]), label=w.name + "_rings")


def test_workload0_parity():
    w = workloads.workload(0)
    inp = workloads.make_inputs(w, device="cpu")
    got = run_gdr("kda", inp)
    ref = oracle_all("kda", inp)
    compare(got, ref, label=w.name)


def test_ckpt_equals_fwd_bwd_bitwise():
    w = workloads.custom("kda", (150, 90), 2, 2, with_h0=True, seed=3)
    inp = workloads.make_inputs(w, device="cpu", dht=True)
    a = run_gdr("kda", inp, dht=inp["dht"])
    b = run_gdr("kda", inp, dht=inp["dht"], ckpt=True)
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_recompute_without_output():
    """GDR_FWD_SAVE | GDR_FWD_SKIP_OUTPUT writes the same tapes as GDR_FWD_SAVE and
    leaves o untouched: the backward after it is bitwise the backward after a full
    forward."""
    import chunked_gated_delta_14_amd as gdr
    from gpu_runner import to_dev

    w = workloads.custom("kda", (170, 64, 33), 2, 2, with_h0=True, seed=8)
    inp = workloads.make_inputs(w, device="cpu", dht=True)
    a = run_gdr("kda", inp, dht=inp["dht"])
    d = to_dev(inp)
    prob = gdr.Problem(gdr.GDR_KDA, d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["h0"])
    ws = prob.alloc_workspace(gdr.GDR_FWD_SAVE)
    ws.fill_(0xFF)
    T, N = prob.T, prob.N
    sentinel = torch.full((T, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    ht = torch.empty((N, 2, 128, 128), dtype=torch.float32, device="cuda")
    gdr.kda_fwd(prob, sentinel, ht, ws, gdr.GDR_FWD_SAVE | gdr.GDR_FWD_SKIP_OUTPUT)
    gdr.kda_fwd(prob, None, None, ws, gdr.GDR_FWD_SAVE | gdr.GDR_FWD_SKIP_OUTPUT)
    g = {k: torch.full_like(a[k], float("nan"), device="cuda").to(v.dtype) for k, v in
         dict(dq=d["q"], dk=d["k"], dv=d["v"], dg=d["g"], dbeta=d["beta"], dh0=ht).items()}
    gdr.kda_bwd(prob, d["dout"], d["dht"], g["dq"], g["dk"], g["dv"], g["dg"], g["dbeta"], g["dh0"], ws)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())
    assert torch.equal(ht.cpu(), a["ht"])
    for key in g:
        assert torch.equal(g[key].float().cpu(), a[key]), key


@pytest.mark.parametrize("walk_layout", [1, 2], ids=["slices", "rings"])
def test_ckpt_graph_replay(walk_layout):
    """The checkpointed step captured in a HIP graph, with either walk layout:
    three replays, with the program's own eager work and synchronisations between
    them, each bitwise equal to the eager call."""
    import chunked_gated_delta_14_amd as gdr
    from gpu_runner import to_dev

    w = workloads.custom("kda", (150, 90), 2, 2, with_h0=True, seed=9)
    inp = workloads.make_inputs(w, device="cpu", dht=True)
    d = to_dev(inp)
    prob = gdr.Problem(gdr.GDR_KDA, d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["h0"],
                       walk_layout=walk_layout)
    ws = prob.alloc_workspace(gdr.GDR_FWD_SAVE)
    T, N = prob.T, prob.N
    bf, f32 = torch.bfloat16, torch.float32
    outs = dict(o=torch.empty((T, 2, 128), dtype=bf, device="cuda"), ht=torch.empty((N, 2, 128, 128), dtype=f32, device="cuda"),
                dq=torch.empty((T, 2, 128), dtype=bf, device="cuda"), dk=torch.empty((T, 2, 128), dtype=bf, device="cuda"),
                dv=torch.empty((T, 2, 128), dtype=bf, device="cuda"), dg=torch.empty((T, 2, 128), dtype=f32, device="cuda"),
                dbeta=torch.empty((T, 2), dtype=bf, device="cuda"), dh0=torch.empty((N, 2, 128, 128), dtype=f32, device="cuda"))

    def step():
        gdr.kda_ckpt(prob, outs["o"], outs["ht"], d["dout"], d["dht"], outs["dq"], outs["dk"], outs["dv"],
                     outs["dg"], outs["dbeta"], outs["dh0"], ws)

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():
            v.fill_(float("nan"))  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], eager[k]), (rep, k)


def test_repeat_bitwise_and_nan_workspace():
    w = workloads.custom("gdn", (100, 180), 1, 3, with_h0=True, seed=4)
    inp = workloads.make_inputs(w, device="cpu", dht=True)
    a = run_gdr("gdn", inp, dht=inp["dht"], nan_workspace=True)
    b = run_gdr("gdn", inp, dht=inp["dht"], nan_workspace=False)
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_forward_without_tapes_matches():
    w = workloads.custom("kda", (300, 45), 2, 2, with_h0=True, seed=5)
    inp = workloads.make_inputs(w, device="cpu")
    a = run_gdr("kda", inp, backward=False)
    b = run_gdr("kda", inp)
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["ht"], b["ht"])


def test_axis_aligned_keys_closed_form():
    """k_t = e_{t mod 8}: each state row is an exponential moving average
    (closed form written out here from the recurrence, not the oracle)."""
    w = workloads.custom("kda", (190, 75), 1, 1, with_h0=True, seed=6)
    inp = workloads.make_inputs(w, device="cpu")
    T = w.T
    cu = inp["cu_seqlens"].numpy()
    k = torch.zeros_like(inp["k"])
    pos = np.concatenate([np.arange(d) for d in w.docs]) % 8
    k[torch.arange(T), 0, torch.from_numpy(pos)] = 1.0
    inp["k"] = k
    got = run_gdr("kda", inp, backward=False)
    q = inp["q"][:, 0].double().numpy()
    v = inp["v"][:, 0].double().numpy()
    a = np.exp(inp["g"][:, 0].double().numpy())
    b = inp["beta"][:, 0].double().numpy()
    o = np.zeros((T, 128))
    for n in range(len(w.docs)):
        S = inp["h0"][n, 0].double().numpy().copy()
        for t in range(cu[n], cu[n + 1]):
            c = pos[t]
            S *= a[t][:, None]
            S[c] = (1 - b[t]) * S[c] + b[t] * v[t]
            o[t] = 128 ** -0.5 * q[t] @ S
    compare({"o": got["o"][:, 0]}, {"o": o}, names=["o"], label="axis-aligned keys")
