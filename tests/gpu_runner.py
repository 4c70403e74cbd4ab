"""Runs libgdr through its C ABI on cuda:0 and compares with the fp64 oracle."""
import numpy as np

import oracle
from helpers import max_abs, rel_rms

# Tolerances of the target statement: o, dq, dk, dv: rel-RMS <= 1e-2 and
# max-abs <= 5e-2; dg, dbeta: rel-RMS <= 2e-2.  States (ht, dh0) are held to
# rel-RMS <= 1e-2 as well.
TOL = {
    "o": (1e-2, 5e-2), "dq": (1e-2, 5e-2), "dk": (1e-2, 5e-2), "dv": (1e-2, 5e-2),
    "dg": (2e-2, None), "dbeta": (2e-2, None), "ht": (1e-2, None), "dh0": (1e-2, None),
}


def to_dev(inp, device="cuda"):
    import torch

    return {k: (v.to(device) if (torch.is_tensor(v) and k != "cu_seqlens") else v) for k, v in inp.items()}


def run_gdr(variant, inp, *, backward=True, dht=None, ckpt=False, ws_fill=0xFF, workspace=None,
            on_device=False, input_flags=0, walk_segments=0, walk_layout=0, walk_plan=0):
    """Forward (with tapes) and backward on the GPU.  Returns CPU fp32 tensors
    (or the device tensors as computed, with on_device=True).

    ws_fill: byte written over the whole workspace first (0xFF: NaN in bf16 and
    fp32; 0x00: zeros; None: left as it is)."""
    import torch

    import chunked_gated_delta_14_amd as gdr

    d = to_dev(inp)
    code = gdr.GDR_KDA if variant == "kda" else gdr.GDR_GDN
    prob = gdr.Problem(code, d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d.get("h0"),
                       input_flags=input_flags, walk_segments=walk_segments, walk_layout=walk_layout,
                       walk_plan=walk_plan)
    T, Hqk, Hv, N = prob.T, prob.H_qk, prob.H_v, prob.N
    ws = workspace if workspace is not None else prob.alloc_workspace(gdr.GDR_FWD_SAVE)
    if ws_fill is not None:
        ws.fill_(ws_fill)
    dev = d["q"].device
    bf, f32 = torch.bfloat16, torch.float32
    o = torch.full((T, Hv, 128), float("nan"), dtype=bf, device=dev)
    ht = torch.full((N, Hv, 128, 128), float("nan"), dtype=f32, device=dev)
    out = {}
    dtd = dht.to(dev) if dht is not None else None
    if backward:
        dq = torch.full((T, Hqk, 128), float("nan"), dtype=bf, device=dev)
        dk = torch.full_like(dq, float("nan"))
        dv = torch.full((T, Hv, 128), float("nan"), dtype=bf, device=dev)
        dg = torch.full(tuple(d["g"].shape), float("nan"), dtype=f32, device=dev)
        dbeta = torch.full(tuple(d["beta"].shape), float("nan"), dtype=d["beta"].dtype, device=dev)
        dh0 = torch.full((N, Hv, 128, 128), float("nan"), dtype=f32, device=dev)
        if ckpt:
            fn = gdr.kda_ckpt if variant == "kda" else gdr.gdn_ckpt
            fn(prob, o, ht, d["dout"], dtd, dq, dk, dv, dg, dbeta, dh0, ws)
        else:
            (gdr.kda_fwd if variant == "kda" else gdr.gdn_fwd)(prob, o, ht, ws, gdr.GDR_FWD_SAVE)
            (gdr.kda_bwd if variant == "kda" else gdr.gdn_bwd)(prob, d["dout"], dtd, dq, dk, dv, dg, dbeta, dh0, ws)
        out.update(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dh0=dh0)
    else:
        (gdr.kda_fwd if variant == "kda" else gdr.gdn_fwd)(prob, o, ht, ws, 0)
    torch.cuda.synchronize()
    out.update(o=o, ht=ht)
    if on_device:
        return out
    return {k: v.float().cpu() for k, v in out.items()}


def oracle_all(variant, inp, dht=None, backward=True, threads=None, qk_l2norm=False, beta_sigmoid=False):
    act = dict(qk_l2norm=qk_l2norm, beta_sigmoid=beta_sigmoid)
    o, ht = oracle.forward_act(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"].numpy(),
                               inp.get("h0"), threads=threads, **act)
    ref = {"o": o, "ht": ht}
    if backward:
        ref.update(oracle.backward_act(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                       inp["cu_seqlens"].numpy(), inp["dout"], inp.get("h0"), dht, threads=threads,
                                       **act))
    return ref


def compare(got, ref, names=None, label=""):
    """Check every tensor against TOL; return the metrics (printed for the log)."""
    names = names or [n for n in TOL if n in ref and n in got]
    report = {}
    failures = []
    for n in names:
        x = got[n].numpy() if hasattr(got[n], "numpy") else got[n]
        r = ref[n]
        assert np.all(np.isfinite(x)), "%s %s has non-finite values" % (label, n)
        rr, ma = rel_rms(x, r), max_abs(x, r)
        report[n] = (rr, ma)
        lim_rr, lim_ma = TOL[n]
        if rr > lim_rr or (lim_ma is not None and ma > lim_ma):
            failures.append("%s: rel_rms=%.3e max_abs=%.3e" % (n, rr, ma))
    print("[parity] %s %s" % (label, " ".join("%s=%.2e/%.2e" % (k, v[0], v[1]) for k, v in report.items())),
          flush=True)
    assert not failures, "%s: %s" % (label, "; ".join(failures))
    return report
