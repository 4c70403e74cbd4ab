"""gdr_kda_ckpt_noalloc: the checkpointed KDA step on the library's static
per-device workspace, through the C ABI, against gdr_kda_ckpt with a workspace
of the caller's (bitwise: the same kernels on the same inputs)."""
import pytest
import torch

from chunked_gated_delta_14_amd import workloads
from gpu_runner import to_dev

pytestmark = pytest.mark.gpu


def _outputs(prob, hv, hqk, d):
    T, N = prob.T, prob.N
    bf, f32 = torch.bfloat16, torch.float32
    nan = float("nan")
    return dict(
        o=torch.full((T, hv, 128), nan, dtype=bf, device="cuda"),
        ht=torch.full((N, hv, 128, 128), nan, dtype=f32, device="cuda"),
        dq=torch.full((T, hqk, 128), nan, dtype=bf, device="cuda"),
        dk=torch.full((T, hqk, 128), nan, dtype=bf, device="cuda"),
        dv=torch.full((T, hv, 128), nan, dtype=bf, device="cuda"),
        dg=torch.full(tuple(d["g"].shape), nan, dtype=f32, device="cuda"),
        dbeta=torch.full(tuple(d["beta"].shape), nan, dtype=d["beta"].dtype, device="cuda"),
        dh0=torch.full((N, hv, 128, 128), nan, dtype=f32, device="cuda"),
    )


def _call(fn, prob, d, outs, *ws):
    fn(prob, outs["o"], outs["ht"], d["dout"], d["dht"], outs["dq"], outs["dk"], outs["dv"], outs["dg"],
       outs["dbeta"], outs["dh0"], *ws)


def test_noalloc_ckpt_matches_ckpt():
    """Two calls in a row, the second on a smaller pack, each bitwise equal to
    gdr_kda_ckpt.  The first call may load the library's array on the device;
    device free memory is the same before and after the second."""
    import chunked_gated_delta_14_amd as gdr

    cases = [((300, 129, 77, 1), 4), ((150, 64), 2)]
    problems = []
    for docs, H in cases:
        w = workloads.custom("kda", docs, H, H, with_h0=True, seed=40 + H)
        inp = workloads.make_inputs(w, device="cpu", dht=True)
        d = to_dev(inp)
        prob = gdr.Problem(gdr.GDR_KDA, d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["h0"])
        assert prob.workspace_bytes(gdr.GDR_FWD_SAVE) <= gdr.GDR_NOALLOC_SCRATCH_BYTES
        ws = prob.alloc_workspace(gdr.GDR_FWD_SAVE)
        ws.fill_(0xFF)
        ref = _outputs(prob, H, H, d)
        _call(gdr.kda_ckpt, prob, d, ref, ws)
        problems.append((w, prob, d, ref, _outputs(prob, H, H, d)))
    torch.cuda.synchronize()
    free = []
    for w, prob, d, ref, got in problems:
        print("[case] no-alloc ckpt", w.name, "H", prob.H_v, flush=True)
        free.append(torch.cuda.mem_get_info()[0])
        _call(gdr.kda_ckpt_noalloc, prob, d, got)
        torch.cuda.synchronize()
        for key in ref:
            assert torch.equal(got[key], ref[key]), "%s: %s differs from gdr_kda_ckpt" % (w.name, key)
    free.append(torch.cuda.mem_get_info()[0])
    assert free[2] == free[1], "the second call changed device free memory by %d bytes" % (free[1] - free[2])


def test_noalloc_rejects_problems_beyond_the_scratch():
    """A problem whose workspace exceeds the static array is refused on the host,
    with GDR_ERR_WORKSPACE, and nothing is written."""
    import chunked_gated_delta_14_amd as gdr

    T, H = 64 * 400, 1  # 400 chunk-heads: more than 64 MiB of workspace
    bf = torch.bfloat16
    q = torch.zeros((T, H, 128), dtype=bf, device="cuda")
    g = torch.zeros((T, H, 128), dtype=torch.float32, device="cuda")
    beta = torch.zeros((T, H), dtype=bf, device="cuda")
    prob = gdr.Problem(gdr.GDR_KDA, q, q, q, g, beta, [0, T])
    assert prob.workspace_bytes(gdr.GDR_FWD_SAVE) > gdr.GDR_NOALLOC_SCRATCH_BYTES
    d = {"g": g, "beta": beta, "dout": q, "dht": None}
    outs = _outputs(prob, H, H, d)
    with pytest.raises(gdr.GdrError) as err:
        _call(gdr.kda_ckpt_noalloc, prob, d, outs)
    assert err.value.status == 3 and "static scratch" in str(err.value)
    torch.cuda.synchronize()
    assert bool(torch.isnan(outs["o"].float()).all())
