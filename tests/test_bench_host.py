"""bench.py's host-side contract (no GPU needed): one GPU only, and the byte and
flop accounting it reports against the rooflines."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "single GPU" in res.stderr


def test_kernel_bytes_per_unit():
    """Per (chunk, head) unit of the KDA pack at H = 16 (full chunks dominate): the
    prep, walk and gradient byte counts of the design."""
    T, H, NC, N = 261392, 16, 4086, 4
    units = NC * H
    prep = bench.kernel_bytes("fwd_prep", T, H, H, NC, N, gdn=False)
    # inputs q, k, v, g, beta per token-head, then the walk operands and saved tapes per unit
    assert prep == 2 * T * H * 256 + T * H * 256 + T * H * 512 + T * H * 2 + units * (
        bench.FWD_OPERANDS + bench.BWD_OPERANDS + bench.TE_SAVED + bench.SHARED_FWD + bench.SHARED_BWD)
    # GDN: the K fragments once per (chunk, Q/K head), for 3 value heads each
    Hqk, Hv = 16, 48
    gprep = bench.kernel_bytes("fwd_prep", T, Hqk, Hv, NC, N, gdn=True)
    kda_like = bench.kernel_bytes("fwd_prep", T, Hv, Hv, NC, N, gdn=True)
    assert kda_like - gprep == 2 * T * (Hv - Hqk) * 256 + NC * (Hv - Hqk) * (bench.SHARED_FWD + bench.SHARED_BWD)
    grad = bench.kernel_bytes("bwd_grad", T, H, H, NC, N, gdn=False)
    per_unit = grad / units
    assert 280e3 < per_unit < 300e3  # ~173 KB + q, k read, ~80 KB written per full chunk
    with pytest.raises(KeyError):
        bench.kernel_bytes("nope", T, H, H, NC, N, gdn=False)


def test_method_bytes_match_the_path_floor():
    """The gradient kernel's algorithmic bytes are the backward's figure of the
    path floor (3332 B per KDA token-head, 1637.3 B per GDN value token-head)
    with exactly full chunks; the four kernels' method bytes add up to the
    fwd + bwd floor plus the dout read twice (adjoint walk and gradients) and
    the final states."""
    for gdn, H_qk, H_v, per_th in ((False, 16, 16, 3332.0), (True, 16, 48, 1637.0 + 1 / 3)):
        T, N = 64 * 1000, 4
        NC = T // 64
        b = bench.method_bytes("bwd_grad", T, H_qk, H_v, NC, N, gdn)
        assert abs(b / (T * H_v) - per_th) < 1e-9
        total = sum(bench.method_bytes(k, T, H_qk, H_v, NC, N, gdn)
                    for k in ("fwd_prep", "fwd_walk", "bwd_walk", "bwd_grad"))
        floor = bench.FLOOR_BYTES_PER_TOKEN_HEAD["gdn" if gdn else "kda"]
        extra = T * H_v * 256 + N * H_v * 65536
        assert abs((total - extra) / (T * H_v) - floor) < 0.5


def test_traffic_summary_matches_workload_only():
    """A committed HBM-traffic summary is reported only for the workload it names."""
    t = bench.traffic_from_profiles("bwd_grad", "kda_pack4_T261392_H16")
    assert t is not None and t > 1e10
    g = bench.traffic_from_profiles("bwd_grad", "gdn_pack6_T241817_Hqk16_Hv48")
    assert g is not None and g != t
    assert bench.traffic_from_profiles("bwd_grad", "kda_pack4_T261392_H4") is None
    assert bench.traffic_from_profiles("no_such_kernel", "kda_pack4_T261392_H16") is None
