"""Host-side tests of libgdr: library load and exports, chunk planner, workspace
sizer and argument validation.  No GPU work is launched here: every error
path is rejected on the host before anything is enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest

import chunked_gated_delta_14_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "gdr.h")).read()
    return sorted(set(re.findall(r"\b(gdr_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert set(names) == set(gdr.EXPORTED_SYMBOLS)
    L = gdr.lib()
    for n in names:
        assert hasattr(L, n), n
    # and they are real dynamic symbols of the shared object
    raw = ctypes.CDLL(gdr._build.LIB_PATH)
    for n in names:
        getattr(raw, n)


def test_status_strings():
    for s in range(6):
        assert gdr.status_string(s)
    assert gdr.status_string(99) == "unknown status"


def _unpack(table, nc, N):
    start, ln, doc = table[:nc], table[nc:2 * nc], table[2 * nc:3 * nc]
    ptr = table[3 * nc:3 * nc + N + 1]
    order = table[3 * nc + N + 1:3 * nc + 2 * N + 1]
    return start, ln, doc, ptr, order


@pytest.mark.parametrize("docs", [[200, 312], [1, 63, 64, 65, 0, 128, 129], [0], [0, 0, 5], [88673, 42024, 73122, 57573]])
def test_plan_chunks(docs):
    cu = np.concatenate([[0], np.cumsum(docs)]).astype(np.int32)
    table, nc = gdr.plan_chunks(cu)
    N = len(docs)
    assert nc == sum((d + 63) // 64 for d in docs)
    assert len(table) == 3 * nc + 2 * N + 1
    start, ln, doc, ptr, order = _unpack(table, nc, N)
    # chunks tile every document exactly, never straddling a boundary
    covered = np.zeros(cu[-1], dtype=int)
    for c in range(nc):
        d = doc[c]
        assert cu[d] <= start[c] and start[c] + ln[c] <= cu[d + 1]
        assert 1 <= ln[c] <= 64
        covered[start[c]:start[c] + ln[c]] += 1
    assert np.all(covered == 1)
    for n in range(N):
        assert ptr[n + 1] - ptr[n] == (docs[n] + 63) // 64
        for c in range(ptr[n], ptr[n + 1]):
            assert doc[c] == n and start[c] == cu[n] + 64 * (c - ptr[n])
    assert sorted(order.tolist()) == list(range(N))
    counts = [ptr[o + 1] - ptr[o] for o in order]
    assert counts == sorted(counts, reverse=True)


def test_plan_chunks_rejects_bad_cu():
    for cu in ([1, 5], [0, 5, 3]):
        with pytest.raises(gdr.GdrError):
            gdr.plan_chunks(np.array(cu, dtype=np.int32))


def test_workspace_bytes_monotone_and_aligned():
    prev = 0
    for nc in (1, 2, 9, 100, 4086):
        for flags in (0, gdr.GDR_FWD_SAVE):
            b = gdr.workspace_bytes(gdr.GDR_KDA, 64 * nc, 1, nc, 4, 4, 128, 128, flags)
            assert b % 256 == 0 and b > 0
        full = gdr.workspace_bytes(gdr.GDR_KDA, 64 * nc, 1, nc, 4, 4, 128, 128, gdr.GDR_FWD_SAVE)
        fwd = gdr.workspace_bytes(gdr.GDR_KDA, 64 * nc, 1, nc, 4, 4, 128, 128, 0)
        assert full > fwd and full > prev
        prev = full
    # GDN sizes by value heads, except what a Q/K head's value heads share: the q/k
    # inverse norms (one pair per (token, Q/K head)) and the walks' K^T and scale Q^T
    # fragments (16 KB each per (chunk, Q/K head); the adjoint walk reads K out of K^T)
    a = gdr.workspace_bytes(gdr.GDR_GDN, 640, 1, 10, 16, 48, 128, 128, 1)
    b = gdr.workspace_bytes(gdr.GDR_KDA, 640, 1, 10, 48, 48, 128, 128, 1)
    assert b - a == 640 * (48 - 16) * 2 * 4 + 2 * 16384 * 10 * (48 - 16)
    # forward only: the shared K^T fragments
    assert gdr.workspace_bytes(gdr.GDR_KDA, 640, 1, 10, 48, 48, 128, 128, 0) - \
        gdr.workspace_bytes(gdr.GDR_GDN, 640, 1, 10, 16, 48, 128, 128, 0) == 16384 * 10 * (48 - 16)
    assert gdr.workspace_bytes(gdr.GDR_KDA, 0, 1, 0, 1, 1, 128, 128, 1) == 0


@pytest.mark.parametrize("args,code", [
    ((gdr.GDR_KDA, 64, 1, 1, 1, 1, 64, 128, 0), 2),      # K != 128
    ((gdr.GDR_KDA, 64, 1, 1, 1, 2, 128, 128, 0), 2),     # KDA needs H_qk == H_v
    ((gdr.GDR_GDN, 64, 1, 1, 2, 3, 128, 128, 0), 2),     # GDN needs H_v % H_qk == 0
    ((gdr.GDR_KDA, 64, 1, 3, 1, 1, 128, 128, 0), 1),     # more chunks than possible
    ((gdr.GDR_KDA, 130, 1, 2, 1, 1, 128, 128, 0), 1),    # too few chunks for T
    ((gdr.GDR_KDA, -1, 1, 0, 1, 1, 128, 128, 0), 1),
    ((gdr.GDR_KDA, 64, 1, 1, 1, 1, 128, 128, 4), 1),     # unknown flag
    ((7, 64, 1, 1, 1, 1, 128, 128, 0), 1),               # unknown variant
])
def test_workspace_bytes_errors(args, code):
    with pytest.raises(gdr.GdrError) as e:
        gdr.workspace_bytes(*args)
    assert e.value.status == code


class _FakeTensor:
    def __init__(self, addr, n=1, esize=1):
        self.addr, self.n, self.esize = addr, n, esize

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n

    def element_size(self):
        return self.esize


def _cproblem(T=128, N=1, Hqk=1, Hv=1, K=128, V=128, nc=2, null=()):
    f = {k: (0 if k in null else 4096) for k in ("q", "k", "v", "g", "beta", "cu", "table")}
    return gdr._CProblem(T, N, Hqk, Hv, K, V, f["q"], f["k"], f["v"], f["g"], f["beta"], f["cu"], f["table"],
                         nc, None, 128 ** -0.5)


@pytest.mark.parametrize("kw,code", [
    (dict(null=("q",)), 1),
    (dict(null=("table",)), 1),
    (dict(K=64), 2),
    (dict(Hqk=1, Hv=2), 2),
    (dict(nc=5), 1),
])
def test_forward_validation_happens_on_host(kw, code):
    """Invalid problems are rejected before any device call (so this runs without a GPU)."""
    L = gdr.lib()
    p = _cproblem(**kw)
    rc = L.gdr_kda_fwd(ctypes.byref(p), ctypes.c_void_p(4096), None, ctypes.c_void_p(4096), 1 << 40, 0, None)
    assert rc == code
    assert L.gdr_last_error().decode()


def test_workspace_checks():
    L = gdr.lib()
    p = _cproblem()
    need = gdr.workspace_bytes(gdr.GDR_KDA, 128, 1, 2, 1, 1, 128, 128, 0)
    rc = L.gdr_kda_fwd(ctypes.byref(p), ctypes.c_void_p(4096), None, ctypes.c_void_p(4096), need - 256, 0, None)
    assert rc == 3
    rc = L.gdr_kda_fwd(ctypes.byref(p), ctypes.c_void_p(4096), None, ctypes.c_void_p(4096 + 16), need, 0, None)
    assert rc == 3
    # the backward needs the full (tape-keeping) workspace
    full = gdr.workspace_bytes(gdr.GDR_KDA, 128, 1, 2, 1, 1, 128, 128, 1)
    rc = L.gdr_kda_bwd(ctypes.byref(p), *([ctypes.c_void_p(4096)] * 8), ctypes.c_void_p(4096), full - 256, None)
    assert rc == 3
    rc = L.gdr_kda_fwd(ctypes.byref(p), ctypes.c_void_p(4096), None, ctypes.c_void_p(4096), 1 << 40, 4, None)
    assert rc == 1


def test_unknown_input_flag_rejected_on_host():
    L = gdr.lib()
    p = _cproblem()
    p.input_flags = 4
    rc = L.gdr_kda_fwd(ctypes.byref(p), ctypes.c_void_p(4096), None, ctypes.c_void_p(4096), 1 << 40, 0, None)
    assert rc == 1 and "input flag" in L.gdr_last_error().decode()


def test_walk_layout_fields_checked_on_host():
    """walk_layout must name a layout and max_doc_chunks lie in [0, n_chunks]."""
    L = gdr.lib()
    for field, value, msg in (("walk_layout", 3, "walk_layout"), ("walk_layout", -1, "walk_layout"),
                              ("max_doc_chunks", -1, "max_doc_chunks"), ("max_doc_chunks", 3, "max_doc_chunks")):
        p = _cproblem()
        setattr(p, field, value)
        rc = L.gdr_kda_fwd(ctypes.byref(p), ctypes.c_void_p(4096), None, ctypes.c_void_p(4096), 1 << 40, 0, None)
        assert rc == 1 and msg in L.gdr_last_error().decode()


@pytest.mark.parametrize("docs", [[200, 312], [0, 5, 0], [88673, 42024, 73122, 57573]])
def test_max_doc_chunks_from_table(docs):
    cu = np.concatenate([[0], np.cumsum(docs)]).astype(np.int32)
    table, nc = gdr.plan_chunks(cu)
    assert gdr.max_doc_chunks(table, len(docs), nc) == max(-(-d // 64) for d in docs)


@pytest.mark.parametrize("index,H,expected", [
    (2, 16, "slices"),  # four long chains per head: the chain step decides
    (2, 64, "rings"),   # 256 chains: the work per compute unit decides
    (2, 4, "slices"),   # segmented walks keep the slices
    (1, 16, "slices"),  # one 511-chunk document, four segments
    (3, None, "rings"),  # GDN, 288 chains
])
def test_walk_layout_policy(index, H, expected):
    """The automatic walk layout at each workload's shape, on a 256-CU device
    (host only: no device call), and the forced layouts."""
    from chunked_gated_delta_14_amd import workloads

    w = workloads.workload(index, H)
    cu = np.concatenate([[0], np.cumsum(w.docs)]).astype(np.int32)
    table, nc = gdr.plan_chunks(cu)
    p = _cproblem(T=w.T, N=len(w.docs), Hqk=w.H_qk, Hv=w.H_v, nc=nc)
    p.max_doc_chunks = gdr.max_doc_chunks(table, len(w.docs), nc)
    code = gdr.GDR_KDA if w.variant == "kda" else gdr.GDR_GDN
    want = gdr.GDR_WALK_RINGS if expected == "rings" else gdr.GDR_WALK_SLICES
    assert gdr.walk_layout_chosen(code, p, 256) == want
    for forced in (gdr.GDR_WALK_SLICES, gdr.GDR_WALK_RINGS):
        p.walk_layout = forced
        assert gdr.walk_layout_chosen(code, p, 256) == forced
    with pytest.raises(gdr.GdrError):
        gdr.walk_layout_chosen(code, p, -1)


def test_skip_output_flag_host_checks():
    """GDR_FWD_SKIP_OUTPUT is a known flag (workspace sizes as without it); o may be
    NULL only with it.  Only paths that stop before any device call are exercised."""
    L = gdr.lib()
    p = _cproblem()
    for flags in (0, 1):
        assert gdr.workspace_bytes(gdr.GDR_KDA, 128, 1, 2, 1, 1, 128, 128, flags | gdr.GDR_FWD_SKIP_OUTPUT) == \
            gdr.workspace_bytes(gdr.GDR_KDA, 128, 1, 2, 1, 1, 128, 128, flags)
    with pytest.raises(gdr.GdrError):
        gdr.workspace_bytes(gdr.GDR_KDA, 128, 1, 2, 1, 1, 128, 128, 4)
    rc = L.gdr_kda_fwd(ctypes.byref(p), None, None, ctypes.c_void_p(4096), 1 << 40, gdr.GDR_FWD_SAVE, None)
    assert rc == 1 and "o" in L.gdr_last_error().decode()


def test_no_cpu_fallback_without_library(monkeypatch, tmp_path):
    """The binding raises when the HIP library is absent instead of computing on the CPU."""
    monkeypatch.setattr(gdr._build, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(gdr, "_lib", None)
    with pytest.raises(RuntimeError):
        gdr.lib()
