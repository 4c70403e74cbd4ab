"""Benchmark of the KDA training hot path on one MI355X.

One step = forward with tapes + backward (every kernel of the path) over the
4-document pack (42024 / 57573 / 73122 / 88673 tokens, T = 261392) at H = 16,
K = V = 128, with synthetic seeded inputs already resident in HBM.  Prints one
JSON line: whole-job throughput in token-heads/s, a roofline entry for the
dominant kernel (timed with HIP events on the stream the library launches
on), and the fp64 CPU oracle timed on a bounded sample on this host.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--H 16] [--workload 2]
"""
from __future__ import annotations

import argparse
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA fwd+bwd token-heads/s, H=16, T=261392 (1 GPU); % MFMA & HBM peak"
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16

# Per (chunk, value head) unit bytes of the workspace regions; the Kbar^T and
# (q Gamma)^T fragments are per (chunk, Q/K head) (with one gate per row they are a
# Q/K head's K^T and scale Q^T, shared by its value heads; KDA has H_qk = H_v).
SHARED_FWD = 16384                             # Kbar^T
SHARED_BWD = 16384                             # (q Gamma)^T
FWD_OPERANDS = 16384 * 2 + 16384 * 2 + 512   # -W, P fragments; U, Oi; gamma
BWD_OPERANDS = 8192                            # M^T
# the adjoint walk also reads the forward walk's -W (per unit) and Kbar^T (shared)
# fragments, for Kbar and -W^T by transposed reads, and gamma
TE_SAVED = 8192 + 5120                         # T^T (bf16 64 x 64) and E's 10 lower tiles (bf16)
S_TAPE, ROW_TAPE = 32768, 16384
# Bytes per token-head that the method must move for fwd + bwd with bf16 state
# tapes: inputs and outputs of both passes plus one 128 x 128 tape per 64 tokens.
FLOOR_BYTES_PER_TOKEN_HEAD = {"kda": 5382.0, "gdn": 2840.0}
FLUSH_BYTES = 512 << 20  # written before every timed call: larger than L2 (8 x 4 MB) and MALL (256 MB)


def method_bytes(name, T, Hqk, Hv, NC, N, gdn, save=True):
    """Algorithmic bytes of one launch: the bytes of the method's own inputs and
    outputs (no workspace intermediates) that this kernel must read or write,
    at the per-token-head figures of the path floor (q, k 256 B each per Q/K
    token-head, v, dout, o, dv 256 B, g 512 B (KDA) or 4 B (GDN), beta 2 B
    (KDA) or 4 B (GDN), one bf16 128 x 128 state tape per chunk-head, fp32
    final states).  The gradient kernel alone reads every backward input (q, k,
    v, g, beta, dout, the state tape) and writes every gradient: 3332 B per KDA
    token-head, 1637.3 B per GDN value token-head."""
    qk = 2 * T * Hqk * 256
    v = T * Hv * 256
    g = T * Hv * (4 if gdn else 512)
    beta = T * Hv * (4 if gdn else 2)
    tape = NC * Hv * 32768
    states = N * Hv * 65536
    if name == "fwd_prep":
        return qk + v + g + beta
    if name == "fwd_walk":
        return v + states + (tape if save else 0)  # o, ht (+ the tape)
    if name == "bwd_walk":
        return v  # dout
    if name == "bwd_grad":
        return (qk + v + g + beta + v + tape) + (qk + v + g + beta)
    raise KeyError(name)


def kernel_bytes(name, T, Hqk, Hv, NC, N, gdn, save=True):
    """Design bytes of one launch: every input and output byte of the kernel as
    built, workspace fragments and tapes included, counted once (q and k once
    per Q/K head).  Reported beside the algorithmic bytes, never as them."""
    units, qk_units = NC * Hv, NC * Hqk
    qk = 2 * T * Hqk * 256
    v = T * Hv * 256
    g = T * Hv * (4 if gdn else 512)
    beta = T * Hv * (4 if gdn else 2)
    fwd_ops = units * FWD_OPERANDS + qk_units * SHARED_FWD
    bwd_ops = units * BWD_OPERANDS + qk_units * SHARED_BWD
    if name == "fwd_prep":
        return qk + v + g + beta + fwd_ops + ((bwd_ops + units * TE_SAVED) if save else 0)
    if name == "fwd_walk":
        return fwd_ops + v + units * ((S_TAPE + ROW_TAPE) if save else 0) + N * Hv * 65536
    if name == "bwd_walk":
        return (bwd_ops + units * 16384 + qk_units * SHARED_FWD + units * (512 + S_TAPE + ROW_TAPE) + v
                + N * Hv * 65536)
    if name == "bwd_grad":
        return (2 * qk + 3 * v + g * 2 + beta * 2) + units * (2 * S_TAPE + 2 * ROW_TAPE + TE_SAVED)
    raise KeyError(name)


def kernel_flops(name, NC, Hv):
    """MFMA flops one launch issues (16x16x32 bf16 MFMA = 16384 flops)."""
    per_unit = {
        # E, M: 10 block pairs x 4 k-steps x 2; W, U and P, Oi: 4 strips x 8 tiles x 1.5 k-steps x 2 each
        "fwd_prep": 10 * 4 * 2 + 2 * (32 * 1.5 * 2),
        "fwd_walk": 48 * 8,   # 48 MFMAs per chunk per 16-column slice, 8 slices
        "bwd_walk": 56 * 8,
        # Y = T^T dVn 8 x (2+2+1+1); tape products 3 x 32 tiles x 4; dM, dA 2 x 10 tiles x 4;
        # gated products (hi/lo split) 12 per (row block, column tile) x 32
        "bwd_grad": 48 + 3 * 32 * 4 + 80 + 12 * 32,
    }[name]
    return per_unit * 16384 * NC * Hv


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--H", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--walk-segments", type=int, default=0,
                    help="gdr_problem.walk_segments: 0 = automatic, n = at most n segments per document walk")
    ap.add_argument("--walk-layout", type=int, default=0,
                    help="walk launch layout: 0 automatic, 1 slice wavefronts, 2 ring workgroups")
    ap.add_argument("--walk-plan", type=int, default=0,
                    help="segment plan of segmented walks: 0 balanced by document length, 1 equal")
    ap.add_argument("--input-flags", type=int, default=0,
                    help="gdr_problem.input_flags: 1 = in-kernel q/k L2 norm, 2 = beta sigmoid (logits as input)")
    ap.add_argument("--cpu-tokens", type=int, default=32768, help="tokens per document in the CPU sample")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time only the fp64 oracle on the whole workload (fwd, bwd, ckpt) on this host; no GPU")
    ap.add_argument("--no-op-timing", action="store_true", help="skip the separate fwd/bwd/ckpt timings")
    ap.add_argument("--no-smi", action="store_true", help="do not sample clock and power with amd-smi")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured MFMA and HBM peak probes")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (HBM counter calibration)")
    return ap.parse_args()


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    kernel on this workload (profiles/<kernel>_<workload>_traffic.md: FETCH_SIZE
    + WRITE_SIZE, scaled by the copy-kernel calibration), if one exists."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    w = re.search(r"traffic_workload:\s*(\S+)", text)
    if not w or w.group(1) != workload:
        return None
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def protocol_cells(ops, dev, groups=3, iters=8):
    """Per-op timing cells: one untimed call, then `groups` groups of `iters`
    calls, each after writing a 512 MB buffer (so no input is cached) and a
    device synchronisation, timed with events around the call on the stream
    the library launches on.  Cell = median of the group medians; drift =
    (last - first group median) / first; the first op is visited a second
    time at the end and its ratio to the first visit reported."""
    import torch

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def visit(fn):
        fn()
        torch.cuda.synchronize()
        meds = []
        for g in range(groups):
            ts = []
            for i in range(iters):
                flush.fill_((g * iters + i) & 0xFF)
                torch.cuda.synchronize()
                s.record()
                fn()
                e.record()
                torch.cuda.synchronize()
                ts.append(s.elapsed_time(e))
            meds.append(statistics.median(ts))
        return {"ms": statistics.median(meds), "group_medians": meds, "drift": (meds[-1] - meds[0]) / meds[0]}

    cells = {}
    for name, fn in ops:
        t0 = time.perf_counter()
        cells[name] = visit(fn)
        cells[name]["window"] = (t0, time.perf_counter())
    name0, fn0 = ops[0]
    cells[name0]["control_ratio"] = visit(fn0)["ms"] / cells[name0]["ms"]
    del flush
    return cells


class SmiSampler:
    """Samples the GPU's clock and socket power with `amd-smi metric` (run as a
    child process) from a background thread, while an untimed replay of the timed
    work runs (a query costs the work around it).  A missing or failing tool is
    recorded, never raised."""

    def __init__(self, period_s=0.25):
        import threading

        self.samples, self.error, self.period = [], None, period_s
        self.path, self.error = self.available()
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def available():
        """amd-smi is a Python script: run it with this interpreter (no shebang
        hop).  Not under a profiler: its preloaded tool library would start the
        GPU runtime in the child before that child starts the interpreter."""
        import shutil

        if any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", ""):
            return None, "not sampled under a profiler"
        path = shutil.which("amd-smi")
        return (path, None) if path else (None, "amd-smi not found")

    def _one(self):
        import subprocess

        r = subprocess.run([sys.executable, self.path, "metric", "-c", "-p", "--json"], capture_output=True,
                           text=True, timeout=20)
        g = json.loads(r.stdout)["gpu_data"][0]
        clks = [v["clk"]["value"] for k, v in g["clock"].items()
                if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        pw = g["power"]["socket_power"]["value"]
        return {"t": time.perf_counter(), "sclk_mhz": sum(clks) / len(clks) if clks else None,
                "power_w": pw if isinstance(pw, (int, float)) else None}

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._one())
            except Exception as ex:  # noqa: BLE001 - the tool is optional
                self.error = "%s: %s" % (type(ex).__name__, str(ex)[:200])
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join(timeout=30)

    def summary(self, t0=None, t1=None):
        xs = [x for x in self.samples if (t0 is None or x["t"] >= t0) and (t1 is None or x["t"] <= t1)]
        clk = [x["sclk_mhz"] for x in xs if x["sclk_mhz"] is not None]
        pw = [x["power_w"] for x in xs if x["power_w"] is not None]
        out = {"samples": len(xs)}
        if clk:
            out.update(sclk_mhz_median=statistics.median(clk), sclk_mhz_min=min(clk), sclk_mhz_max=max(clk))
        if pw:
            out.update(power_w_median=statistics.median(pw), power_w_max=max(pw))
        if self.error:
            out["error"] = self.error
        return out


def measured_peaks(dev, gib=2):
    """Rates measured on this device with the probe kernels (libgdr_probe.so): a
    pure bf16 MFMA loop (eight independent 16x16x32 chains per wavefront, two
    wavefronts per SIMD) and 16-byte grid-stride copy / read / fill kernels over
    `gib` GiB buffers; each timed with events on the current stream, best of 3."""
    import ctypes

    import torch

    from chunked_gated_delta_14_amd import _build

    if not os.path.exists(_build.PROBE_PATH):
        _build.build_probe()
    L = ctypes.CDLL(_build.PROBE_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.gdr_probe_mfma.argtypes = [vp, i32, i32, i32, vp]
    L.gdr_probe_stream.argtypes = [i32, vp, vp, vp, i64, i32, vp]
    st = vp(torch.cuda.current_stream().cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def best(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return min(out)

    blocks, iters = 2 * cus, 40000  # 4 wavefronts per block: two per SIMD
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    ms16 = best(lambda: L.gdr_probe_mfma(vp(sink.data_ptr()), blocks, iters, 0, st))
    ms32 = best(lambda: L.gdr_probe_mfma(vp(sink.data_ptr()), blocks, iters, 1, st))
    tf16 = blocks * 4 * iters * 8 * 16384 / (ms16 / 1e3) / 1e12
    tf32 = blocks * 4 * iters * 4 * 32768 / (ms32 / 1e3) / 1e12
    n = gib << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    s32 = torch.zeros(1, dtype=torch.int32, device=dev)
    rates = {}
    for mode, name, mult in ((0, "copy", 2), (1, "read", 1), (2, "write", 1)):
        ms = best(lambda: L.gdr_probe_stream(mode, vp(src.data_ptr()), vp(dst.data_ptr()), vp(s32.data_ptr()),
                                             n, 8 * cus, st))
        rates[name + "_GB_s"] = mult * n / (ms / 1e3) / 1e9
    del src, dst
    torch.cuda.synchronize()
    return dict(mfma_bf16_TFLOPs=max(tf16, tf32), mfma_16x16x32_TFLOPs=tf16, mfma_32x32x16_TFLOPs=tf32, **rates,
                note="probe kernels on this device; copy counts read + write bytes; best of 3")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, docs, tokens_per_doc):
    """The fp64 oracle (as it stands) on a bounded sample of the same pack:
    the first `tokens_per_doc` tokens of every document, all heads."""
    import numpy as np
    import torch

    import oracle

    cu = np.concatenate([[0], np.cumsum(docs)])
    take = [min(tokens_per_doc, d) for d in docs]
    idx = torch.cat([torch.arange(int(cu[i]), int(cu[i]) + take[i]) for i in range(len(docs))])
    sample = {k: inp[k].index_select(0, idx.to(inp[k].device)).cpu() for k in ("q", "k", "v", "g", "beta", "dout")}
    scu = np.concatenate([[0], np.cumsum(take)]).astype(np.int32)
    threads = oracle.default_threads()
    oracle.build()
    t0 = time.perf_counter()
    oracle.forward(sample["q"], sample["k"], sample["v"], sample["g"], sample["beta"], scu, threads=threads)
    t1 = time.perf_counter()
    oracle.backward(sample["q"], sample["k"], sample["v"], sample["g"], sample["beta"], scu, sample["dout"],
                    threads=threads)
    t2 = time.perf_counter()
    th = int(sum(take)) * int(inp["v"].shape[1])
    return {"value": th / (t2 - t0), "unit": "token-heads/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "first %d tokens of each of the %d documents, all %d heads (%d token-heads); "
                      "fwd %.2f s + bwd %.2f s" % (tokens_per_doc, len(docs), inp["v"].shape[1], th,
                                                   t1 - t0, t2 - t1)}


def cpu_full(w):
    """The fp64 oracle (as it stands) on the whole workload on this host's cores:
    one timed forward and one timed backward (which replays the forward from its
    64-token checkpoints); ckpt = 2 x forward + backward."""
    import oracle
    from chunked_gated_delta_14_amd import workloads

    t0 = time.perf_counter()
    inp = workloads.make_inputs(w, device="cpu")
    t_gen = time.perf_counter() - t0
    cu = inp["cu_seqlens"].numpy()
    threads = oracle.default_threads()
    oracle.build()
    print("[cpu-full] %s: inputs drawn in %.1f s; forward on %d threads" % (w.name, t_gen, threads),
          file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    oracle.forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cu, inp["h0"], threads=threads)
    t1 = time.perf_counter()
    print("[cpu-full] forward %.1f s; backward" % (t1 - t0), file=sys.stderr, flush=True)
    oracle.backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cu, inp["dout"], inp["h0"], threads=threads)
    t2 = time.perf_counter()
    print("[cpu-full] backward %.1f s" % (t2 - t1), file=sys.stderr, flush=True)
    th = w.T * w.H_v
    fwd_s, bwd_s = t1 - t0, t2 - t1
    return {"workload": w.name, "token_heads": th, "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
            "fwd_s": fwd_s, "bwd_s": bwd_s, "ckpt_s": 2 * fwd_s + bwd_s,
            "fwd_bwd_token_heads_per_s": th / (fwd_s + bwd_s), "input_generation_s": t_gen}


def main():
    args = parse_args()
    if args.cpu_full:
        from chunked_gated_delta_14_amd import workloads

        print(json.dumps(cpu_full(workloads.workload(args.workload, args.H))), flush=True)
        return
    if args.gpus != 1:
        print("bench.py measures a single GPU; libgdr has no multi-GPU path. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import chunked_gated_delta_14_amd as gdr
    from chunked_gated_delta_14_amd import _build, workloads

    if _build.stale():
        _build.build()
    gdr.check_device()
    dev = torch.device("cuda:0")
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = workloads.workload(args.workload, args.H)
    gdn = w.variant == "gdn"
    inp = workloads.make_inputs(w, device=dev)
    prob = gdr.Problem(gdr.GDR_GDN if gdn else gdr.GDR_KDA, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                       inp["cu_seqlens"], inp["h0"], input_flags=args.input_flags, walk_segments=args.walk_segments,
                       walk_layout=args.walk_layout, walk_plan=args.walk_plan)
    ws = prob.alloc_workspace(gdr.GDR_FWD_SAVE)
    T, Hqk, Hv, N, NC = prob.T, prob.H_qk, prob.H_v, prob.N, prob.n_chunks
    bf, f32 = torch.bfloat16, torch.float32
    o = torch.empty(T, Hv, 128, dtype=bf, device=dev)
    ht = torch.empty(N, Hv, 128, 128, dtype=f32, device=dev)
    dq = torch.empty(T, Hqk, 128, dtype=bf, device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty(T, Hv, 128, dtype=bf, device=dev)
    dg = torch.empty(tuple(inp["g"].shape), dtype=f32, device=dev)
    dbeta = torch.empty(tuple(inp["beta"].shape), dtype=inp["beta"].dtype, device=dev)
    fwd = gdr.gdn_fwd if gdn else gdr.kda_fwd
    bwd = gdr.gdn_bwd if gdn else gdr.kda_bwd
    dout = inp["dout"]

    def step():
        fwd(prob, o, ht, ws, gdr.GDR_FWD_SAVE)
        bwd(prob, dout, None, dq, dk, dv, dg, dbeta, None, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, per-kernel HIP events inside the library on the same stream.
    # No amd-smi query runs during it (each one costs the steps around it; measured
    # 0.3-1 % of the step time).
    gdr.timing_read(reset=True)
    gdr.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gdr.timing_enable(False)
    kern = gdr.timing_read(reset=True)
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # clock and socket power: sampled over an untimed replay of the same steps right
    # after the timed region (at least 1.5 s of them, so that several samples land)
    smi = SmiSampler()
    if args.no_smi:
        smi.path, smi.error = None, "disabled (--no-smi)"
    smi.__enter__()
    smi_t0 = time.perf_counter()
    if smi.path:
        while time.perf_counter() - smi_t0 < 1.5:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
    smi_t1 = time.perf_counter()
    smi.__exit__()

    # per-op cells (events on torch's current stream = the library's stream); the
    # backward reuses the tapes of one untimed forward with GDR_FWD_SAVE
    ops = {}
    if not args.no_op_timing:
        ckpt = gdr.gdn_ckpt if gdn else gdr.kda_ckpt
        fwd(prob, o, ht, ws, gdr.GDR_FWD_SAVE)
        ops = protocol_cells([
            ("fwd", lambda: fwd(prob, o, ht, ws, 0)),
            ("fwd_save", lambda: fwd(prob, o, ht, ws, gdr.GDR_FWD_SAVE)),
            ("bwd", lambda: bwd(prob, dout, None, dq, dk, dv, dg, dbeta, None, ws)),
            ("ckpt", lambda: ckpt(prob, o, ht, dout, None, dq, dk, dv, dg, dbeta, None, ws)),
        ], dev)

    for c in ops.values():
        c.pop("window")

    kernels = {}
    total_flops = 0.0
    for name, (ms, n) in kern.items():
        if n == 0:
            continue
        avg = ms / n
        b = method_bytes(name, T, Hqk, Hv, NC, N, gdn)
        db = kernel_bytes(name, T, Hqk, Hv, NC, N, gdn)
        fl = kernel_flops(name, NC, Hv)
        total_flops += fl * n / args.steps
        kernels[name] = {"avg_ms": avg, "launches": n, "bytes": b, "GB_s": b / avg / 1e6,
                         "hbm_frac": b / avg / 1e6 / HBM_PEAK_GBS, "design_bytes": db,
                         "design_GB_s": db / avg / 1e6, "mfma_TFLOPs": fl / avg / 1e9,
                         "mfma_frac": fl / avg / 1e9 / MFMA_BF16_PEAK_TFLOPS}
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches"])
    # dependent steps of the walks: chunks of the longest document (unsegmented
    # walks: 8 N H_v >= 512 wavefronts, or one chunk per document at most)
    longest = max((d + 63) // 64 for d in w.docs)
    unsegmented = args.walk_segments == 1 or 8 * N * Hv >= 512 or NC <= N
    walk_us = {k: kernels[k]["avg_ms"] * 1e3 / longest for k in ("fwd_walk", "bwd_walk")
               if k in kernels and unsegmented}
    floor_ms = T * Hv * FLOOR_BYTES_PER_TOKEN_HEAD[w.variant] / (HBM_PEAK_GBS * 1e6)
    dk_ = kernels[dom]
    traffic = traffic_from_profiles(dom, w.name)
    token_heads = T * Hv
    result = {
        "metric": METRIC,
        "value": token_heads / (ms_per_step / 1e3),
        "unit": "token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "variant": w.variant, "T": T, "docs": list(w.docs), "H_qk": Hqk,
                   "H_v": Hv, "K": 128, "V": 128, "n_chunks": NC, "input_flags": args.input_flags,
                   "walk_segments": args.walk_segments, "walk_layout": args.walk_layout,
                   "walk_plan": "equal" if args.walk_plan else "balanced",
                   "walk_layout_run": "rings" if gdr.walk_layout_chosen(gdr.GDR_GDN if gdn else gdr.GDR_KDA, prob)
                   == gdr.GDR_WALK_RINGS else "slices",
                   "step": "forward with tapes + backward (prep, walk, adjoint walk, gradients)"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": dk_["GB_s"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": dk_["GB_s"] / HBM_PEAK_GBS, "traffic": traffic,
                     "bytes_per_launch": dk_["bytes"], "avg_launch_ms": dk_["avg_ms"],
                     "traffic_over_algorithmic": traffic / dk_["bytes"] if traffic else None,
                     "design_bytes_per_launch": dk_["design_bytes"], "design_GB_s": dk_["design_GB_s"],
                     "note": "achieved = the method's bytes for this kernel (bytes_per_launch) / avg_launch_ms; "
                             "design bytes add the workspace fragments and tapes the kernels pass each other"},
        "ms": {k: v["ms"] for k, v in ops.items()},
        "cells": ops,
        "path_floor": {"ms": floor_ms, "frac": floor_ms / ms_per_step,
                       "bytes_per_token_head": FLOOR_BYTES_PER_TOKEN_HEAD[w.variant]},
        "us_per_walk_step": walk_us,
        "smi": dict(smi.summary(smi_t0, smi_t1), note="amd-smi metric: mean gfx clock over the XCDs, socket "
                    "power; sampled over an untimed replay of the timed steps right after them (no query runs "
                    "during the timed steps or the per-op cells)"),
        "longest_chain_chunks": longest,
        "mfma": {"TFLOPs": total_flops / (ms_per_step / 1e3) / 1e12,
                 "frac": total_flops / (ms_per_step / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "kernels": kernels,
    }
    if not args.no_peaks:
        peaks = measured_peaks(dev)
        result["measured_peaks"] = peaks
        result["roofline"]["measured_copy_GB_s"] = peaks["copy_GB_s"]
        result["roofline"]["frac_of_measured_copy"] = dk_["GB_s"] / peaks["copy_GB_s"]
        result["mfma"]["frac_of_measured"] = result["mfma"]["TFLOPs"] / peaks["mfma_bf16_TFLOPs"]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, list(w.docs), args.cpu_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
