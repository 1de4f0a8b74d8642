#!/usr/bin/env python3
"""Benchmark: gated delta-net forward + backward tokens/s on one MI355X.

Headline workload: 4 sequences x 4096 tokens, 16 key heads shared by 48 value heads, head
size 128, q/k/v as bf16 row views of one packed [16384, 10240] projection, float32 gates and
state, chunk 64, S0 = 0, dS_T ~ N(0, 0.1^2) (the 27B-layer training shape; seeded synthetic
inputs from synth.config_case(3)). One step = gdn_fwd (saving chunk states) + gdn_bwd over
the whole batch, inputs resident in HBM before timing.

Protocol: W untimed warmup steps, then exactly K timed steps, each bracketed by HIP events on
the launch stream, with a 512 MiB scratch write between steps (outside the events) so that
no step finds the previous one's data in the 256 MB Infinity Cache or the L2s; ``ms_per_step``
is the median step. The headline steps are replays of the step captured once in a HIP graph
(the same kernels on the same buffers, fewer launch gaps); the eager step, timed the same way
with the library's per-kernel events on, is reported beside it and gives the kernel times. The same protocol times the extra lines: the forward alone (saving and
forward-only), the strided v_repeat 3 workload (one sequence of 2048 tokens, S0 and dS0) and
the varlen workload (8 sequences of U[256, 8192] tokens, S0 and dS0), the step with the q/k
L2 norm and gate chain fused, a decode step and the causal conv1d + SiLU.

Prints one JSON line. ``roofline`` covers the kernel with the largest share of the step:
``achieved`` is the method's own bytes that kernel reads and writes (the caller's tensors:
q, k, v, g, beta, dO, o, dq, dk, dv, dg, dbeta and the state tensors; never the saved chunk
factors, which are ``design_bytes``) per launch, over its average launch time from HIP
events the library records around each launch on the launch stream. ``traffic`` is the
measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, each scaled by what the
counter reads for a plain copy of known size) from the committed counter summary, or null
when the kernel sources changed since. ``mfma_busy`` comes from the committed
SQ_VALU_MFMA_BUSY_CYCLES summary under the same rule. ``cpu_baseline`` times the float64
oracle on the host cores (all the process may use) on the whole batch, and on one core on a
bounded sample of the strided workload.

Counter runs: ``--profile-step`` runs only the plain training step (for rocprofv3);
``--pmc-calib`` first copies a buffer of known size; ``--summarize-counters OUT DIR...``
turns rocprofv3 counter result directories into a committed summary.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN fwd+bwd tokens/s @Hk16/Hv48/D128 T=4096; % MFMA / HBM roofline"
PEAK = {"f32_mfma": 157.3e12, "bf16_mfma": 2.5e15, "hbm": 8.0e12}
N_CU, SIMD_PER_CU = 256, 4
WORKLOAD_TAG = "B4_T4096_Hk16_Hv48_D128_bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", f"gdn_kernels_{WORKLOAD_TAG}_hbm_traffic.md")
MFMA_FILE = os.path.join(ROOT, "profiles", f"gdn_kernels_{WORKLOAD_TAG}_mfma_counters.md")
CALIB_BYTES = 3 << 27  # the calibration copy reads and writes 384 MiB
FLUSH_BYTES = 512 << 20


def source_hash():
    """Hash of the HIP sources and headers: counter summaries are valid for this code only."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_34_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- models
def kernel_model(name, C, D, Hk, Hv, T, n_chunks, N, es=2, S0=False, dST=True):
    """Per launch of a kernel: the MFMA flops of the products it forms, the method's own bytes
    it moves (the caller's tensors it reads or writes, each once) and the design bytes (the
    saved chunk factors it reads or writes, and re-reads of q, k by the value heads that share
    a key head beyond the first). Units: ch (chunk, value head) and ck (chunk, key head)."""
    ch, ck, r = n_chunks * Hv, n_chunks * Hk, Hv // Hk
    cd, dd = C * D * es, D * D * es
    cc = 128 * (C // 16) * (C // 16 + 1) * es  # T or M: the blocks on and below the diagonal
    qk, vv, gates = 2 * Hk * D * es, Hv * D * es, 2 * Hv * 4  # per token
    dqk, dgb = 2 * Hk * D * es, 2 * Hv * 4
    state = N * Hv * D * D * 4
    rec_sweep, rec_grad = 4 * C * 4, 2 * C * 4  # gate-record rows the sweeps / grad kernel read
    step_flops = 6 * C * D * D + 4 * C * C * D
    m = {
        "k_table": (0, 0, 0),
        # K K^T, Q K^T per key head; T, M and the gate record (5 rows) written per value head.
        "k_prep": (ck * 4 * C * C * D, T * (qk + gates), ch * (2 * cc + 5 * C * 4)),
        # K S, T X, Q S, M Delta, K^T (e o Delta); reads T, M, gates; saves S_c and Delta.
        "k_fwd_sweep": (ch * step_flops, T * (qk + 2 * vv) + state * (1 + int(S0)),
                        ch * (2 * cc + rec_sweep + dd + cd) + ck * (r - 1) * 2 * cd),
        "k_fwd_sweep_nosave": (ch * step_flops, T * (qk + 2 * vv) + state * (1 + int(S0)),
                               ch * (2 * cc + rec_sweep) + ck * (r - 1) * 2 * cd),
        # K dS, M^T dO, T^T dDelta, Q^T dO, K^T A; reads T, M, gates; writes dV, saves dS_c and A.
        "k_bwd_sweep": (ch * step_flops, T * (qk + 2 * vv) + state * (1 + int(dST)),
                        ch * (2 * cc + rec_sweep + dd + cd) + ck * (r - 1) * 2 * cd),
        # per value head dO S0^T, A S0^T, Delta dS^T, dO Delta^T, A Delta^T; per key head Q K^T,
        # K K^T and the products folding the head sums into dq, dk. Reads S_c, dS_c, Delta, A.
        "k_bwd_grad": (ch * step_flops + ck * 10 * C * C * D, T * (qk + 2 * vv + dqk + dgb),
                       ch * (2 * dd + 2 * cd + rec_grad)),
    }
    return m.get(name)


# Whole-path algorithmic work per token at Hk=16, Hv=48, D=128: q, k, v, g, beta in and o out
# (forward); q, k, v, g, beta, dO in and dq, dk, dv, dg, dbeta out (backward).
PATH_BYTES_PER_TOKEN = {"fwd": 33152, "fwd+bwd": 87168}
PATH_FLOPS_PER_TOKEN = {"fwd": 7.60e6, "fwd+bwd": 29.36e6}


# ----------------------------------------------------------------------------- counters
def _kernel_key(name):
    m = re.search(r"gdn(?:::|\d+)(k_\w+?)(?:I|<|\()", name)
    if not m:
        return None
    k = m.group(1)
    if k == "k_fwd_sweep" and re.search(r"Lb0E|, false>", name):
        k = "k_fwd_sweep_nosave"
    return k


def _read_counters(d):
    """{counter: [(dispatch id, kernel name, value)]} from a rocprofv3 result directory."""
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            out.setdefault(r["Counter_Name"], []).append(
                (int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return {k: sorted(v) for k, v in out.items()}


def _blob(path):
    try:
        text = open(path).read()
        return json.loads(text[text.index("```json") + 7: text.rindex("```")])
    except (OSError, ValueError):
        return None


def summarize_counters(out_path, dirs, command):
    """Write a counter summary for the gdn kernels: per kernel the median of each counter over
    its dispatches (the plain training step; repeated identical dispatches agree to <1%). With
    FETCH_SIZE / WRITE_SIZE the calibrated HBM bytes (scaled by the counts of the calibration
    copy of CALIB_BYTES); with rocprofv3's derived MfmaUtil the MFMA busy fraction of the
    chip's SIMDs over the kernel's dispatches."""
    counters = {}
    for d in dirs:
        counters.update(_read_counters(d))
    agg = {}
    for cname, rows in counters.items():
        for _, kname, v in rows:
            k = _kernel_key(kname)
            if k:
                agg.setdefault(k, {}).setdefault(cname, []).append(v)
    summary = {"source_hash": source_hash(), "kernels": {}}
    lines = [f"# Counter summary: gdn kernels, 4 x 4096 tokens, Hk=16, Hv=48, D=128, bf16, chunk 64", "",
             "rocprofv3 counter passes of the plain training step (one pass per counter group); REPO is the "
             "repository root:", "", "```", command, "```", ""]
    scales = {}
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = counters.get(cname)
        if not rows:
            continue
        for did, kname, v in rows:
            if _kernel_key(kname) is None and 0.5 * CALIB_BYTES < v * 1024 < 2.0 * CALIB_BYTES:
                scales[cname] = CALIB_BYTES / (v * 1024)
                lines.append(f"Calibration: the {CALIB_BYTES >> 20} MiB copy (dispatch {did}) reads {cname} = "
                             f"{v:.0f} KiB: scale {scales[cname]:.4f} bytes per counted byte.")
                break
        else:
            raise SystemExit(f"calibration copy not found for {cname} (run the pass with --pmc-calib)")
    summary["scales"] = {k: round(v, 4) for k, v in scales.items()}
    names = sorted({c for k in agg for c in agg[k]})
    lines += ["", "Per kernel, the median over its dispatches:", "",
              "| kernel | dispatches | " + " | ".join(names) + " | derived |",
              "|---|---|" + "---|" * len(names) + "---|"]
    for k in sorted(agg):
        med = {c: statistics.median(v) for c, v in agg[k].items()}
        ent = {c: round(v, 1) for c, v in med.items()}
        derived = []
        if "FETCH_SIZE" in med and "WRITE_SIZE" in med and len(scales) == 2:
            b = med["FETCH_SIZE"] * 1024 * scales["FETCH_SIZE"] + med["WRITE_SIZE"] * 1024 * scales["WRITE_SIZE"]
            ent["hbm_bytes"] = int(b)
            derived.append(f"HBM {b / 1e6:.1f} MB")
        if "MfmaUtil" in med:  # rocprofv3's derived counter: MFMA busy cycles / (GPU busy cycles x SIMDs)
            ent["mfma_busy"] = round(med["MfmaUtil"] / 100.0, 4)
            derived.append(f"MFMA busy {med['MfmaUtil']:.1f}%")
        if "SQ_INSTS_VALU" in med and med.get("SQ_INSTS_MFMA"):
            ent["valu_per_mfma"] = round(med["SQ_INSTS_VALU"] / med["SQ_INSTS_MFMA"], 2)
            derived.append(f"VALU/MFMA {ent['valu_per_mfma']}")
        if "SQ_LDS_BANK_CONFLICT" in med and med.get("SQ_LDS_IDX_ACTIVE"):
            ent["lds_conflict_frac"] = round(med["SQ_LDS_BANK_CONFLICT"] / med["SQ_LDS_IDX_ACTIVE"], 4)
            derived.append(f"LDS cycles in conflicts {100 * ent['lds_conflict_frac']:.1f}%")
        if "LdsUtil" in med:
            derived.append(f"LDS busy {med['LdsUtil']:.1f}%")
        summary["kernels"][k] = ent
        n = max(len(v) for v in agg[k].values())
        lines.append(f"| {k} | {n} | " + " | ".join(f"{med.get(c, float('nan')):.0f}" for c in names) +
                     f" | {'; '.join(derived)} |")
    lines += ["", "Machine-readable (bench.py reads it; valid while the kernel sources hash to `source_hash`):",
              "", "```json", json.dumps(summary, indent=1), "```", ""]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def summarize_stats(out_path, stats_csv, command, title):
    """Write a kernel-statistics summary from a rocprofv3 ``--stats`` kernel_stats.csv: per gdn
    kernel the calls and the average, minimum and maximum duration."""
    rows = []
    for r in csv.DictReader(open(stats_csv)):
        k = _kernel_key(r["Name"])
        if k:
            rows.append((k, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    lines = [f"# Kernel statistics: {title}", "", "Command (one MI355X; REPO is the repository root):", "", "```",
             command, "```", "", f"Source: rocprofv3 `--stats` kernel statistics (`{os.path.basename(stats_csv)}`). "
             "Warmup and timed calls are both counted; the minima are the steady-state figures.", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | share of GPU time |", "|---|---|---|---|---|---|"]
    for k, n, avg, mn, mx, pct in rows:
        lines.append(f"| {k} | {n} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f} % |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def committed_counter(path, kernel, key):
    blob = _blob(path)
    if not blob or blob.get("source_hash") != source_hash():
        return None
    return blob.get("kernels", {}).get(kernel, {}).get(key)


# ----------------------------------------------------------------------------- timing
class Timer:
    """Times fn over iterations, each bracketed by HIP events on torch's current stream (the
    library's launch stream), with a FLUSH_BYTES scratch write between iterations."""

    def __init__(self, torch):
        self.torch = torch
        self.flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    def flush(self, i):
        self.flush_buf.fill_(float(i))

    def run(self, fn, iters, warmup):
        torch = self.torch
        for i in range(warmup):
            self.flush(i)
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        t0 = time.perf_counter()
        for i, (a, b) in enumerate(ev):
            self.flush(i)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [a.elapsed_time(b) for a, b in ev]
        return {"median_ms": statistics.median(ms), "mean_ms": statistics.fmean(ms), "min_ms": min(ms),
                "iters": iters, "wall_s": wall}


def workload(G, torch, case, fused=False):
    """Device buffers and the step closures of one workload."""
    from synth.device import problem, to_device

    d = to_device(case)
    p = problem(case, d)
    T, Hv, D = case.T_total, case.Hv, case.Dk
    dev = d["v"].device
    g, beta = d["g"], d["beta"]
    if fused:  # raw q/k rows, alpha and beta_raw: the L2 norm and the gate chain run in the kernels
        d["a_log"] = torch.full((Hv,), -0.5, dtype=torch.float32, device=dev)
        d["dt_bias"] = torch.full((Hv,), 0.5, dtype=torch.float32, device=dev)
        p.qk_l2norm, p.a_log, p.dt_bias = 1, d["a_log"].data_ptr(), d["dt_bias"].data_ptr()
        g, beta = torch.zeros_like(d["g"]), torch.zeros_like(d["beta"])
    o = torch.empty(T, Hv, D, dtype=d["v"].dtype, device=dev)
    S_T = torch.empty(case.N, Hv, D, D, dtype=torch.float32, device=dev)
    states = torch.empty(G.gdn_chunk_state_bytes(p), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(G.gdn_fwd_workspace_bytes(p), G.gdn_bwd_workspace_bytes(p)), dtype=torch.uint8,
                     device=dev)
    dg = torch.empty(T, Hv, dtype=torch.float32, device=dev)
    dbeta = torch.empty(T, Hv, dtype=torch.float32, device=dev)
    dS0 = torch.empty(case.N, Hv, D, D, dtype=torch.float32, device=dev)

    def fwd():
        G.gdn_fwd(p, d["q"], d["k"], d["v"], g, beta, d["S0"], o, S_T, states, None)

    def fwd_only():
        G.gdn_fwd(p, d["q"], d["k"], d["v"], g, beta, d["S0"], o, S_T, None, ws)

    def bwd():
        G.gdn_bwd(p, d["q"], d["k"], d["v"], g, beta, d["S0"], states, d["dO"], d["dST"],
                  d["dq"], d["dk"], d["dv"], dg, dbeta, dS0, ws)

    def step():
        fwd()
        bwd()

    return {"step": step, "fwd": fwd, "fwd_only": fwd_only, "keep": (d, o, S_T, states, ws, dg, dbeta, dS0)}


def capture(torch, fn):
    """fn's kernel launches captured once in a HIP graph (torch.cuda.graph: the library enqueues
    on torch's current stream, the capture stream); returns the graph's replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph.replay


def decode_bench(G, torch, timer, iters, N=256, Hk=16, Hv=48, D=128):
    """One decode step (gdn_decode) for a serving batch of N rows at the training heads: bf16
    q/k/v rows of a packed projection, float32 state pool of N slots (identity map). Bytes: the
    state read and written once, plus the rows in and out."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    width = 2 * Hk * D + Hv * D
    buf = (0.1 * torch.randn(N, width, device="cuda", generator=gen)).to(torch.bfloat16)
    q, k, v = buf[:, : Hk * D], buf[:, Hk * D: 2 * Hk * D], buf[:, 2 * Hk * D:]
    g = 0.5 + 0.5 * torch.rand(N, Hv, device="cuda", generator=gen)
    beta = torch.rand(N, Hv, device="cuda", generator=gen)
    state = 0.3 * torch.randn(N, Hv, D, D, device="cuda", generator=gen)
    o = torch.empty(N, Hv * D, dtype=torch.bfloat16, device="cuda")
    p = G.make_problem(N, N, Hk, Hv, D, T=1, dtype="bf16")
    G.gdn_trace_enable(True)
    G.gdn_trace_collect()
    t = timer.run(lambda: G.gdn_decode(p, q, k, v, g, beta, state, None, o), iters, 3)
    G.gdn_trace_enable(False)
    tr = G.gdn_trace_collect()
    k_ms = tr["k_decode"][0] / tr["k_decode"][1]
    nbytes = 2 * N * Hv * D * D * 4 + N * width * 2 + N * Hv * 8 + N * Hv * D * 2
    return {"workload": f"{N} rows x 1 token, Hk{Hk} Hv{Hv} D{D}, bf16 packed rows, f32 state pool of {N} slots",
            "rows_per_s": round(N / (t["median_ms"] / 1e3), 1), "ms_per_step": round(t["median_ms"], 4),
            "kernel_ms": round(k_ms, 4), "bytes": nbytes, "GB/s": round(nbytes / (k_ms / 1e3) / 1e9, 1),
            "hbm_frac": round(nbytes / (k_ms / 1e3) / PEAK["hbm"], 4)}


def conv_bench(G, torch, timer, iters, rows=16384, ch=10240, K=4):
    """Causal conv1d + SiLU forward and input gradient over the training shape's packed
    projection (16384 rows x 10240 channels, bf16, 4 sequences of 4096, K = 4). Bytes: x read
    and y written (forward); x, dy read and dx written (backward)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    x = torch.randn(rows, ch, device="cuda", generator=gen).to(torch.bfloat16)
    dy = torch.randn(rows, ch, device="cuda", generator=gen).to(torch.bfloat16)
    w = torch.rand(ch, K, device="cuda", generator=gen) - 0.5
    y, dx = torch.empty_like(x), torch.empty_like(x)
    p = G.make_conv_problem(4, rows, ch, K, T=rows // 4, dtype="bf16")
    out = {"workload": f"{rows} rows x {ch} channels (4 x {rows // 4}), K {K}, bf16"}
    for name, fn, nb in (("k_conv_fwd", lambda: G.gdn_conv1d_silu_fwd(p, x, w, y), 2 * rows * ch * 2),
                         ("k_conv_bwd", lambda: G.gdn_conv1d_silu_bwd(p, x, w, dy, dx), 3 * rows * ch * 2)):
        G.gdn_trace_enable(True)
        G.gdn_trace_collect()
        timer.run(fn, iters, 3)
        G.gdn_trace_enable(False)
        tr = G.gdn_trace_collect()
        ms = tr[name][0] / tr[name][1]
        out[name] = {"ms": round(ms, 4), "bytes": nb, "GB/s": round(nb / (ms / 1e3) / 1e9, 1),
                     "hbm_frac": round(nb / (ms / 1e3) / PEAK["hbm"], 4)}
    return out


# ----------------------------------------------------------------------------- host cpu
def host_cpu():
    """CPU model, logical CPUs, the CPUs this process may run on and the cgroup CPU quota."""
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    nproc = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = nproc
    quota = None
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()
        if q != "max":
            quota = float(q) / float(per)
    except (OSError, ValueError):
        pass
    usable = avail if quota is None else max(1, min(avail, int(quota + 0.5)))
    return {"model": model, "nproc": nproc, "affinity": avail, "cgroup_quota": quota, "usable": usable}


def cpu_baseline(case3, case2):
    """The float64 oracle as it stands: the whole training batch, fwd + bwd, on every core the
    process may use (repeated to at least 10 s), and one core on a bounded sample of the strided
    workload (its first key-head group: 2048 tokens x 3 of the 48 value heads)."""
    import oracle

    oracle.build()
    cpu = host_cpu()
    n = cpu["usable"]
    t0, reps = time.perf_counter(), 0
    while True:
        oracle.run_case(case3, backward=True, nthreads=n)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 8:
            break
    used = min(n, case3.N * case3.Hk)
    t1 = time.perf_counter()
    oracle.run_case(case2, backward=True, nthreads=1, key_heads=[0])
    dt1 = time.perf_counter() - t1
    frac = (case2.Hv // case2.Hk) / case2.Hv
    return {"value": round(reps * case3.T_total / dt, 2), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"the whole training batch ({case3.N} x {case3.lens[0]} tokens, all {case3.Hv} value heads) "
                      f"x {reps}, fwd+bwd, float64, {used} threads (one per sequence x key-head group, of {n} usable "
                      f"CPUs); {dt:.1f} s",
            "cpu": cpu,
            "single_core": {"value": round(case2.T_total * frac / dt1, 2), "unit": "tokens/s (all 48 heads)",
                            "cores": 1, "sample": f"strided workload, 1 sequence x {case2.T_total} tokens, key head 0 "
                                                  f"(value heads 0-2), fwd+bwd, float64, 1 thread; {dt1:.2f} s, "
                                                  f"scaled by 3/48"}}


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-step", action="store_true",
                    help="run only warmup + timed plain training steps (for rocprofv3)")
    ap.add_argument("--fwd-only", action="store_true",
                    help="with --profile-step: time forward-only calls instead of training steps")
    ap.add_argument("--pmc-calib", action="store_true",
                    help="first copy a buffer of known size (the counter calibration dispatch)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PATH",
                    help="OUT_MD DIR...: write a counter summary from rocprofv3 counter result directories")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("OUT_MD", "STATS_CSV", "TITLE"),
                    help="write a kernel-statistics summary from a rocprofv3 kernel_stats.csv")
    ap.add_argument("--command", default="", help="command line recorded in a counter or statistics summary")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1:], args.command)
        return
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats[:2], args.command, args.summarize_stats[2])
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the recurrence shards "
              "without communication by key-head group or sequence, one process per GPU); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_34_amd as G
    from synth import config_case

    if args.pmc_calib:  # a plain copy of known size, for the FETCH_SIZE / WRITE_SIZE scale factors
        src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    case = config_case(3)
    T, Hk, Hv, D, C = case.T_total, case.Hk, case.Hv, case.Dk, case.chunk
    timer = Timer(torch)
    wl = workload(G, torch, case)
    print(f"[bench] workload ready: T_total={T} Hk={Hk} Hv={Hv} D={D} C={C}", file=sys.stderr, flush=True)

    step_fn = wl["fwd_only"] if (args.profile_step and args.fwd_only) else wl["step"]
    G.gdn_trace_enable(True)
    G.gdn_trace_collect()  # (warmup launches are collected and dropped below)
    for i in range(args.warmup):
        timer.flush(i)
        step_fn()
    torch.cuda.synchronize()
    G.gdn_trace_collect()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    eager_t = timer.run(step_fn, args.steps, 0)
    G.gdn_trace_enable(False)
    trace = G.gdn_trace_collect()
    print(f"[bench] eager: {eager_t['median_ms']:.4f} ms/step (median of {args.steps})", file=sys.stderr, flush=True)
    if args.profile_step:
        return
    # The headline: the same step (the same four kernels on the same buffers) captured once in
    # a HIP graph and replayed, so the launch gaps between the kernels shrink.
    step_graph = capture(torch, wl["step"])
    main_t = timer.run(step_graph, args.steps, 3)
    ms_step = main_t["median_ms"]
    print(f"[bench] timed (graph replay): {ms_step:.4f} ms/step (median of {args.steps})", file=sys.stderr,
          flush=True)

    iters = max(args.steps, 20)
    fwd_t = timer.run(capture(torch, wl["fwd"]), iters, 3)
    # forward-only: kernel times from the library's events on an eager run, tokens/s from
    # replays of its graph (as the headline)
    G.gdn_trace_enable(True)
    G.gdn_trace_collect()
    fwdo_eager = timer.run(wl["fwd_only"], iters, 3)
    G.gdn_trace_enable(False)
    trace_fo = G.gdn_trace_collect()
    fwdo_t = timer.run(capture(torch, wl["fwd_only"]), iters, 3)
    print(f"[bench] fwd {fwd_t['median_ms']:.4f} ms, fwd-only {fwdo_t['median_ms']:.4f} ms (eager "
          f"{fwdo_eager['median_ms']:.4f})", file=sys.stderr, flush=True)
    fused = workload(G, torch, case, fused=True)
    fused_t = timer.run(capture(torch, fused["step"]), iters, 3)
    del fused
    extra = {}
    for i, tag in ((2, "strided_B1_T2048"), (4, "varlen_8seq")):
        c = config_case(i)
        w = workload(G, torch, c)
        st, fo = timer.run(capture(torch, w["step"]), iters, 3), timer.run(capture(torch, w["fwd_only"]), iters, 3)
        extra[tag] = {"workload": c.name, "tokens": c.T_total,
                      "fwd_bwd": {"ms": round(st["median_ms"], 4), "tokens_per_s": round(c.T_total / st["median_ms"] * 1e3, 1)},
                      "fwd_only": {"ms": round(fo["median_ms"], 4), "tokens_per_s": round(c.T_total / fo["median_ms"] * 1e3, 1)}}
        print(f"[bench] {tag}: fwd+bwd {st['median_ms']:.4f} ms, fwd-only {fo['median_ms']:.4f} ms", file=sys.stderr,
              flush=True)
        del w
    wl_keep = wl  # noqa: F841  (the headline buffers stay allocated to the end)
    decode = decode_bench(G, torch, timer, iters)
    conv = conv_bench(G, torch, timer, iters)
    print(f"[bench] decode {decode['GB/s']} GB/s; conv1d fwd {conv['k_conv_fwd']['GB/s']} bwd "
          f"{conv['k_conv_bwd']['GB/s']} GB/s", file=sys.stderr, flush=True)

    n_chunks = T // C
    model = lambda k: kernel_model(k, C, D, Hk, Hv, T, n_chunks, case.N, S0=case.S0 is not None,
                                   dST=case.dST is not None)
    kernels = {}
    for k, (tot, n) in sorted(trace.items(), key=lambda kv: -kv[1][0]):
        t = tot / n / 1e3
        ent = {"ms": round(t * 1e3, 4), "launches_per_step": n // args.steps}
        m = model(k)
        if m:
            ent.update({"TFLOP/s": round(m[0] / t / 1e12, 1), "method_GB/s": round(m[1] / t / 1e9, 1),
                        "with_design_GB/s": round((m[1] + m[2]) / t / 1e9, 1)})
            tr = committed_counter(TRAFFIC_FILE, k, "hbm_bytes")
            if tr:
                ent["counter_GB/s"] = round(tr / t / 1e9, 1)
        kernels[k] = ent
    dom = max(trace.items(), key=lambda kv: kv[1][0])[0]
    avg_s = trace[dom][0] / trace[dom][1] / 1e3
    flops, mbytes, dbytes = model(dom)
    if flops / PEAK["bf16_mfma"] >= mbytes / PEAK["hbm"]:
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(flops / avg_s / 1e12, 3),
                    "peak": PEAK["bf16_mfma"] / 1e12, "unit": "TFLOP/s", "frac": round(flops / avg_s / PEAK["bf16_mfma"], 4)}
    else:
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(mbytes / avg_s / 1e9, 1),
                    "peak": PEAK["hbm"] / 1e9, "unit": "GB/s", "frac": round(mbytes / avg_s / PEAK["hbm"], 4)}
    roofline.update({"traffic": committed_counter(TRAFFIC_FILE, dom, "hbm_bytes"), "avg_launch_ms": round(avg_s * 1e3, 4),
                     "algorithmic_bytes": mbytes, "design_bytes": dbytes, "algorithmic_flops": flops,
                     "mfma_frac": round(flops / avg_s / PEAK["bf16_mfma"], 4),
                     "hbm_frac": round(mbytes / avg_s / PEAK["hbm"], 4),
                     "mfma_busy": committed_counter(MFMA_FILE, dom, "mfma_busy")})
    path = {}
    for tag, ms in (("fwd+bwd", ms_step), ("fwd", fwdo_t["median_ms"])):
        b = PATH_BYTES_PER_TOKEN[tag] * T + (2 if tag == "fwd" else 3) * case.N * Hv * D * D * 4
        f = PATH_FLOPS_PER_TOKEN[tag] * T
        path[tag] = {"bytes": b, "flops": f, "hbm_frac": round(b / (ms / 1e3) / PEAK["hbm"], 4),
                     "mfma_frac": round(f / (ms / 1e3) / PEAK["bf16_mfma"], 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, config_case(2))
        print(f"[bench] cpu baseline {cpu['value']} tokens/s on {cpu['cores']} threads", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC, "value": round(T / (ms_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "B4 T4096 Hk16 Hv48 Dk=Dv=128, bf16 packed qkv [16384,10240], f32 gates/state, "
                               "chunk 64, fwd (saving chunk states) + bwd",
                   "global_batch": case.N, "seq_len": case.lens[0], "parallelism": "single GPU"},
        "timing": {"statistic": f"median of {args.steps} steps, each a replay of the step's HIP graph "
                                f"bracketed by HIP events, {FLUSH_BYTES >> 20} MiB scratch write between steps",
                   "mean_ms": round(main_t["mean_ms"], 4), "min_ms": round(main_t["min_ms"], 4),
                   "eager_ms_per_step": round(eager_t["median_ms"], 4)},
        "fwd_tokens_per_s": round(T / (fwd_t["median_ms"] / 1e3), 1),
        "fwd_only_tokens_per_s": round(T / (fwdo_t["median_ms"] / 1e3), 1),
        "fwd_only_eager_ms": round(fwdo_eager["median_ms"], 4),
        "fwd_only_kernels_ms": {k: round(v[0] / v[1], 4) for k, v in trace_fo.items()},
        "fused_l2norm_gate_chain": {"ms_per_step": round(fused_t["median_ms"], 4),
                                    "tokens_per_s": round(T / (fused_t["median_ms"] / 1e3), 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "path_roofline": path,
        "workloads": extra,
        "decode": decode,
        "conv1d": conv,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
