#!/usr/bin/env python3
"""Benchmark: gated delta-net forward + backward tokens/s on one MI355X.

Workload: 4 sequences x 4096 tokens, 16 key heads shared by 48 value heads, head size
128, q/k/v as bf16 row views of one packed [16384, 10240] projection, float32 gates
and state, chunk 64, S0 = 0, dS_T ~ N(0, 0.1^2) (the 27B-layer training shape; inputs
from synth.config_case(3), seeded, synthetic). One step = gdn_fwd (saving chunk
states) + gdn_bwd over the whole batch; inputs are resident in HBM before timing.

Prints one JSON line. ``roofline`` covers the kernel with the largest share of the
step, timed live with HIP events recorded by the library around each launch on the
launch stream; its ``traffic`` is the measured HBM bytes per launch from the committed
counter summary (rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by what the counter
reads for a plain copy of known size), or null when the kernels changed since those
counters were taken. ``cpu_baseline`` times the float64 oracle on the whole batch (all
four sequences, all 48 heads), fwd + bwd, on the host cores, repeated to at least 10 s.
``decode`` is a separate measurement outside the timed training steps: one gdn_decode
step for 256 rows at the same heads (float32 state pool, bf16 packed rows), with its
kernel time, bytes and fraction of the HBM peak. ``conv1d`` likewise times the causal
conv1d + SiLU forward and input gradient over the same packed projection.

Counter runs: ``--pmc-calib`` first copies a buffer of known size (the calibration
dispatch); ``--summarize-pmc FETCH_DIR WRITE_DIR`` turns the two rocprofv3 result
directories into the committed summary.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN fwd+bwd tokens/s @Hk16/Hv48/D128 T=4096; % MFMA / HBM roofline"
PEAK = {"f32_mfma": 157.3e12, "bf16_mfma": 2.5e15, "hbm": 8.0e12}
WORKLOAD_TAG = "B4_T4096_Hk16_Hv48_D128_bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", f"gdn_kernels_{WORKLOAD_TAG}_hbm_traffic.md")
CALIB_BYTES = 3 << 27  # the calibration copy reads and writes 384 MiB


def source_hash():
    """Hash of the HIP sources and headers: counter summaries are valid for this code only."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_34_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _kernel_key(name):
    m = re.search(r"gdn(?:::|\d+)(k_\w+?)(?:I|<|\()", name)
    return m.group(1) if m else None


def _read_counters(d, counter):
    """[(dispatch id, kernel name, value)] of one counter from a rocprofv3 result directory."""
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return sorted(out)


def summarize_pmc(fetch_dir, write_dir, out_path, command):
    """Write the traffic summary: per gdn kernel the average FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch) and the calibrated HBM bytes, with the copy-kernel scale factors."""
    fetch, write = _read_counters(fetch_dir, "FETCH_SIZE"), _read_counters(write_dir, "WRITE_SIZE")

    def calib(rows):
        # the calibration copy is the first non-gdn dispatch that reads (or writes) ~CALIB_BYTES
        for did, name, v in rows:
            if _kernel_key(name) is None and 0.5 * CALIB_BYTES < v * 1024 < 2.0 * CALIB_BYTES:
                return did, v
        raise SystemExit("calibration copy not found (run the counter passes with --pmc-calib)")

    (fd, fv), (wd, wv) = calib(fetch), calib(write)
    f_scale, w_scale = CALIB_BYTES / (fv * 1024), CALIB_BYTES / (wv * 1024)
    agg = {}
    for rows, key in ((fetch, "fetch_kib"), (write, "write_kib")):
        for _, name, v in rows:
            k = _kernel_key(name)
            if k:
                agg.setdefault(k, {}).setdefault(key, []).append(v)
    summary = {"source_hash": source_hash(), "calib_bytes": CALIB_BYTES, "fetch_scale": round(f_scale, 4),
               "write_scale": round(w_scale, 4), "kernels": {}}
    lines = [f"# HBM traffic per launch: gdn kernels, 4 x 4096 tokens, Hk=16, Hv=48, D=128, bf16, chunk 64", "",
             "Two rocprofv3 counter passes of the same bench command (one counter each); REPO is the repository root:",
             "", "```", command, "```", "",
             f"Calibration: a plain copy of {CALIB_BYTES >> 20} MiB (torch `copy_`, the first large non-gdn dispatch) "
             f"reads FETCH_SIZE = {fv:.0f} KiB (dispatch {fd}) and WRITE_SIZE = {wv:.0f} KiB (dispatch {wd}); "
             f"scale factors {f_scale:.4f} (fetch) and {w_scale:.4f} (write) turn counter KiB into bytes.", "",
             "Per kernel the smallest count over its dispatches (the plain step's launches; the fused-prologue "
             "step's prep and gradient kernels move more).", "",
             "| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes per launch (calibrated) |",
             "|---|---|---|---|---|"]
    for k in sorted(agg):
        # the smallest count over the kernel's dispatches: the bench also runs the step with the
        # q/k L2 norm and gate chain fused, whose prep and gradient kernels move more bytes, and
        # the plain step's launches are the ones the roofline line describes (repeated
        # identical dispatches agree to within 0.1%)
        fk = min(agg[k].get("fetch_kib", [0]))
        wk = min(agg[k].get("write_kib", [0]))
        total = fk * 1024 * f_scale + wk * 1024 * w_scale
        summary["kernels"][k] = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1), "bytes": int(total)}
        lines.append(f"| {k} | {len(agg[k].get('fetch_kib', []))} | {fk:.0f} | {wk:.0f} | {total / 1e6:.1f} MB |")
    lines += ["", "Machine-readable (bench.py reads it; valid while the kernel sources hash to `source_hash`):", "",
              "```json", json.dumps(summary, indent=1), "```", ""]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def measured_traffic(kernel):
    """Calibrated HBM bytes per launch of `kernel` from the committed summary, or None when
    there is none or the sources changed since the counters were taken."""
    try:
        text = open(TRAFFIC_FILE).read()
        blob = json.loads(text[text.index("```json") + 7: text.rindex("```")])
    except (OSError, ValueError):
        return None
    if blob.get("source_hash") != source_hash():
        return None
    k = blob.get("kernels", {}).get(kernel)
    return k["bytes"] if k else None


def kernel_model(name, C, D, Hk, Hv, n_chunks, es=2):
    """Algorithmic MFMA flops and HBM bytes of one launch of a kernel: the products it
    forms and the tensors it must read and write, each counted once per unit of work
    (chunk x value head, or chunk x key head for what the r value heads of a key head
    share), times the units of one launch. Activations are es bytes, gates float32."""
    ch, ck = n_chunks * Hv, n_chunks * Hk  # (chunk, value head) and (chunk, key head) units
    cd, cc, dd = C * D * es, C * C * es, D * D * es
    gates = 8 * C  # gamma and beta (or g and beta) per unit, float32
    grec = 16 * C  # the gate record: gamma, beta, b = 2^gamma, e = 2^(gamma_last - gamma)
    model = {
        # K K^T and Q K^T per key head. Reads K, Q, g, beta; writes T, M and the gate record.
        "k_prep": (ck * 4 * C * C * D, ck * 2 * cd + ch * (gates + 2 * cc + grec)),
        # K S, Q S, T X, M Delta, K^T (e o Delta). Reads K, Q, V, T, M, gates; writes S, Delta, O.
        "k_fwd_sweep": (ch * (6 * C * D * D + 4 * C * C * D), ck * 2 * cd + ch * (cd + 2 * cc + grec + dd + 2 * cd)),
        # K dS, M^T dO, T^T dDelta, Q^T dO, K^T (nb o A). Reads K, Q, dO, T, M, gates; writes dS,
        # A^T (A = T^T dDelta) and dV.
        "k_bwd_sweep": (ch * (6 * C * D * D + 4 * C * C * D), ck * 2 * cd + ch * (cd + 2 * cc + grec + dd + 2 * cd)),
        # Per value head dO S0^T, Delta dS^T, A S0^T, dO Delta^T, A Delta^T; per key head Q K^T,
        # K K^T and the three products that fold the head sums into dq and dk. Reads S0, dS,
        # Delta, A^T, dO, V, gates and g per value head, K and Q per key head; writes dg, dbeta
        # per value head and dq, dk per key head.
        "k_bwd_grad": (ch * (6 * C * D * D + 4 * C * C * D) + ck * 10 * C * C * D,
                       ch * (2 * dd + 4 * cd + gates + 4 * C + 8 * C) + ck * 4 * cd),
    }
    return model.get(name)


# Whole-path algorithmic work per token at Hk=16, Hv=48, D=128 (q, k, v, g, beta, o in the
# forward; q, k, v, g, beta, dO in and dq, dk, dv, dg, dbeta out in the backward), and the
# bytes of one float32 state tensor per sequence.
PATH_BYTES_PER_TOKEN = 87168
PATH_FLOPS_PER_TOKEN = 29.36e6


def decode_bench(G, torch, steps, N=256, Hk=16, Hv=48, D=128):
    """One decode step (gdn_decode) for a serving batch of N rows at the training heads:
    bf16 q/k/v rows of a packed projection, float32 state pool of N slots (identity map),
    timed over ``steps`` calls; the kernel time comes from the library's HIP events on the
    launch stream. Bytes: the state read and written once, plus the rows in and out."""
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    width = 2 * Hk * D + Hv * D
    buf = (0.1 * torch.randn(N, width, device=dev, generator=gen)).to(torch.bfloat16)
    q, k, v = buf[:, : Hk * D], buf[:, Hk * D: 2 * Hk * D], buf[:, 2 * Hk * D:]
    g = 0.5 + 0.5 * torch.rand(N, Hv, device=dev, generator=gen)
    beta = torch.rand(N, Hv, device=dev, generator=gen)
    state = 0.3 * torch.randn(N, Hv, D, D, device=dev, generator=gen)
    o = torch.empty(N, Hv * D, dtype=torch.bfloat16, device=dev)
    p = G.make_problem(N, N, Hk, Hv, D, T=1, dtype="bf16")

    def step():
        G.gdn_decode(p, q, k, v, g, beta, state, None, o)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    G.gdn_trace_enable(True)
    G.gdn_trace_collect()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    G.gdn_trace_enable(False)
    tr = G.gdn_trace_collect()
    ms = start.elapsed_time(end) / steps
    k_ms = tr["k_decode"][0] / tr["k_decode"][1]
    nbytes = 2 * N * Hv * D * D * 4 + N * width * 2 + N * Hv * 8 + N * Hv * D * 2
    return {"workload": f"{N} rows x 1 token, Hk{Hk} Hv{Hv} D{D}, bf16 packed rows, f32 state pool of {N} slots",
            "rows_per_s": round(N / (ms / 1e3), 1), "ms_per_step": round(ms, 4), "kernel_ms": round(k_ms, 4),
            "bytes": nbytes, "GB/s": round(nbytes / (k_ms / 1e3) / 1e9, 1),
            "hbm_frac": round(nbytes / (k_ms / 1e3) / PEAK["hbm"], 4)}


def conv_bench(G, torch, steps, rows=16384, ch=10240, K=4):
    """Causal conv1d + SiLU forward and input gradient over the training shape's packed
    projection (16384 rows x 10240 channels, bf16, 4 sequences of 4096, K = 4), timed over
    ``steps`` calls each with the library's HIP events. Bytes: x read and y written
    (forward); x, dy read and dx written (backward)."""
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    x = torch.randn(rows, ch, device=dev, generator=gen).to(torch.bfloat16)
    dy = torch.randn(rows, ch, device=dev, generator=gen).to(torch.bfloat16)
    w = torch.rand(ch, K, device=dev, generator=gen) - 0.5
    y, dx = torch.empty_like(x), torch.empty_like(x)
    p = G.make_conv_problem(4, rows, ch, K, T=rows // 4, dtype="bf16")
    for _ in range(3):
        G.gdn_conv1d_silu_fwd(p, x, w, y)
        G.gdn_conv1d_silu_bwd(p, x, w, dy, dx)
    torch.cuda.synchronize()
    G.gdn_trace_enable(True)
    G.gdn_trace_collect()
    for _ in range(steps):
        G.gdn_conv1d_silu_fwd(p, x, w, y)
        G.gdn_conv1d_silu_bwd(p, x, w, dy, dx)
    torch.cuda.synchronize()
    G.gdn_trace_enable(False)
    tr = G.gdn_trace_collect()
    out = {"workload": f"{rows} rows x {ch} channels (4 x {rows // 4}), K {K}, bf16"}
    for name, nb in (("k_conv_fwd", 2 * rows * ch * 2), ("k_conv_bwd", 3 * rows * ch * 2)):
        ms = tr[name][0] / tr[name][1]
        out[name] = {"ms": round(ms, 4), "bytes": nb, "GB/s": round(nb / (ms / 1e3) / 1e9, 1),
                     "hbm_frac": round(nb / (ms / 1e3) / PEAK["hbm"], 4)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-calib", action="store_true",
                    help="first copy a buffer of known size (the counter calibration dispatch)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM traffic summary from two rocprofv3 counter result directories")
    ap.add_argument("--pmc-command", default="", help="command line recorded in the traffic summary")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], TRAFFIC_FILE, args.pmc_command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the recurrence shards "
              "without communication by key-head group or sequence, one process per GPU); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_34_amd as G
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gdn_gpu import problem, to_device
    from synth import config_case

    if args.pmc_calib:  # a plain copy of known size, for the FETCH_SIZE / WRITE_SIZE scale factors
        src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    case = config_case(3)
    d = to_device(case)
    p = problem(case, d)
    T, Hk, Hv, D, C = case.T_total, case.Hk, case.Hv, case.Dk, case.chunk
    dev = d["v"].device
    o = torch.empty(T, Hv, D, dtype=torch.bfloat16, device=dev)
    S_T = torch.empty(case.N, Hv, D, D, dtype=torch.float32, device=dev)
    states = torch.empty(G.gdn_chunk_state_bytes(p), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(G.gdn_fwd_workspace_bytes(p), G.gdn_bwd_workspace_bytes(p)), dtype=torch.uint8,
                     device=dev)
    dg = torch.empty(T, Hv, dtype=torch.float32, device=dev)
    dbeta = torch.empty(T, Hv, dtype=torch.float32, device=dev)
    dS0 = torch.empty(case.N, Hv, D, D, dtype=torch.float32, device=dev)

    def fwd():
        G.gdn_fwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, S_T, states, ws)

    def bwd():
        G.gdn_bwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], states, d["dO"], d["dST"],
                  d["dq"], d["dk"], d["dv"], dg, dbeta, dS0, ws)

    def step():
        fwd()
        bwd()

    print(f"[bench] workload ready: T_total={T} Hk={Hk} Hv={Hv} D={D} C={C}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    G.gdn_trace_enable(True)
    G.gdn_trace_collect()
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    G.gdn_trace_enable(False)
    trace = G.gdn_trace_collect()
    ms_step = start.elapsed_time(end) / args.steps

    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        fwd()
    end.record()
    torch.cuda.synchronize()
    ms_fwd = start.elapsed_time(end) / args.steps
    print(f"[bench] timed: {ms_step:.3f} ms/step, fwd {ms_fwd:.3f} ms", file=sys.stderr, flush=True)

    # The same step with the layer's q/k L2 normalisation and gate chain fused into the
    # kernels (raw q, k rows; alpha and beta_raw in place of g and beta): what the fusion
    # costs over the plain step (outside the timed region above).
    ta_log = torch.full((Hv,), -0.5, dtype=torch.float32, device=dev)
    tdt = torch.full((Hv,), 0.5, dtype=torch.float32, device=dev)
    pf = problem(case, d)
    pf.qk_l2norm, pf.a_log, pf.dt_bias = 1, ta_log.data_ptr(), tdt.data_ptr()
    states_f = torch.empty(G.gdn_chunk_state_bytes(pf), dtype=torch.uint8, device=dev)
    alpha, beta_raw = torch.zeros_like(d["g"]), torch.zeros_like(d["beta"])

    def step_fused():
        G.gdn_fwd(pf, d["q"], d["k"], d["v"], alpha, beta_raw, d["S0"], o, S_T, states_f, ws)
        G.gdn_bwd(pf, d["q"], d["k"], d["v"], alpha, beta_raw, d["S0"], states_f, d["dO"], d["dST"],
                  d["dq"], d["dk"], d["dv"], dg, dbeta, dS0, ws)

    for _ in range(args.warmup):
        step_fused()
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step_fused()
    end.record()
    torch.cuda.synchronize()
    ms_fused = start.elapsed_time(end) / args.steps
    del states_f
    decode = decode_bench(G, torch, args.steps)
    print(f"[bench] decode: {decode['kernel_ms']:.4f} ms per step, {decode['GB/s']} GB/s", file=sys.stderr, flush=True)
    conv = conv_bench(G, torch, args.steps)
    print(f"[bench] conv1d: fwd {conv['k_conv_fwd']['GB/s']} GB/s, bwd {conv['k_conv_bwd']['GB/s']} GB/s",
          file=sys.stderr, flush=True)

    n_chunks = T // C
    kernels = {k: round(v[0] / v[1], 4) for k, v in sorted(trace.items(), key=lambda kv: -kv[1][0])}
    dom = max(trace.items(), key=lambda kv: kv[1][0])[0]
    avg_s = trace[dom][0] / trace[dom][1] / 1e3
    flops, nbytes = kernel_model(dom, C, D, Hk, Hv, n_chunks)
    # the binding roofline is the one whose peak takes longer for this launch's work
    if flops / PEAK["bf16_mfma"] >= nbytes / PEAK["hbm"]:
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(flops / avg_s / 1e12, 3),
                    "peak": PEAK["bf16_mfma"] / 1e12, "unit": "TFLOP/s",
                    "frac": round(flops / avg_s / PEAK["bf16_mfma"], 4), "operand_dtype": "bf16"}
    else:
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(nbytes / avg_s / 1e9, 1),
                    "peak": PEAK["hbm"] / 1e9, "unit": "GB/s", "frac": round(nbytes / avg_s / PEAK["hbm"], 4)}
    roofline.update({"traffic": measured_traffic(dom), "avg_launch_ms": round(avg_s * 1e3, 4),
                     "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                     "mfma_frac": round(flops / avg_s / PEAK["bf16_mfma"], 4),
                     "hbm_frac": round(nbytes / avg_s / PEAK["hbm"], 4)})
    per_kernel = {}
    for k in kernels:
        m = kernel_model(k, C, D, Hk, Hv, n_chunks)
        if m:
            t = trace[k][0] / trace[k][1] / 1e3
            per_kernel[k] = {"ms": round(t * 1e3, 4), "TFLOP/s": round(m[0] / t / 1e12, 1),
                             "GB/s": round(m[1] / t / 1e9, 1)}
    state_bytes = case.N * Hv * D * D * 4
    n_state = 3 if d["S0"] is None else 5  # S_T, dS_T, dS0 (+ S0 read twice)
    path_bytes = PATH_BYTES_PER_TOKEN * T + n_state * state_bytes
    path = {"bytes": path_bytes, "flops": PATH_FLOPS_PER_TOKEN * T,
            "hbm_frac": round(path_bytes / (ms_step / 1e3) / PEAK["hbm"], 4),
            "mfma_frac": round(PATH_FLOPS_PER_TOKEN * T / (ms_step / 1e3) / PEAK["bf16_mfma"], 4)}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        oracle.build()
        nthreads = min(oracle.default_threads(), 16)
        t0 = time.perf_counter()
        reps = 0
        while True:  # the whole batch, repeated until at least 10 s of host work
            oracle.run_case(case, backward=True, nthreads=nthreads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or reps >= 8:
                break
        cpu = {"value": round(reps * T / dt, 2), "unit": "tokens/s", "cores": min(nthreads, case.N * Hk),
               "kind": "oracle",
               "sample": f"the whole batch ({case.N} x {case.lens[0]} tokens, all {Hv} value heads) x {reps}, "
                         f"fwd+bwd, float64; {dt:.1f} s"}

    line = {
        "metric": METRIC, "value": round(T / (ms_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "B4 T4096 Hk16 Hv48 Dk=Dv=128, bf16 packed qkv [16384,10240], f32 gates/state, "
                               "chunk 64, fwd (saving chunk states) + bwd",
                   "global_batch": case.N, "seq_len": case.lens[0], "parallelism": "single GPU"},
        "fwd_tokens_per_s": round(T / (ms_fwd / 1e3), 1),
        "fused_l2norm_gate_chain": {"ms_per_step": round(ms_fused, 4), "tokens_per_s": round(T / (ms_fused / 1e3), 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_avg_ms": kernels,
        "kernels": per_kernel,
        "path_roofline": path,
        "decode": decode,
        "conv1d": conv,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
