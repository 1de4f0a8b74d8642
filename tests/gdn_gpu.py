"""Helpers for the GPU tests: move a synth.GdnCase onto the device in the layout the
workload uses (packed qkv rows or contiguous), run the HIP path through the C ABI
binding, and compare with the oracle (normwise max|a-b| / max|b| per tensor)."""
from __future__ import annotations

import numpy as np

import oracle
from synth.device import problem, to_device  # noqa: F401  (re-exported for the tests)

OUT_NAMES = ("o", "S_T")
GRAD_NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def normwise(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    den = float(np.max(np.abs(b)))
    num = float(np.max(np.abs(a - b)))
    return num / den if den > 0 else num


def tol_of(case):
    return 2e-4 if case.dtype == "f32" else 2e-2


def run_gpu(case, backward=True, chunk=None, packed=None, d=None, p=None):
    """Run forward (+ backward) through the C ABI; returns numpy float64 results."""
    import torch
    import gated_delta_rule_34_amd as G

    d = d or to_device(case, packed=packed)
    p = p or problem(case, d, chunk)
    T, Hk, Hv, D = case.T_total, case.Hk, case.Hv, case.Dk
    o = torch.empty(T, Hv, D, dtype=d["v"].dtype, device=d["v"].device)
    o, S_T, states = G.forward(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o=o)
    res = dict(o=o, S_T=S_T)
    if backward:
        grads = dict(dq=d["dq"], dk=d["dk"], dv=d["dv"],
                     dg=torch.empty(T, Hv, dtype=torch.float32, device=o.device),
                     dbeta=torch.empty(T, Hv, dtype=torch.float32, device=o.device),
                     dS0=torch.empty(case.N, Hv, D, D, dtype=torch.float32, device=o.device))
        G.backward(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], states, d["dO"], d["dST"], grads=grads)
        res.update(grads)
    torch.cuda.synchronize()
    out = {}
    for name, t in res.items():
        a = t.float().cpu().numpy().astype(np.float64)
        if name in ("o", "dv"):
            a = a.reshape(T, Hv, D)
        elif name in ("dq", "dk"):
            a = a.reshape(T, Hk, D)
        out[name] = a
    return out


def compare(case, gpu, ref, names, tol=None, report=None):
    """Per-tensor normwise error of gpu vs oracle on the oracle's (possibly sampled)
    rows and heads. Returns {name: err}; asserts each below tol."""
    tol = tol_of(case) if tol is None else tol
    rows, vheads, kheads, seqs = ref["rows"], ref["vheads"], ref["key_heads"], ref["seqs"]
    errs = {}
    for name in names:
        g = gpu[name]
        if name in ("o", "dv", "dg", "dbeta"):
            g = g[rows][:, vheads]
        elif name in ("dq", "dk"):
            g = g[rows][:, kheads]
        elif name in ("S_T", "dS0"):
            g = g[seqs][:, vheads]
        errs[name] = normwise(g, ref[name])
    if report is not None:
        report.update(errs)
    bad = {k: v for k, v in errs.items() if not v < tol}
    assert not bad, f"{case.name}: normwise errors above {tol}: {bad} (all: {errs})"
    return errs
