"""Device placement of a seeded case (``synth.GdnCase``) for the HIP library's binding.

Marshalling only: it copies the case's already-rounded arrays to the GPU in the layout the
workload uses (one packed [T, 2 Hk Dk + Hv Dv] projection buffer with q, k, v as row views,
or contiguous tensors) and builds the matching ``gdn_problem``. It holds none of the
recurrence's arithmetic, so the tests and the benchmark share it without sharing anything
with the oracle.
"""
from __future__ import annotations

import numpy as np


def to_device(case, device="cuda", packed=None):
    """Device tensors for a case. Packed workloads get one [T, 2*Hk*Dk + Hv*Dv] buffer with
    q, k, v as row views; dq/dk/dv are views into one packed gradient buffer too."""
    import torch

    dt = torch.float32 if case.dtype == "f32" else torch.bfloat16
    packed = case.packed if packed is None else packed
    T, Hk, Hv, D = case.T_total, case.Hk, case.Hv, case.Dk

    def tt(a, dtype=torch.float32):
        if a is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32).to(dtype).to(device)

    d = {}
    if packed:
        width = 2 * Hk * D + Hv * D
        buf = torch.empty(T, width, dtype=dt, device=device)
        buf[:, : Hk * D] = tt(case.q.reshape(T, Hk * D), dt)
        buf[:, Hk * D: 2 * Hk * D] = tt(case.k.reshape(T, Hk * D), dt)
        buf[:, 2 * Hk * D:] = tt(case.v.reshape(T, Hv * D), dt)
        d["packed"] = buf
        d["q"], d["k"], d["v"] = buf[:, : Hk * D], buf[:, Hk * D: 2 * Hk * D], buf[:, 2 * Hk * D:]
        gbuf = torch.empty(T, width, dtype=dt, device=device)
        d["gpacked"] = gbuf
        d["dq"], d["dk"], d["dv"] = gbuf[:, : Hk * D], gbuf[:, Hk * D: 2 * Hk * D], gbuf[:, 2 * Hk * D:]
    else:
        d["q"], d["k"], d["v"] = tt(case.q, dt), tt(case.k, dt), tt(case.v, dt)
        d["dq"] = torch.empty(T, Hk, D, dtype=dt, device=device)
        d["dk"] = torch.empty(T, Hk, D, dtype=dt, device=device)
        d["dv"] = torch.empty(T, Hv, D, dtype=dt, device=device)
    d["g"], d["beta"] = tt(case.g), tt(case.beta)
    d["S0"], d["dST"] = tt(case.S0), tt(case.dST)
    d["dO"] = tt(case.dO, dt)
    d["cu"] = torch.tensor(case.cu_seqlens, dtype=torch.int32, device=device) if case.varlen else None
    return d


def problem(case, d, chunk=None):
    """The gdn_problem of a case placed by ``to_device``."""
    import gated_delta_rule_34_amd as G

    if case.varlen:
        return G.make_problem(case.N, case.T_total, case.Hk, case.Hv, case.Dk, cu_seqlens=d["cu"],
                              chunk=chunk or case.chunk, scale=case.scale, dtype=case.dtype)
    T = case.lens[0] if case.N else 0
    assert all(L == T for L in case.lens)
    return G.make_problem(case.N, case.T_total, case.Hk, case.Hv, case.Dk, T=T, chunk=chunk or case.chunk,
                          scale=case.scale, dtype=case.dtype)
