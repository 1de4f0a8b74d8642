"""GPU parity at large offsets: two sequences of 131072 tokens at the training heads
(Hk 16 / Hv 48 / D 128, bf16 packed q/k/v rows: 262144 rows, 5.4 GB of projection, saved
chunk states past 3 GB), so that row, chunk-state and workspace offsets pass 2^31 bytes.

* Prefixes against the oracle: dO is nonzero on the first 4096 rows of each sequence only
  (and dS_T = 0), so no loss term depends on later rows and the outputs and gradients of
  those rows are exactly those of the 4096-row prefix alone, which the oracle computes
  (three key-head groups). The second sequence's prefix starts at row 131072.
* The long range by consistency: the second half of sequence 2 run as its own problem
  from the state the first half ends in (row offsets from 0) equals the full run's rows
  131072 + 65536 .. 262143 bit for bit, o and final state.
Inputs are drawn on the device (seeded): q, k L2-normalised per head, v N(0, 1), g in
[0.9, 1], beta in [0, 1], S0 = 0.
"""
import numpy as np
import pytest

import oracle
from gdn_gpu import normwise

pytestmark = pytest.mark.gpu

TOL = 2e-2


def test_large_offsets_prefixes_and_split():
    import torch
    import gated_delta_rule_34_amd as G

    N, T, Hk, Hv, D, P = 2, 131072, 16, 48, 128, 4096
    R, r = N * T, Hv // Hk
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(2024)
    width = 2 * Hk * D + Hv * D
    buf = torch.empty(R, width, dtype=torch.bfloat16, device=dev)
    for lo in (0, Hk * D):
        x = torch.randn(R, Hk, D, device=dev, generator=gen)
        buf[:, lo:lo + Hk * D] = torch.nn.functional.normalize(x, dim=-1).reshape(R, -1).to(torch.bfloat16)
        del x
    buf[:, 2 * Hk * D:] = torch.randn(R, Hv * D, device=dev, generator=gen).to(torch.bfloat16)
    q, k, v = buf[:, : Hk * D], buf[:, Hk * D: 2 * Hk * D], buf[:, 2 * Hk * D:]
    g = 0.9 + 0.1 * torch.rand(R, Hv, device=dev, generator=gen)
    beta = torch.rand(R, Hv, device=dev, generator=gen)
    dO = torch.zeros(R, Hv * D, dtype=torch.bfloat16, device=dev)
    for n in range(N):
        dO[n * T: n * T + P] = torch.randn(P, Hv * D, device=dev, generator=gen).to(torch.bfloat16)
    print("[large] inputs ready", flush=True)

    p = G.make_problem(N, R, Hk, Hv, D, T=T, dtype="bf16")
    o, S_T, states = G.forward(p, q, k, v, g, beta, None)
    grads = G.backward(p, q, k, v, g, beta, None, states, dO, None, want_dS0=False)
    torch.cuda.synchronize()
    print("[large] forward and backward done", flush=True)

    # prefixes against the oracle
    khs = [0, 7, 15]
    vhs = [kh * r + j for kh in khs for j in range(r)]
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    for n in range(N):
        rows = slice(n * T, n * T + P)
        qn = f64(q[rows]).reshape(P, Hk, D)[:, khs]
        kn = f64(k[rows]).reshape(P, Hk, D)[:, khs]
        vn = f64(v[rows]).reshape(P, Hv, D)[:, vhs]
        gn, bn = f64(g[rows])[:, vhs], f64(beta[rows])[:, vhs]
        dOn = f64(dO[rows]).reshape(P, Hv, D)[:, vhs]
        cu = np.array([0, P], dtype=np.int64)
        o_ref, _ = oracle.gdn_fwd(cu, qn, kn, vn, gn, bn, None, p.scale)
        gr = oracle.gdn_bwd(cu, qn, kn, vn, gn, bn, None, dOn, None, p.scale)
        got = dict(o=f64(o[rows]).reshape(P, Hv, D)[:, vhs], dv=f64(grads["dv"][rows])[:, vhs],
                   dq=f64(grads["dq"][rows])[:, khs], dk=f64(grads["dk"][rows])[:, khs],
                   dg=f64(grads["dg"][rows])[:, vhs], dbeta=f64(grads["dbeta"][rows])[:, vhs])
        ref = dict(o=o_ref, **{name: gr[name] for name in ("dv", "dq", "dk", "dg", "dbeta")})
        errs = {name: normwise(got[name], ref[name]) for name in got}
        print(f"[large] sequence {n} prefix errors {errs}", flush=True)
        assert all(e < TOL for e in errs.values()), (n, errs)

    # the second half of sequence 2 from the state its first half ends in
    half = T // 2
    a0, a1 = T, T + half  # rows of the first half of sequence 2
    ph = G.make_problem(1, half, Hk, Hv, D, T=half, dtype="bf16")
    _, S_mid, _ = G.forward(ph, q[a0:a1], k[a0:a1], v[a0:a1], g[a0:a1], beta[a0:a1], None)
    o2, S_end, _ = G.forward(ph, q[a1:R], k[a1:R], v[a1:R], g[a1:R], beta[a1:R], S_mid)
    torch.cuda.synchronize()
    assert torch.equal(o2.reshape(half, -1), o[a1:R].reshape(half, -1))
    assert torch.equal(S_end[0], S_T[1])
    assert torch.isfinite(o.float()).all() and torch.isfinite(S_T).all()
