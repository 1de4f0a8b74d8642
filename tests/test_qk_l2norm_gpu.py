"""GPU parity of the fused q/k L2 normalisation (gdn_problem.qk_l2norm): the kernels take
raw q, k rows, normalise every head row as x / sqrt(sum x^2 + 1e-6) themselves, and the
backward returns the gradients of the raw rows. Reference: oracle.l2norm_rows feeding the
oracle's recurrence, and oracle.l2norm_rows_grad on its dq, dk. Also with the gate chain
fused at the same time, and in the decode step.

Inputs: synth's (seeded) normalised q, k rows scaled per head row by U(0.2, 5) (and
rounded to the storage type), so that the kernels' normalisation is not the identity.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from synth import make_case, round_bf16, round_f32
from gdn_gpu import GRAD_NAMES, OUT_NAMES, compare, normwise, problem, run_gpu, to_device

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_ragged_r3_D128": dict(lens=[130, 67], Hk=2, Hv=6, D=128, dtype="bf16", chunk=64, varlen=True),
    "f32_D32_C16": dict(lens=[100], Hk=1, Hv=2, D=32, dtype="f32", chunk=16, varlen=False),
    "f32_D16_C64_two_seqs": dict(lens=[40, 40], Hk=2, Hv=4, D=16, dtype="f32", chunk=64, varlen=False),
    # bf16 at the small head sizes: two and eight lanes per row in the row dots of the norm's
    # backward
    "bf16_D16_C64": dict(lens=[90], Hk=2, Hv=4, D=16, dtype="bf16", chunk=64, varlen=False),
    "bf16_D64_C16_varlen": dict(lens=[33, 0, 70], Hk=1, Hv=3, D=64, dtype="bf16", chunk=16, varlen=True),
}
SMALL = list(CASES)
# the training shape (4 x 4096 tokens, 16 key heads, 48 value heads, D = 128, bf16 packed rows)
CASES["bf16_training_shape"] = dict(lens=[4096] * 4, Hk=16, Hv=48, D=128, dtype="bf16", chunk=64, varlen=False)


def _raw(case, seed):
    rng = np.random.default_rng(seed)
    rnd = round_bf16 if case.dtype == "bf16" else round_f32
    s = lambda: rng.uniform(0.2, 5.0, (case.T_total, case.Hk, 1))
    return rnd(case.q * s()), rnd(case.k * s())


def _run(name, chain):
    import torch

    kw = CASES[name]
    base = make_case(700 + len(name), kw["lens"], kw["Hk"], kw["Hv"], kw["D"], dtype=kw["dtype"], chunk=kw["chunk"],
                     gate="raw", with_S0=True, with_dST=True, packed=True, varlen=kw["varlen"], name=name)
    q_raw, k_raw = _raw(base, 3)
    q_hat, rq = oracle.l2norm_rows(q_raw)
    k_hat, rk = oracle.l2norm_rows(k_raw)
    case = dataclasses.replace(base, q=q_hat, k=k_hat)
    if chain:
        rng = np.random.default_rng(5)
        T, Hv = base.T_total, base.Hv
        alpha, beta_raw = round_f32(rng.standard_normal((T, Hv))), round_f32(rng.standard_normal((T, Hv)))
        a_log, dt_bias = round_f32(rng.uniform(-1, 0, Hv)), round_f32(rng.uniform(0, 1, Hv))
        g, beta = oracle.gate_chain(alpha, a_log, dt_bias, beta_raw)
        case = dataclasses.replace(case, g=g, beta=beta)
    ref = oracle.run_case(case)
    ref["dq"] = oracle.l2norm_rows_grad(q_hat, rq, ref["dq"])
    ref["dk"] = oracle.l2norm_rows_grad(k_hat, rk, ref["dk"])
    raw = dataclasses.replace(case, q=q_raw, k=k_raw)
    d = to_device(raw)
    p = problem(raw, d)
    p.qk_l2norm = 1
    keep = []
    if chain:
        ref["dg"], ref["dbeta"] = oracle.gate_chain_grads(alpha, a_log, dt_bias, beta_raw, ref["dg"], ref["dbeta"])
        dev = d["v"].device
        d["g"] = torch.from_numpy(alpha).float().to(dev)
        d["beta"] = torch.from_numpy(beta_raw).float().to(dev)
        keep = [torch.from_numpy(a_log).float().to(dev), torch.from_numpy(dt_bias).float().to(dev)]
        p.a_log, p.dt_bias = keep[0].data_ptr(), keep[1].data_ptr()
    gpu = run_gpu(raw, d=d, p=p)
    compare(raw, gpu, ref, OUT_NAMES + GRAD_NAMES)


@pytest.mark.parametrize("name", SMALL)
def test_qk_l2norm_fused(name):
    _run(name, chain=False)


def test_qk_l2norm_and_gate_chain_fused():
    _run("bf16_ragged_r3_D128", chain=True)


def test_qk_l2norm_and_gate_chain_fused_training_shape():
    """Both fused prologues at the shape the bench times them, every element of every output
    and gradient against the oracle."""
    _run("bf16_training_shape", chain=True)


def test_qk_l2norm_decode():
    import torch
    import gated_delta_rule_34_amd as G

    rng = np.random.default_rng(21)
    N, Hk, Hv, D = 24, 2, 6, 128
    q = round_f32(rng.standard_normal((N, Hk, D)) * 2)
    k = round_f32(rng.standard_normal((N, Hk, D)) * 0.5)
    v = round_f32(rng.standard_normal((N, Hv, D)))
    g = round_f32(rng.uniform(0.5, 1.0, (N, Hv)))
    beta = round_f32(rng.uniform(0.0, 1.0, (N, Hv)))
    state = round_f32(0.3 * rng.standard_normal((N, Hv, D, D)))
    o_ref, st_ref = oracle.gdn_decode(oracle.l2norm_rows(q)[0], oracle.l2norm_rows(k)[0], v, g, beta, state)
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).float().to(dev)
    st = t(state)
    o = torch.empty(N, Hv, D, dtype=torch.float32, device=dev)
    p = G.make_problem(N, N, Hk, Hv, D, T=1, dtype="f32", qk_l2norm=True)
    G.gdn_decode(p, t(q), t(k), t(v), t(g), t(beta), st, None, o)
    torch.cuda.synchronize()
    assert normwise(o.cpu().numpy(), o_ref) < 2e-4
    assert normwise(st.cpu().numpy(), st_ref) < 2e-4
