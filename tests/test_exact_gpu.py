"""GPU structural exactness and determinism (HIP path vs itself, bit for bit).

* varlen-packed (cu_seqlens) equals per-sequence calls, on every output;
* strided row views of a packed projection equal contiguous copies;
* v_repeat = r equals explicit replication of q/k (r = 1): o, S_T, dv, dg, dbeta and dS0
  bit-identical; dq/dk, which the library folds in float32 before one rounding,
  within tolerance of the host-side sum of the replicated heads;
* two runs are bit-identical (no atomics anywhere);
* split resume at a chunk boundary: [0, m) then [m, T) with S0 = S_m equals the whole run;
* the forward runs without a workspace, and the backward's outputs do not depend on what
  its workspace holds on entry.
"""
import numpy as np
import pytest

import oracle
from synth import make_case
from gdn_gpu import GRAD_NAMES, normwise, run_gpu

pytestmark = pytest.mark.gpu

ALL = ("o", "S_T") + GRAD_NAMES


def _case(lens, Hk=2, Hv=6, D=64, dtype="bf16", chunk=64, varlen=False, packed=True, seed=77):
    return make_case(seed, lens, Hk, Hv, D, dtype=dtype, chunk=chunk, gate="clamp09", with_S0=True,
                     with_dST=True, packed=packed, varlen=varlen, name=f"exact{lens}")


def _sub(case, n):
    """Sequence n of a case as its own single-sequence case."""
    import copy

    cu = case.cu_seqlens
    a, b = cu[n], cu[n + 1]
    c = copy.copy(case)
    c.lens = [int(b - a)]
    c.varlen = False
    for name in ("q", "k", "v", "g", "beta", "dO"):
        setattr(c, name, getattr(case, name)[a:b])
    c.S0 = case.S0[n:n + 1]
    c.dST = case.dST[n:n + 1]
    return c


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_equals_per_sequence(dtype):
    case = _case([70, 0, 129, 64, 5], dtype=dtype, varlen=True, D=64 if dtype == "bf16" else 32)
    full = run_gpu(case)
    cu = case.cu_seqlens
    for n in range(case.N):
        if case.lens[n] == 0:
            assert np.array_equal(full["S_T"][n], case.S0[n])
            assert np.array_equal(full["dS0"][n], case.dST[n])
            continue
        one = run_gpu(_sub(case, n))
        rows = slice(cu[n], cu[n + 1])
        for name in ("o", "dq", "dk", "dv", "dg", "dbeta"):
            assert np.array_equal(full[name][rows], one[name]), (n, name)
        for name in ("S_T", "dS0"):
            assert np.array_equal(full[name][n], one[name][0]), (n, name)


def test_strided_equals_contiguous():
    case = _case([150, 150])
    a = run_gpu(case, packed=True)
    b = run_gpu(case, packed=False)
    for name in ALL:
        assert np.array_equal(a[name], b[name]), name


def test_vrepeat_equals_replication():
    case = _case([140], Hk=2, Hv=6)
    r = case.Hv // case.Hk
    heads = np.arange(case.Hv) // r
    import copy

    rep = copy.copy(case)
    rep.Hk = case.Hv
    rep.q = case.q[:, heads]
    rep.k = case.k[:, heads]
    a = run_gpu(case)
    b = run_gpu(rep)
    for name in ("o", "S_T", "dv", "dg", "dbeta", "dS0"):
        assert np.array_equal(a[name], b[name]), name
    for name in ("dq", "dk"):
        folded = np.zeros_like(a[name])
        for h in range(case.Hv):
            folded[:, h // r] += b[name][:, h]
        assert normwise(a[name], folded) < 1e-2, name


def test_determinism_bitwise():
    case = _case([300, 300], Hk=2, Hv=6, D=128)
    a = run_gpu(case)
    b = run_gpu(case)
    for name in ALL:
        assert np.array_equal(a[name], b[name]), name


def test_split_resume_at_chunk_boundary():
    import copy

    case = _case([256], Hk=1, Hv=3, D=32, dtype="f32")
    full = run_gpu(case)
    m = 128
    first, second = copy.copy(case), copy.copy(case)
    first.lens, second.lens = [m], [256 - m]
    for name in ("q", "k", "v", "g", "beta", "dO"):
        setattr(first, name, getattr(case, name)[:m])
        setattr(second, name, getattr(case, name)[m:])
    a = run_gpu(first, backward=False)
    second.S0 = a["S_T"]
    b = run_gpu(second)
    first.dST = b["dS0"]
    a = run_gpu(first)
    assert np.array_equal(np.concatenate([a["o"], b["o"]]), full["o"])
    assert np.array_equal(b["S_T"], full["S_T"])
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.array_equal(np.concatenate([a[name], b[name]]), full[name]), name
    assert np.array_equal(a["dS0"], full["dS0"])


def test_workspace_contents_ignored():
    """A forward that saves chunk states takes no workspace (NULL is accepted: its chunk table
    is saved with the states; only a forward-only call needs one); the backward's outputs do
    not depend on what its workspace holds on entry (zero bytes against all-one bytes, NaN in
    both storage types): bit-identical."""
    import torch
    import gated_delta_rule_34_amd as G
    from gdn_gpu import problem, to_device

    case = _case([200, 77], Hk=2, Hv=6, D=128, varlen=True)
    d = to_device(case)
    p = problem(case, d, None)
    T, Hv, D, dev = case.T_total, case.Hv, case.Dk, d["v"].device
    o = torch.empty(T, Hv, D, dtype=d["v"].dtype, device=dev)
    S_T = torch.empty(case.N, Hv, D, D, dtype=torch.float32, device=dev)
    states = torch.empty(G.gdn_chunk_state_bytes(p), dtype=torch.uint8, device=dev)
    G.gdn_fwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, S_T, states, None)
    runs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((G.gdn_bwd_workspace_bytes(p),), fill, dtype=torch.uint8, device=dev)
        dg = torch.empty(T, Hv, dtype=torch.float32, device=dev)
        dbeta = torch.empty_like(dg)
        dS0 = torch.empty(case.N, Hv, D, D, dtype=torch.float32, device=dev)
        G.gdn_bwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], states, d["dO"], d["dST"], d["dq"],
                  d["dk"], d["dv"], dg, dbeta, dS0, ws)
        torch.cuda.synchronize()
        runs.append({name: t.clone() for name, t in
                     dict(dq=d["dq"], dk=d["dk"], dv=d["dv"], dg=dg, dbeta=dbeta, dS0=dS0).items()})
    for name, t in runs[0].items():
        assert torch.isfinite(t.float()).all(), name
        assert torch.equal(t, runs[1][name]), name


def test_fused_prologue_determinism_bitwise():
    """With the q/k L2 norm and the gate chain fused (raw rows scaled per row, alpha and
    beta_raw), two runs are bit-identical on every output."""
    import dataclasses

    import torch
    from gdn_gpu import problem, to_device
    from synth import round_bf16, round_f32

    base = _case([300, 77], Hk=2, Hv=6, D=128, varlen=True)
    rng = np.random.default_rng(31)
    s = lambda: rng.uniform(0.2, 5.0, (base.T_total, base.Hk, 1))
    case = dataclasses.replace(base, q=round_bf16(base.q * s()), k=round_bf16(base.k * s()),
                               g=round_f32(rng.standard_normal((base.T_total, base.Hv))),
                               beta=round_f32(rng.standard_normal((base.T_total, base.Hv))))
    outs = []
    for _ in range(2):
        d = to_device(case)
        dev = d["v"].device
        a_log = torch.full((case.Hv,), -0.4, dtype=torch.float32, device=dev)
        dt_bias = torch.full((case.Hv,), 0.6, dtype=torch.float32, device=dev)
        p = problem(case, d)
        p.qk_l2norm, p.a_log, p.dt_bias = 1, a_log.data_ptr(), dt_bias.data_ptr()
        outs.append(run_gpu(case, d=d, p=p))
    for name in ALL:
        assert np.array_equal(outs[0][name], outs[1][name]), name


@pytest.mark.parametrize("lens,dtype", [([0], "f32"), ([0, 0, 0], "bf16")])
def test_all_sequences_empty(lens, dtype):
    """A batch whose sequences are all empty: no chunk slot at all ([0]: the chunk table then
    comes from its own one-workgroup kernel) or only unused slots ([0, 0, 0]: prep runs and
    writes an empty table). Nothing is read or written per token; the final state is S0 and
    the state gradient is dS_T, bit for bit, as the oracle has them."""
    case = make_case(7, lens, 2, 4, 32, dtype=dtype, chunk=64, gate="clamp09", with_S0=True, with_dST=True,
                     packed=(dtype == "bf16"), varlen=True, name="all_empty")
    gpu = run_gpu(case)
    ref = oracle.run_case(case, backward=True)
    assert gpu["o"].shape[0] == 0 and gpu["dq"].shape[0] == 0
    assert np.array_equal(gpu["S_T"], ref["S_T"])
    assert np.array_equal(gpu["dS0"], ref["dS0"])
    assert np.array_equal(ref["S_T"], np.asarray(case.S0, dtype=np.float64))
