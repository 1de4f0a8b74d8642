"""Pins of the float64 oracle to things other than itself (CPU only).

Each test ties the oracle to a fact fixed by the mathematics of the recurrence
(lattice-inference 0.6.0, src/attention/gdn_backward.rs, "Forward recap" and
gdn_backward steps 4a-4d), chosen so a plausible slip -- a dropped term, a wrong
sign or index, a transposed operand, a wrong head map -- fails at least one:

* central finite differences of the oracle's own forward for every gradient
  (the check the dormouse KDA log uses: f64 loss, derived step size, the smaller
  of the errors at h and h/10, normwise max|a-b|/max|b|);
* a second formulation of the recurrence (the Householder form
  S_t = g (I - beta k k^T) S_{t-1} + beta k v^T) in torch float64, with gradients by
  autograd, not by the oracle's hand-derived backward;
* closed forms: beta = 0 (pure decay of S0), T = 1, and g = beta = 1 with orthonormal
  keys (the delta rule writes v exactly);
* v_repeat = r equals explicit replication of q/k with dq/dk summed over the group
  (the asymmetric-heads source-parity idea of the lattice-inference tests);
* zero upstream gradient gives exactly zero gradients (same page's gradcheck tests);
* linearity in V and in S0, split-sequence resume, zero-length sequences;
* falsification: builds of the oracle with a planted mistake must fail a pin.
"""
import json
import os
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import make_case


def normwise(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b)) if b.size else 0.0
    num = np.max(np.abs(a - b)) if a.size else 0.0
    return num / den if den > 0 else num


def small_case(seed, lens, Hk, Hv, D, s0=True, dst=True, gate="raw"):
    return make_case(seed, lens, Hk, Hv, D, dtype="f32", chunk=16, gate=gate,
                     with_S0=s0, with_dST=dst)


def loss_of(case, lib=None, **over):
    arrs = dict(q=case.q, k=case.k, v=case.v, g=case.g, beta=case.beta, S0=case.S0)
    arrs.update(over)
    o, ST = oracle.gdn_fwd(case.cu_seqlens, arrs["q"], arrs["k"], arrs["v"], arrs["g"],
                           arrs["beta"], arrs["S0"], case.scale, nthreads=1, lib=lib)
    L = float(np.sum(case.dO * o))
    if case.dST is not None:
        L += float(np.sum(case.dST * ST))
    return L


def fd_check(case, lib=None, max_coords=48, seed=0):
    """Return {tensor: normwise error} of the oracle backward vs central differences."""
    grads = oracle.gdn_bwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0,
                           case.dO, case.dST, case.scale, nthreads=1, lib=lib)
    L0 = loss_of(case, lib)
    eps = np.finfo(np.float64).eps
    rng = np.random.default_rng(seed)
    errs = {}
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta")]
    if case.S0 is not None:
        names.append(("S0", "dS0"))
    for name, gname in names:
        x = getattr(case, name)
        an = grads[gname]
        gmax = max(np.max(np.abs(an)), 1e-30)
        h0 = (3.0 * eps * max(abs(L0), 1.0) / gmax) ** (1.0 / 3.0)
        idx = np.arange(x.size)
        if x.size > max_coords:
            idx = rng.choice(x.size, size=max_coords, replace=False)
        best = np.inf
        for h in (h0, h0 / 10):
            fd = np.empty(len(idx))
            for c, i in enumerate(idx):
                xp = x.copy().reshape(-1)
                xm = x.copy().reshape(-1)
                xp[i] += h
                xm[i] -= h
                fd[c] = (loss_of(case, lib, **{name: xp.reshape(x.shape)})
                         - loss_of(case, lib, **{name: xm.reshape(x.shape)})) / (2 * h)
            best = min(best, normwise(an.reshape(-1)[idx], fd))
        errs[gname] = best
    return errs


FD_SHAPES = [
    # (lens, Hk, Hv, D)
    ([9], 1, 1, 4),
    ([7, 12], 1, 2, 4),
    ([16], 2, 6, 8),
    ([5, 0, 11], 2, 4, 8),
    ([24], 1, 3, 16),
]


@pytest.mark.parametrize("shape", FD_SHAPES, ids=lambda s: f"lens{s[0]}_Hk{s[1]}_Hv{s[2]}_D{s[3]}")
def test_fd_all_gradients(oracle_lib, shape):
    lens, Hk, Hv, D = shape
    case = small_case(7 + sum(lens), lens, Hk, Hv, D)
    errs = fd_check(case)
    for name, e in errs.items():
        assert e < 1e-6, f"{name}: FD normwise error {e:.3e}"


def householder_torch(case):
    """Second formulation, torch float64 autograd: S_t = g (S - beta k (k^T S)) + beta k v^T."""
    import torch

    t = lambda a: None if a is None else torch.tensor(a, dtype=torch.float64, requires_grad=True)
    q, k, v, g, beta = map(t, (case.q, case.k, case.v, case.g, case.beta))
    S0 = t(case.S0)
    r = case.Hv // case.Hk
    heads = torch.arange(case.Hv) // r
    cu = case.cu_seqlens
    outs, finals = [], []
    for n in range(case.N):
        if S0 is not None:
            S = S0[n]
        else:
            S = torch.zeros(case.Hv, case.Dk, case.Dv, dtype=torch.float64)
        for tt in range(cu[n], cu[n + 1]):
            kt = k[tt][heads]  # [Hv, Dk]
            qt = q[tt][heads]
            bt = beta[tt][:, None, None]
            gt = g[tt][:, None, None]
            kS = torch.einsum("hi,hij->hj", kt, S)
            S = gt * (S - bt * kt[:, :, None] * kS[:, None, :]) + bt * kt[:, :, None] * v[tt][:, None, :]
            outs.append(case.scale * torch.einsum("hij,hi->hj", S, qt))
        finals.append(S)
    o = torch.stack(outs) if outs else torch.zeros(0, case.Hv, case.Dv, dtype=torch.float64)
    ST = torch.stack(finals)
    L = (o * torch.tensor(case.dO)).sum()
    if case.dST is not None:
        L = L + (ST * torch.tensor(case.dST)).sum()
    L.backward()
    grads = dict(dq=q.grad, dk=k.grad, dv=v.grad, dg=g.grad, dbeta=beta.grad,
                 dS0=None if S0 is None else S0.grad)
    return o.detach().numpy(), ST.detach().numpy(), {a: None if b is None else b.numpy() for a, b in grads.items()}


@pytest.mark.parametrize("shape", [([20], 2, 4, 8), ([6, 17], 1, 3, 4), ([33], 2, 2, 16)],
                         ids=["r2", "r3_two_seqs", "r1"])
@pytest.mark.parametrize("s0", [False, True])
def test_householder_form_and_autograd(oracle_lib, shape, s0):
    lens, Hk, Hv, D = shape
    case = small_case(11 + D, lens, Hk, Hv, D, s0=s0, dst=s0)
    o_ref, ST_ref, g_ref = householder_torch(case)
    o, ST = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0, case.scale)
    assert normwise(o, o_ref) < 1e-13
    assert normwise(ST, ST_ref) < 1e-13
    gr = oracle.gdn_bwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0,
                        case.dO, case.dST, case.scale)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert normwise(gr[name], g_ref[name]) < 1e-12, name
    if s0:
        assert normwise(gr["dS0"], g_ref["dS0"]) < 1e-12


def test_beta_zero_is_pure_decay(oracle_lib):
    case = small_case(3, [13, 5], 2, 4, 8, s0=True, dst=True)
    case.beta[:] = 0.0
    o, ST = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0, case.scale)
    r = case.Hv // case.Hk
    cu = case.cu_seqlens
    for n in range(case.N):
        decay = np.ones(case.Hv)
        for t in range(cu[n], cu[n + 1]):
            decay = decay * case.g[t]
            for h in range(case.Hv):
                expect = case.scale * decay[h] * case.S0[n, h].T @ case.q[t, h // r]
                np.testing.assert_allclose(o[t, h], expect, rtol=1e-13, atol=1e-15)
        for h in range(case.Hv):
            np.testing.assert_allclose(ST[n, h], decay[h] * case.S0[n, h], rtol=1e-13, atol=1e-16)
    gr = oracle.gdn_bwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0,
                        case.dO, case.dST, case.scale)
    assert np.all(gr["dv"] == 0.0)


@pytest.mark.parametrize("s0", [False, True])
def test_unit_gate_orthonormal_keys_write_v(oracle_lib, s0):
    """g = beta = 1 and orthonormal keys: S_T^T k_r = v_r for every written key, and with
    q_t = k_t the output is scale * v_t exactly (the delta rule overwrites the slot)."""
    D, T = 8, 8
    rng = np.random.default_rng(5)
    Qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
    case = small_case(5, [T], 1, 2, D, s0=s0, dst=False)
    case.k[:, 0, :] = Qm.T[:T]
    case.q[:, 0, :] = Qm.T[:T]
    case.g[:] = 1.0
    case.beta[:] = 1.0
    o, ST = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0, case.scale)
    for h in range(case.Hv):
        for t in range(T):
            np.testing.assert_allclose(ST[0, h].T @ case.k[t, 0], case.v[t, h], rtol=0, atol=1e-13)
            np.testing.assert_allclose(o[t, h], case.scale * case.v[t, h], rtol=0, atol=1e-13)


def test_single_token_closed_form(oracle_lib):
    case = small_case(17, [1], 1, 1, 8, s0=True, dst=True)
    q, k, v = case.q[0, 0], case.k[0, 0], case.v[0, 0]
    g, b = case.g[0, 0], case.beta[0, 0]
    S0, dST, dO, sc = case.S0[0, 0], case.dST[0, 0], case.dO[0, 0], case.scale
    delta = b * (v - g * (S0.T @ k))
    S1 = g * S0 + np.outer(k, delta)
    o_ref = sc * S1.T @ q
    o, ST = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0, sc)
    np.testing.assert_allclose(o[0, 0], o_ref, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(ST[0, 0], S1, rtol=1e-14, atol=1e-16)
    # hand derivation of L = <dO, o> + <dS_T, S_1>
    dS1 = dST + sc * np.outer(q, dO)
    dq = sc * S1 @ dO
    dd = dS1.T @ k
    dk = dS1 @ delta - g * b * (S0 @ dd)
    dv = b * dd
    dbeta = (v - g * (S0.T @ k)) @ dd
    dg = np.sum(S0 * dS1) - b * (S0.T @ k) @ dd
    dS0 = g * dS1 - g * b * np.outer(k, dd)
    gr = oracle.gdn_bwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0,
                        case.dO, case.dST, sc)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv), ("dS0", dS0)):
        np.testing.assert_allclose(gr[name].reshape(ref.shape), ref, rtol=1e-12, atol=1e-14, err_msg=name)
    np.testing.assert_allclose(gr["dbeta"][0, 0], dbeta, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gr["dg"][0, 0], dg, rtol=1e-12, atol=1e-14)


def test_vrepeat_equals_replication(oracle_lib):
    case = small_case(23, [10, 19], 2, 6, 8, s0=True, dst=True)
    r = case.Hv // case.Hk
    heads = np.arange(case.Hv) // r
    o, ST = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0, case.scale)
    qr, kr = case.q[:, heads], case.k[:, heads]
    o2, ST2 = oracle.gdn_fwd(case.cu_seqlens, qr, kr, case.v, case.g, case.beta, case.S0, case.scale)
    assert np.array_equal(o, o2) and np.array_equal(ST, ST2)
    g1 = oracle.gdn_bwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0,
                        case.dO, case.dST, case.scale)
    g2 = oracle.gdn_bwd(case.cu_seqlens, qr, kr, case.v, case.g, case.beta, case.S0,
                        case.dO, case.dST, case.scale)
    for name in ("dv", "dg", "dbeta", "dS0"):
        assert np.array_equal(g1[name], g2[name]), name
    for name in ("dq", "dk"):
        folded = np.zeros_like(g1[name])
        for h in range(case.Hv):  # ascending head order, as the fold adds them
            folded[:, h // r] += g2[name][:, h]
        assert np.array_equal(g1[name], folded), name


def test_zero_upstream_gives_zero_gradients(oracle_lib):
    case = small_case(29, [14, 3], 2, 4, 8, s0=True, dst=False)
    case.dO[:] = 0.0
    gr = oracle.gdn_bwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0,
                        case.dO, None, case.scale)
    for name, a in gr.items():
        assert np.all(a == 0.0), name


def test_linearity_in_v_and_s0(oracle_lib):
    case = small_case(31, [21], 1, 2, 8, s0=True, dst=False)
    o1, S1 = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, None, case.scale)
    o2, S2 = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, 0.37 * case.v, case.g, case.beta, None, case.scale)
    np.testing.assert_allclose(o2, 0.37 * o1, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(S2, 0.37 * S1, rtol=1e-12, atol=1e-15)
    zero_v = np.zeros_like(case.v)
    oa, _ = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, zero_v, case.g, case.beta, case.S0, case.scale)
    ob, _ = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, zero_v, case.g, case.beta, -2.5 * case.S0, case.scale)
    np.testing.assert_allclose(ob, -2.5 * oa, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("m", [1, 37, 64, 70])
def test_split_resume(oracle_lib, m):
    T = 100
    case = small_case(37, [T], 1, 2, 8, s0=True, dst=True)
    full_o, full_ST = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0, case.scale)
    full = oracle.gdn_bwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0,
                          case.dO, case.dST, case.scale)
    a, b = slice(0, m), slice(m, T)
    cu_a, cu_b = np.array([0, m]), np.array([0, T - m])
    oa, Sm = oracle.gdn_fwd(cu_a, case.q[a], case.k[a], case.v[a], case.g[a], case.beta[a], case.S0, case.scale)
    ob, ST = oracle.gdn_fwd(cu_b, case.q[b], case.k[b], case.v[b], case.g[b], case.beta[b], Sm, case.scale)
    assert np.array_equal(np.concatenate([oa, ob]), full_o)
    assert np.array_equal(ST, full_ST)
    gb = oracle.gdn_bwd(cu_b, case.q[b], case.k[b], case.v[b], case.g[b], case.beta[b], Sm,
                        case.dO[b], case.dST, case.scale)
    ga = oracle.gdn_bwd(cu_a, case.q[a], case.k[a], case.v[a], case.g[a], case.beta[a], case.S0,
                        case.dO[a], gb["dS0"], case.scale)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        np.testing.assert_allclose(np.concatenate([ga[name], gb[name]]), full[name], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ga["dS0"], full["dS0"], rtol=1e-12, atol=1e-14)


def test_zero_length_sequences(oracle_lib):
    case = small_case(41, [0, 6, 0], 1, 2, 4, s0=True, dst=True)
    o, ST = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0, case.scale)
    assert np.array_equal(ST[0], case.S0[0]) and np.array_equal(ST[2], case.S0[2])
    gr = oracle.gdn_bwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0,
                        case.dO, case.dST, case.scale)
    assert np.array_equal(gr["dS0"][0], case.dST[0]) and np.array_equal(gr["dS0"][2], case.dST[2])


def test_threads_do_not_change_results(oracle_lib):
    case = small_case(43, [40, 25, 33], 2, 6, 8, s0=True, dst=True)
    a = oracle.gdn_bwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0,
                       case.dO, case.dST, case.scale, nthreads=1)
    b = oracle.gdn_bwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0,
                       case.dO, case.dST, case.scale, nthreads=5)
    for name in a:
        assert np.array_equal(a[name], b[name]), name


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    """A hand-worked example: inputs and expected values as exact fractions."""
    with open(os.path.join(GOLDEN, name)) as f:
        fx = json.load(f)
    arr = lambda x: np.array(x, dtype=object).astype(str)
    num = lambda x: np.vectorize(lambda s: float(Fraction(s)))(arr(x)).astype(np.float64)
    ins = {k: num(v) for k, v in fx["inputs"].items()}
    exp = {k: num(v) for k, v in fx["expected"].items()}
    return fx, ins, exp


def _golden_errors(lib, name="scalar_state_two_heads.json"):
    """Largest absolute error of the oracle on a golden example, per output."""
    fx, x, e = _golden(name)
    cu = np.array(fx["cu_seqlens"], dtype=np.int64)
    sc = float(Fraction(fx["scale"]))
    o, ST = oracle.gdn_fwd(cu, x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], sc, lib=lib)
    gr = oracle.gdn_bwd(cu, x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], x["dO"], x["dS_T"], sc, lib=lib)
    got = dict(o=o, S_T=ST, **gr)
    return {k: float(np.max(np.abs(got[k] - e[k]))) for k in e}


def test_golden_hand_worked_example(oracle_lib):
    """tests/golden/scalar_state_two_heads.json: two tokens, Dk = Dv = 1, two value heads
    on one key head, every output derived by hand from the page's recurrence (the
    derivation is in the file). Exact in binary, so the oracle must match to rounding."""
    errs = _golden_errors(oracle.LIB)
    assert all(v < 1e-14 for v in errs.values()), errs


def test_decode_replays_the_hand_worked_example():
    """The decode step, called once per token with the state carried in its slot,
    reproduces the hand-worked example's o (token by token) and final state."""
    fx, x, e = _golden("scalar_state_two_heads.json")
    sc = float(Fraction(fx["scale"]))
    state = x["S0"].copy()
    for t in range(2):
        row = slice(t, t + 1)
        o, state = oracle.gdn_decode(x["q"][row], x["k"][row], x["v"][row], x["g"][row], x["beta"][row], state,
                                     None, sc)
        assert np.max(np.abs(o[0] - e["o"][t])) < 1e-14, t
    assert np.max(np.abs(state - e["S_T"])) < 1e-14


def test_decode_slot_map():
    """Decode rows reach their states through the slot map: each row equals a one-token
    forward from its slot; rows whose slot is outside [0, n_slots) are skipped (NaN o),
    and the slots no row names keep their values."""
    rng = np.random.default_rng(5)
    N, Hk, Hv, D, n_slots = 6, 2, 4, 8, 9
    q, k = rng.standard_normal((N, Hk, D)), rng.standard_normal((N, Hk, D)) / np.sqrt(D)
    v = rng.standard_normal((N, Hv, D))
    g, beta = rng.uniform(0.5, 1.0, (N, Hv)), rng.uniform(0.0, 1.0, (N, Hv))
    state = rng.standard_normal((n_slots, Hv, D, D))
    slots = np.array([7, 2, -1, 0, 9, 4])
    o, new = oracle.gdn_decode(q, k, v, g, beta, state, slots)
    one = np.array([0, 1], dtype=np.int64)
    for n in range(N):
        s_ = slots[n]
        if not 0 <= s_ < n_slots:
            assert np.isnan(o[n]).all()
            continue
        o1, st1 = oracle.gdn_fwd(one, q[n:n + 1], k[n:n + 1], v[n:n + 1], g[n:n + 1], beta[n:n + 1], state[s_:s_ + 1])
        assert np.array_equal(o[n], o1[0]) and np.array_equal(new[s_], st1[0]), n
    rest = [s_ for s_ in range(n_slots) if s_ not in (7, 2, 0, 4)]
    assert np.array_equal(new[rest], state[rest])


def _pins_fail(lib):
    """Run a cheap subset of the pins against an oracle build; return names that failed."""
    failed = []
    case = small_case(101, [12], 2, 4, 4, s0=True, dst=True)
    errs = fd_check(case, lib=lib, max_coords=16)
    if any(e > 1e-6 for e in errs.values()):
        failed.append("fd")
    o_ref, _, g_ref = householder_torch(case)
    o, _ = oracle.gdn_fwd(case.cu_seqlens, case.q, case.k, case.v, case.g, case.beta, case.S0,
                          case.scale, lib=lib)
    if normwise(o, o_ref) > 1e-12:
        failed.append("householder")
    if any(v > 1e-14 for v in _golden_errors(lib).values()):
        failed.append("golden")
    return failed


@pytest.mark.parametrize("plant", [1, 2, 3, 4],
                         ids=["modulo_head_map", "drop_dk_retrieval_term", "dg_sign", "dq_no_scale"])
def test_planted_mistake_is_caught(oracle_lib, plant):
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.build(os.path.join(d, f"liboracle_plant{plant}.so"), plant=plant)
        failed = _pins_fail(lib)
    assert failed, f"planted mistake {plant} passed every pin"


def test_unplanted_passes_the_same_pins(oracle_lib):
    assert _pins_fail(oracle.LIB) == []


# --- causal depthwise conv1d + SiLU (oracle/conv.py)

def _conv_case(seed=3, lens=(10, 0, 35, 1), ch=24, K=4):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = rng.standard_normal((int(cu[-1]), ch))
    w = rng.uniform(-0.8, 0.8, (ch, K))
    dy = rng.standard_normal(x.shape)
    return cu, x, w, dy


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_matches_torch_conv1d_and_autograd(K):
    """Per sequence, the oracle equals torch's grouped conv1d with K - 1 zeros of left
    padding followed by silu, and its input gradient equals torch autograd of that."""
    import torch
    from oracle.conv import conv1d_silu_bwd, conv1d_silu_fwd

    cu, x, w, dy = _conv_case(K=K)
    y = conv1d_silu_fwd(cu, x, w)
    dx = conv1d_silu_bwd(cu, x, w, dy)
    wt = torch.from_numpy(w)[:, None, :]  # [ch, 1, K]
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:
            continue
        xt = torch.from_numpy(x[a:b].T.copy())[None].requires_grad_(True)  # [1, ch, len]
        yt = torch.nn.functional.silu(torch.nn.functional.conv1d(xt, wt, padding=K - 1, groups=x.shape[1])[..., : b - a])
        (yt * torch.from_numpy(dy[a:b].T.copy())[None]).sum().backward()
        assert np.max(np.abs(yt.detach()[0].numpy().T - y[a:b])) < 1e-13, n
        assert np.max(np.abs(xt.grad[0].numpy().T - dx[a:b])) < 1e-13, n


def test_conv_input_gradient_finite_differences():
    from oracle.conv import conv1d_silu_bwd, conv1d_silu_fwd

    cu, x, w, dy = _conv_case(seed=9, lens=(7, 12), ch=8, K=4)
    dx = conv1d_silu_bwd(cu, x, w, dy)
    rng = np.random.default_rng(1)
    h = 1e-6
    for _ in range(12):
        t, c = int(rng.integers(x.shape[0])), int(rng.integers(x.shape[1]))
        xp, xm = x.copy(), x.copy()
        xp[t, c] += h
        xm[t, c] -= h
        fd = np.sum((conv1d_silu_fwd(cu, xp, w) - conv1d_silu_fwd(cu, xm, w)) * dy) / (2 * h)
        assert abs(fd - dx[t, c]) < 1e-7 * max(1.0, abs(fd)), (t, c, fd, dx[t, c])


# --- the layer's gate chain (oracle.gate_chain / gate_chain_grads)

def test_gate_chain_matches_torch_autograd_and_fd():
    """g = exp(-exp(a_log) softplus(alpha + dt_bias)), beta = sigmoid(beta_raw): values and
    the backward to alpha and beta_raw against torch (float64, torch's softplus and sigmoid,
    autograd), and central differences."""
    import torch

    rng = np.random.default_rng(12)
    T, Hv = 9, 5
    alpha, beta_raw = rng.standard_normal((T, Hv)) * 3, rng.standard_normal((T, Hv)) * 3
    a_log, dt_bias = rng.uniform(-2, 1, Hv), rng.uniform(-1, 1, Hv)
    dg, dbeta = rng.standard_normal((T, Hv)), rng.standard_normal((T, Hv))
    g, beta = oracle.gate_chain(alpha, a_log, dt_bias, beta_raw)
    da, dbr = oracle.gate_chain_grads(alpha, a_log, dt_bias, beta_raw, dg, dbeta)
    ta = torch.tensor(alpha, requires_grad=True)
    tb = torch.tensor(beta_raw, requires_grad=True)
    tg = torch.exp(-torch.exp(torch.tensor(a_log))[None] * torch.nn.functional.softplus(ta + torch.tensor(dt_bias)[None]))
    tbe = torch.sigmoid(tb)
    ((tg * torch.tensor(dg)).sum() + (tbe * torch.tensor(dbeta)).sum()).backward()
    assert np.max(np.abs(tg.detach().numpy() - g)) < 1e-14 and np.max(np.abs(tbe.detach().numpy() - beta)) < 1e-14
    assert np.max(np.abs(ta.grad.numpy() - da)) < 1e-13 and np.max(np.abs(tb.grad.numpy() - dbr)) < 1e-13
    h = 1e-6
    for t, j in [(0, 0), (4, 2), (8, 4)]:
        ap, am = alpha.copy(), alpha.copy()
        ap[t, j] += h
        am[t, j] -= h
        fd = (oracle.gate_chain(ap, a_log, dt_bias, beta_raw)[0][t, j] - oracle.gate_chain(am, a_log, dt_bias, beta_raw)[0][t, j]) / (2 * h)
        assert abs(fd * dg[t, j] - da[t, j]) < 1e-7 * max(1.0, abs(da[t, j]))


def test_l2norm_rows_matches_torch_autograd():
    """x / sqrt(sum x^2 + 1e-6) and its backward against torch autograd (float64), including
    a zero row (where the epsilon decides)."""
    import torch

    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 3, 16)) * 2
    x[2, 1] = 0.0
    dxh = rng.standard_normal(x.shape)
    xh, r = oracle.l2norm_rows(x)
    dx = oracle.l2norm_rows_grad(xh, r, dxh)
    tx = torch.tensor(x, requires_grad=True)
    th = tx / torch.sqrt((tx * tx).sum(-1, keepdim=True) + 1e-6)
    (th * torch.tensor(dxh)).sum().backward()
    assert np.max(np.abs(th.detach().numpy() - xh)) < 1e-14
    assert np.max(np.abs(tx.grad.numpy() - dx)) < 1e-12


# --- hand-worked values of the gate chain and the L2 norm (tests/golden/gate_chain_l2norm.json)

def _num(s):
    """A number of the golden file: a decimal or fraction string, or ln2 / ln3 forms."""
    import math

    s = str(s)
    named = {"ln2": math.log(2.0), "-ln2": -math.log(2.0), "ln3": math.log(3.0), "-ln3": -math.log(3.0),
             "ln3-1/2": math.log(3.0) - 0.5}
    return named[s] if s in named else float(Fraction(s))


def _gate_golden():
    with open(os.path.join(GOLDEN, "gate_chain_l2norm.json")) as f:
        return json.load(f)


def _gate_chain_errors(gate_chain, gate_chain_grads):
    """Largest absolute errors of a gate_chain / gate_chain_grads pair on the golden rows."""
    fx = _gate_golden()["gate_chain"]
    col = lambda k: np.array([_num(x) for x in fx[k]])
    a_log, dt_bias, alpha, beta_raw = col("a_log"), col("dt_bias"), col("alpha")[None, :], col("beta_raw")[None, :]
    g, beta = gate_chain(alpha, a_log, dt_bias, beta_raw)
    da, dbr = gate_chain_grads(alpha, a_log, dt_bias, beta_raw, np.ones_like(alpha), np.ones_like(beta_raw))
    got = dict(g=g[0], beta=beta[0], dalpha=da[0], dbeta_raw=dbr[0])
    return {k: float(np.max(np.abs(got[k] - col(k)))) for k in got}


def _l2norm_errors(l2norm_rows, l2norm_rows_grad):
    """Largest relative errors of an l2norm_rows / l2norm_rows_grad pair on the golden rows."""
    fx = _gate_golden()["l2norm"]
    errs = {"r": 0.0, "x_hat": 0.0, "dx": 0.0}
    rel = lambda a, b: float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-300))) if np.any(b) else float(np.max(np.abs(a)))
    for row in fx["rows"]:
        xh, r = l2norm_rows(np.array(row["x"], np.float64)[None, :])
        errs["r"] = max(errs["r"], rel(r[0, 0], _num(row["r"])))
        errs["x_hat"] = max(errs["x_hat"], rel(xh[0], np.array([_num(v) for v in row["x_hat"]])))
    for row in fx["grad"]:
        xh, r = l2norm_rows(np.array(row["x"], np.float64)[None, :])
        dx = l2norm_rows_grad(xh, r, np.array(row["dx_hat"], np.float64)[None, :])
        errs["dx"] = max(errs["dx"], rel(dx[0], np.array([_num(v) for v in row["dx"]])))
    return errs


def test_gate_chain_hand_worked_values():
    """g, beta and their derivatives at the golden rows, worked by hand from the page's
    formulas (a_log = 0 or +-ln 2 and alpha + dt_bias = 0 or ln 3 give g = 1/2 or 1/4)."""
    errs = _gate_chain_errors(oracle.gate_chain, oracle.gate_chain_grads)
    assert all(v < 1e-15 for v in errs.values()), errs


def test_l2norm_hand_worked_values():
    """r, x_hat and the backward at the golden rows, from the series of (1 + eps / |x|^2)^(-1/2)
    (the epsilon inside the square root decides the eighth significant digit of (3, 4) / 5)."""
    errs = _l2norm_errors(oracle.l2norm_rows, oracle.l2norm_rows_grad)
    assert all(v < 1e-15 for v in errs.values()), errs


def _mutant(fn, old, new, extra=None):
    """fn rebuilt from its source with one textual change (a planted mistake)."""
    import inspect
    import textwrap

    src = textwrap.dedent(inspect.getsource(fn))
    assert old in src, (fn.__name__, old)
    ns = {"np": np}
    ns.update(extra or {})
    exec(compile(src.replace(old, new, 1), f"<mutant {fn.__name__}>", "exec"), ns)
    return ns[fn.__name__]


GATE_MUTANTS = [
    ("gate_chain", "np.exp(-np.exp(a_log)[None, :] * softplus)", "np.exp(-a_log[None, :] * softplus)"),  # exp dropped on a_log
    ("gate_chain", "alpha + dt_bias[None, :]", "alpha"),  # dt_bias dropped
    ("gate_chain", "np.logaddexp(0.0, alpha + dt_bias[None, :])", "np.log1p(alpha + dt_bias[None, :])"),  # not softplus
    ("gate_chain", "np.exp(-np.exp(a_log)", "np.exp(np.exp(a_log)"),  # sign
    ("gate_chain", "np.exp(-beta_raw)", "np.exp(beta_raw)"),  # sigmoid of -beta_raw
    ("gate_chain_grads", "* sig", ""),  # softplus' derivative dropped
    ("gate_chain_grads", "(-np.exp(a_log)[None, :])", "(-a_log[None, :])"),
    ("gate_chain_grads", "dbeta * beta * (1.0 - beta)", "dbeta * beta"),
]


@pytest.mark.parametrize("fn,old,new", GATE_MUTANTS, ids=[f"{m[0]}-{i}" for i, m in enumerate(GATE_MUTANTS)])
def test_gate_chain_planted_mistake_is_caught(fn, old, new):
    gc, gg = oracle.gate_chain, oracle.gate_chain_grads
    if fn == "gate_chain":
        gc = _mutant(gc, old, new)
        gg = _mutant(gg, "g, beta = gate_chain(", "g, beta = gate_chain(", {"gate_chain": gc})
    else:
        gg = _mutant(gg, old, new, {"gate_chain": gc})
    errs = _gate_chain_errors(gc, gg)
    assert max(errs.values()) > 1e-6, errs


L2_MUTANTS = [
    ("l2norm_rows", "np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)",
     "(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + 1e-6)"),  # epsilon outside the root
    ("l2norm_rows", "keepdims=True) + 1e-6)", "keepdims=True))"),  # epsilon dropped
    ("l2norm_rows", "1.0 / np.sqrt(", "1.0 / ("),  # squared norm instead of norm
    ("l2norm_rows_grad", "dx_hat - x_hat * np.sum(x_hat * dx_hat, axis=-1, keepdims=True)", "dx_hat"),  # projection dropped
    ("l2norm_rows_grad", "return r * (", "return ("),  # factor r dropped
]


@pytest.mark.parametrize("fn,old,new", L2_MUTANTS, ids=[f"{m[0]}-{i}" for i, m in enumerate(L2_MUTANTS)])
def test_l2norm_planted_mistake_is_caught(fn, old, new):
    ln, lg = oracle.l2norm_rows, oracle.l2norm_rows_grad
    if fn == "l2norm_rows":
        ln = _mutant(ln, old, new)
    else:
        lg = _mutant(lg, old, new)
    with np.errstate(all="ignore"):  # (a mutant may divide the zero row by zero)
        errs = _l2norm_errors(ln, lg)
    assert not max(errs.values()) <= 1e-9, errs
