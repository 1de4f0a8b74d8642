"""GPU: a NaN in one input element reaches only the outputs that depend on it, and the calls
return normally.

Dependence is at chunk granularity in the chunked form: within a chunk the products treat
every row together (a zero factor times NaN is NaN), so a NaN in row t may also reach the
earlier rows of t's own chunk. Across chunks, sequences and heads the reach is exact:

* NaN in v[t, h, j] (sequence n): value columns never mix, so o and S_T of (n, h) change in
  column j only; the forward outputs of (n, h) before t's chunk, every output
  of the other sequences, of the other key-head groups and of the other value heads of h's
  group, and dv and dS0 of (n, h) itself (the state adjoint never reads v), are bit-identical
  to a clean run; the backward's dq, dk (key head of h), dg, dbeta of (n, h) are unchanged on
  the chunks before t's; o[t, h, j] and column j of S_T[n, h] are NaN.
* NaN in g[t, h]: the state adjoint carries the decay backwards, so every backward output of
  (n, h) may change; the other sequences, groups and value heads stay bit-identical, and so
  do the forward outputs of (n, h) before t's chunk.
"""
import dataclasses

import numpy as np
import pytest

from synth import make_case
from gdn_gpu import run_gpu

pytestmark = pytest.mark.gpu

C = 64


def _case():
    return make_case(1500, [150, 100], 2, 6, 64, dtype="bf16", chunk=C, gate="clamp09", with_S0=True,
                     with_dST=True, packed=True, varlen=True, name="nan")


def _same(a, b):
    assert a.shape == b.shape
    return bool(np.array_equal(a, b))


def _check_untouched(case, clean, bad, n, h):
    """Everything that does not depend on (sequence n, value head h) is bit-identical."""
    cu = case.cu_seqlens
    r = case.Hv // case.Hk
    kh = h // r
    other_rows = np.r_[0:cu[n], cu[n + 1]:case.T_total]
    for name in ("o", "dv", "dg", "dbeta", "dq", "dk"):
        assert _same(clean[name][other_rows], bad[name][other_rows]), ("other sequences", name)
    for name in ("S_T", "dS0"):
        others = [m for m in range(case.N) if m != n]
        assert _same(clean[name][others], bad[name][others]), ("other sequences", name)
    grp = [j for j in range(case.Hv) if j // r != kh]
    for name in ("o", "dv", "dg", "dbeta"):
        assert _same(clean[name][:, grp], bad[name][:, grp]), ("other groups", name)
    for name in ("S_T", "dS0"):
        assert _same(clean[name][:, grp], bad[name][:, grp]), ("other groups", name)
    okh = [j for j in range(case.Hk) if j != kh]
    for name in ("dq", "dk"):
        assert _same(clean[name][:, okh], bad[name][:, okh]), ("other key heads", name)
    sib = [j for j in range(kh * r, kh * r + r) if j != h]
    for name in ("o", "dv", "dg", "dbeta"):
        assert _same(clean[name][:, sib], bad[name][:, sib]), ("other value heads of the group", name)
    for name in ("S_T", "dS0"):
        assert _same(clean[name][:, sib], bad[name][:, sib]), ("other value heads of the group", name)


def test_nan_in_v_reaches_only_its_dependents():
    case = _case()
    n, h, t_local = 0, 1, 70  # sequence 0, value head 1 (key head 0), row 70: the second chunk
    t = int(case.cu_seqlens[n]) + t_local
    c0 = int(case.cu_seqlens[n]) + (t_local // C) * C  # first row of t's chunk
    v = case.v.copy()
    v[t, h, 5] = np.nan
    print(f"[nan] v[{t}, {h}, 5]", flush=True)
    clean = run_gpu(case)
    bad = run_gpu(dataclasses.replace(case, v=v))
    _check_untouched(case, clean, bad, n, h)
    pre = slice(int(case.cu_seqlens[n]), c0)
    assert _same(clean["o"][pre, h], bad["o"][pre, h])
    # value columns never mix: the NaN stays in column 5 of o and of the state
    assert np.isnan(bad["o"][t, h, 5]) and np.isfinite(np.delete(bad["o"][t, h], 5)).all()
    assert np.isnan(bad["S_T"][n, h][:, 5]).all() and np.isfinite(np.delete(bad["S_T"][n, h], 5, axis=1)).all()
    # the state adjoint and dv never read v
    rows = slice(int(case.cu_seqlens[n]), int(case.cu_seqlens[n + 1]))
    assert _same(clean["dv"][rows, h], bad["dv"][rows, h]) and _same(clean["dS0"][n, h], bad["dS0"][n, h])
    kh = h // (case.Hv // case.Hk)
    for name, col in (("dg", h), ("dbeta", h)):
        assert _same(clean[name][pre, col], bad[name][pre, col]), name
    for name in ("dq", "dk"):
        assert _same(clean[name][pre, kh], bad[name][pre, kh]), name
    assert not np.isfinite(bad["dg"][t:int(case.cu_seqlens[n + 1]), h]).all()


def test_nan_in_g_reaches_only_its_dependents():
    case = _case()
    n, h = 1, 4  # sequence 1, value head 4 (key head 1)
    t_local = 66
    t = int(case.cu_seqlens[n]) + t_local
    c0 = int(case.cu_seqlens[n]) + (t_local // C) * C
    g = case.g.copy()
    g[t, h] = np.nan
    print(f"[nan] g[{t}, {h}]", flush=True)
    clean = run_gpu(case)
    bad = run_gpu(dataclasses.replace(case, g=g))
    _check_untouched(case, clean, bad, n, h)
    pre = slice(int(case.cu_seqlens[n]), c0)
    assert _same(clean["o"][pre, h], bad["o"][pre, h])
    assert np.isnan(bad["o"][t, h]).all() and np.isnan(bad["S_T"][n, h]).any()
    assert np.isnan(bad["dg"][t, h])
