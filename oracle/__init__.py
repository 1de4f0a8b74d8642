"""Float64 CPU oracle of the gated delta-net recurrence (forward and backward).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``; never by the product package. It shares no code
with the HIP path. The arithmetic lives in ``gdn_oracle.c`` (plain C, float64, no
contraction, one thread per (sequence, key head) group); this module builds it with
gcc and marshals numpy arrays through ctypes.

Pins (tests/test_oracle.py) tie it to things other than itself: central finite
differences of its own forward, a second formulation of the recurrence
(S_t = g_t (I - beta_t k k^T) S_{t-1} + beta_t k v^T) differentiated by torch
autograd, closed forms (beta = 0, T = 1, g = beta = 1 with orthonormal keys),
the v_repeat / replication identity, linearity, zero upstream gradient and split
resume. ``gdn_decode`` (one step per row, state slots) is the forward over one-token
sequences; its own pins replay the hand-worked example token by token and check the
slot map against per-row forwards. ``gate_chain`` / ``gate_chain_grads`` (the layer's
g = exp(-exp(a_log) softplus(alpha + dt_bias)), beta = sigmoid(beta_raw) and their
derivatives) and ``l2norm_rows`` / ``l2norm_rows_grad`` (the q/k normalisation and its
backward) are pinned to values worked by hand from the page's formulas
(``tests/golden/gate_chain_l2norm.json``: a_log = 0 or +-ln 2 with alpha + dt_bias = 0 or
ln 3 give g = 1/2 or 1/4; the series of (1 + eps/|x|^2)^(-1/2) for the norm), with planted
mistakes (the epsilon outside the root, exp dropped on a_log, dt_bias dropped, ...) that must
fail them; their gradients are also checked against finite differences. No function here is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "gdn_oracle.c")
# GDN_ORACLE_LIBRARY may name another build of gdn_oracle.c (the sanitizer build, for instance).
LIB = os.environ.get("GDN_ORACLE_LIBRARY") or os.path.join(_HERE, "libgdn_oracle.so")

_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-pthread"]


def build(out: str = LIB, plant: Optional[int] = None) -> str:
    """Compile the oracle with gcc. ``plant`` builds a deliberately broken
    variant (used only by the falsification test). A build named by GDN_ORACLE_LIBRARY is
    used as it is (not rebuilt)."""
    if out == LIB and plant is None and os.environ.get("GDN_ORACLE_LIBRARY"):
        return out
    cmd = ["gcc", *_CFLAGS, SRC, "-o", out]
    if plant is not None:
        cmd.insert(1, f"-DORACLE_PLANT={int(plant)}")
    subprocess.run(cmd, check=True)
    return out


_libs = {}


def _load(path: str = LIB):
    if path not in _libs:
        if path == LIB and not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_gdn_fwd.argtypes = [I, P, I, I, I, I, ctypes.c_double] + [P] * 8 + [I]
        lib.oracle_gdn_fwd.restype = I
        lib.oracle_gdn_bwd.argtypes = [I, P, I, I, I, I, ctypes.c_double] + [P] * 14 + [I]
        lib.oracle_gdn_bwd.restype = I
        _libs[path] = lib
    return _libs[path]


def _c(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def gdn_fwd(cu, q, k, v, g, beta, S0=None, scale=None, nthreads=None, lib=None):
    """Forward. q, k [T, Hk, Dk]; v [T, Hv, Dv]; g, beta [T, Hv]; S0 [N, Hv, Dk, Dv] or None.
    Returns (o [T, Hv, Dv], S_T [N, Hv, Dk, Dv])."""
    cu = np.ascontiguousarray(cu, dtype=np.int64)
    q, k, v, g, beta, S0 = map(_c, (q, k, v, g, beta, S0))
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    N = len(cu) - 1
    assert cu[-1] == T and k.shape == q.shape and v.shape[0] == T and g.shape == (T, Hv)
    if scale is None:
        scale = 1.0 / np.sqrt(Dk)
    o = np.zeros((T, Hv, Dv))
    ST = np.zeros((N, Hv, Dk, Dv))
    L = _load(lib or LIB)
    rc = L.oracle_gdn_fwd(N, _p(cu), Hk, Hv, Dk, Dv, float(scale), _p(q), _p(k), _p(v), _p(g),
                          _p(beta), _p(S0), _p(o), _p(ST), int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_gdn_fwd failed ({rc})")
    return o, ST


def gdn_bwd(cu, q, k, v, g, beta, S0, dO, dST, scale=None, nthreads=None, lib=None):
    """Backward. Returns dict dq, dk [T, Hk, Dk], dv [T, Hv, Dv], dg, dbeta [T, Hv],
    dS0 [N, Hv, Dk, Dv]."""
    cu = np.ascontiguousarray(cu, dtype=np.int64)
    q, k, v, g, beta, S0, dO, dST = map(_c, (q, k, v, g, beta, S0, dO, dST))
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    N = len(cu) - 1
    if scale is None:
        scale = 1.0 / np.sqrt(Dk)
    out = dict(
        dq=np.zeros((T, Hk, Dk)), dk=np.zeros((T, Hk, Dk)), dv=np.zeros((T, Hv, Dv)),
        dg=np.zeros((T, Hv)), dbeta=np.zeros((T, Hv)), dS0=np.zeros((N, Hv, Dk, Dv)),
    )
    L = _load(lib or LIB)
    rc = L.oracle_gdn_bwd(N, _p(cu), Hk, Hv, Dk, Dv, float(scale), _p(q), _p(k), _p(v), _p(g),
                          _p(beta), _p(S0), _p(dO), _p(dST), _p(out["dq"]), _p(out["dk"]),
                          _p(out["dv"]), _p(out["dg"]), _p(out["dbeta"]), _p(out["dS0"]),
                          int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_gdn_bwd failed ({rc})")
    return out


def gate_chain(alpha, a_log, dt_bias, beta_raw):
    """The layer's gate chain (the gdn_backward.rs page, "decay gate g per value-head" and
    "sigmoid(beta)"): g = exp(-exp(a_log[h]) softplus(alpha + dt_bias[h])) and
    beta = sigmoid(beta_raw). alpha, beta_raw [T, Hv]; a_log, dt_bias [Hv]. Returns (g, beta)."""
    alpha, beta_raw = np.asarray(alpha, np.float64), np.asarray(beta_raw, np.float64)
    a_log, dt_bias = np.asarray(a_log, np.float64), np.asarray(dt_bias, np.float64)
    softplus = np.logaddexp(0.0, alpha + dt_bias[None, :])
    g = np.exp(-np.exp(a_log)[None, :] * softplus)
    beta = 1.0 / (1.0 + np.exp(-beta_raw))
    return g, beta


def gate_chain_grads(alpha, a_log, dt_bias, beta_raw, dg, dbeta):
    """d alpha and d beta_raw from the gradients dg, dbeta of g and beta (the page's steps 4e
    and 4h): dg/d alpha = g (-exp(a_log)) sigmoid(alpha + dt_bias), dbeta/d beta_raw =
    beta (1 - beta). Returns (dalpha, dbeta_raw)."""
    g, beta = gate_chain(alpha, a_log, dt_bias, beta_raw)
    a_log, dt_bias = np.asarray(a_log, np.float64), np.asarray(dt_bias, np.float64)
    sig = 1.0 / (1.0 + np.exp(-(np.asarray(alpha, np.float64) + dt_bias[None, :])))
    return dg * g * (-np.exp(a_log)[None, :]) * sig, dbeta * beta * (1.0 - beta)


def l2norm_rows(x):
    """x_hat = x / sqrt(sum x^2 + 1e-6) over the last axis (the gdn_backward.rs page, "L2-normalize
    q, k", epsilon inside the square root). Returns (x_hat, r) with r = 1 / sqrt(sum x^2 + 1e-6)."""
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)
    return x * r, r


def l2norm_rows_grad(x_hat, r, dx_hat):
    """Gradient with respect to x of x_hat = x r (the page's step 4f):
    r (dx_hat - x_hat (x_hat . dx_hat))."""
    return r * (dx_hat - x_hat * np.sum(x_hat * dx_hat, axis=-1, keepdims=True))


def gdn_decode(q, k, v, g, beta, state, slot_idx=None, scale=None, nthreads=None, lib=None):
    """One decode step: row n is one token of its own sequence, whose state is
    ``state[slot_idx[n]]`` (slot n when ``slot_idx`` is None); a row whose slot lies outside
    [0, n_slots) is skipped. This is the forward above over N one-token sequences (the
    per-token recurrence of the "Forward recap" module doc, one step), with no arithmetic
    of its own. q, k [N, Hk, Dk]; v [N, Hv, Dv]; g, beta [N, Hv]; state [n_slots, Hv, Dk, Dv].
    Returns (o [N, Hv, Dv], NaN on skipped rows; the updated copy of ``state``)."""
    N = q.shape[0]
    n_slots = state.shape[0]
    slots = np.arange(N) if slot_idx is None else np.asarray(slot_idx, dtype=np.int64)
    rows = np.array([n for n in range(N) if 0 <= slots[n] < n_slots], dtype=np.int64)
    assert len(set(slots[rows].tolist())) == len(rows), "two rows share a slot"
    o = np.full((N,) + v.shape[1:], np.nan)
    new = np.array(state, dtype=np.float64, copy=True)
    if len(rows):
        cu = np.arange(len(rows) + 1, dtype=np.int64)
        o_r, ST = gdn_fwd(cu, q[rows], k[rows], v[rows], g[rows], beta[rows], new[slots[rows]], scale, nthreads, lib)
        o[rows] = o_r
        new[slots[rows]] = ST
    return o, new


def run_case(case, backward=True, nthreads=None, lib=None, seqs=None, key_heads=None):
    """Run the oracle on a ``synth.GdnCase``. ``seqs`` / ``key_heads`` restrict it to a
    subset of sequences and key-head groups (each group is independent of the others,
    so the restriction is exact). Returns dict with o, S_T and, if backward, the
    gradients, indexed like the restricted problem, plus the index maps used."""
    r = case.Hv // case.Hk
    seqs = list(range(case.N)) if seqs is None else list(seqs)
    key_heads = list(range(case.Hk)) if key_heads is None else list(key_heads)
    vheads = [kh * r + j for kh in key_heads for j in range(r)]
    cu_full = case.cu_seqlens
    rows = np.concatenate([np.arange(cu_full[n], cu_full[n + 1]) for n in seqs]) if seqs else np.zeros(0, np.int64)
    lens = [int(cu_full[n + 1] - cu_full[n]) for n in seqs]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    sel = lambda a, heads: a[rows][:, heads]
    q, k = sel(case.q, key_heads), sel(case.k, key_heads)
    v, g, beta, dO = sel(case.v, vheads), sel(case.g, vheads), sel(case.beta, vheads), sel(case.dO, vheads)
    S0 = None if case.S0 is None else case.S0[seqs][:, vheads]
    dST = None if case.dST is None else case.dST[seqs][:, vheads]
    o, ST = gdn_fwd(cu, q, k, v, g, beta, S0, case.scale, nthreads, lib)
    res = dict(o=o, S_T=ST, rows=rows, vheads=vheads, key_heads=key_heads, seqs=seqs)
    if backward:
        res.update(gdn_bwd(cu, q, k, v, g, beta, S0, dO, dST, case.scale, nthreads, lib))
    return res
