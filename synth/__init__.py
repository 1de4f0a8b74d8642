"""Seeded synthetic inputs for the gated delta-net recurrence.

This module only draws random numbers and rounds them to the storage
precision. It holds none of the recurrence's arithmetic: both the oracle
(``oracle/``) and the HIP path receive the arrays produced here, so the two
sides always see the same values.

Recipe (the five workloads the pages' shapes call for):

* q, k ~ N(0, 1), then each head row is L2-normalised as x / sqrt(sum x^2 + 1e-6)
  (the epsilon sits inside the square root, as in the q/k normalisation of the
  lattice-inference ``gdn_backward.rs`` forward, "L2-normalize q, k").
  The recurrence itself takes q-hat/k-hat as given; the normalisation is part of
  how the inputs are made, not part of the operation under test.
* v ~ N(0, 1); beta = sigmoid(N(0, 1)).
* g_raw = exp(-exp(a) * softplus(x + 0.5)) with one a ~ U(-1, 0) per value head and
  x ~ N(0, 1) per (token, value head) (the decay-gate formula of the same page,
  "decay gate g per value-head", with dt_bias = 0.5).
  Workloads 1-3 clamp g = max(g_raw, 0.9); workload 4 maps g = 0.8 + 0.2 * g_raw.
* S0 and dS_T ~ N(0, 0.1^2) where the workload has them, otherwise absent (zero).
* dO ~ N(0, 1).

Every value is drawn in float64 with ``numpy.random.default_rng(seed)`` in the
fixed order lengths (varlen only), q, k, v, a, x, beta_raw, S0, dO, dS_T, and is
then rounded once, round-to-nearest-even, to its storage type: float32, or
bfloat16 for q/k/v/dO of the bf16 workloads (g, beta and states are float32).
The arrays returned hold those rounded values as float64.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

__all__ = ["GdnCase", "round_bf16", "round_f32", "make_case", "config_case", "CONFIG_SPECS"]


def round_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest float32 (RNE), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (8 significant bits, RNE), as float64.

    Rounds in one step from float64 (no intermediate float32 rounding).
    Values here are far from the bf16 overflow and subnormal ranges.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def _l2_rows(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


@dataclasses.dataclass
class GdnCase:
    """One seeded problem. Arrays are float64 holding storage-precision values.

    Shapes: q, k [T_total, Hk, Dk]; v, dO [T_total, Hv, Dv]; g, beta [T_total, Hv];
    S0, dST [N, Hv, Dk, Dv] or None (zero).
    """

    name: str
    lens: List[int]
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    chunk: int
    dtype: str  # "f32" or "bf16": storage of q, k, v, o, dO, dq, dk, dv
    packed: bool  # q/k/v are row views of one packed projection
    varlen: bool  # passed with cu_seqlens
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    S0: Optional[np.ndarray]
    dO: np.ndarray
    dST: Optional[np.ndarray]

    @property
    def N(self) -> int:
        return len(self.lens)

    @property
    def T_total(self) -> int:
        return int(sum(self.lens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lens)]).astype(np.int64)


def make_case(
    seed: int,
    lens: List[int],
    Hk: int,
    Hv: int,
    D: int,
    *,
    dtype: str = "f32",
    chunk: int = 16,
    gate: str = "raw",
    with_S0: bool = False,
    with_dST: bool = False,
    packed: bool = False,
    varlen: bool = False,
    draw_lens: Optional[tuple] = None,
    name: str = "custom",
) -> GdnCase:
    """Draw one problem. ``gate`` is "raw", "clamp09" or "affine08"."""
    rng = np.random.default_rng(seed)
    if draw_lens is not None:
        n, lo, hi = draw_lens
        lens = [int(x) for x in rng.integers(lo, hi + 1, size=n)]
    T = int(sum(lens))
    N = len(lens)
    rnd = round_bf16 if dtype == "bf16" else round_f32
    q = rnd(_l2_rows(rng.standard_normal((T, Hk, D))))
    k = rnd(_l2_rows(rng.standard_normal((T, Hk, D))))
    v = rnd(rng.standard_normal((T, Hv, D)))
    a = rng.uniform(-1.0, 0.0, size=(Hv,))
    x = rng.standard_normal((T, Hv))
    beta_raw = rng.standard_normal((T, Hv))
    g_raw = np.exp(-np.exp(a)[None, :] * _softplus(x + 0.5))
    if gate == "raw":
        g = g_raw
    elif gate == "clamp09":
        g = np.maximum(g_raw, 0.9)
    elif gate == "affine08":
        g = 0.8 + 0.2 * g_raw
    else:
        raise ValueError(gate)
    g = round_f32(g)
    beta = round_f32(1.0 / (1.0 + np.exp(-beta_raw)))
    S0 = round_f32(0.1 * rng.standard_normal((N, Hv, D, D))) if with_S0 else None
    dO = rnd(rng.standard_normal((T, Hv, D)))
    dST = round_f32(0.1 * rng.standard_normal((N, Hv, D, D))) if with_dST else None
    return GdnCase(
        name=name, lens=list(lens), Hk=Hk, Hv=Hv, Dk=D, Dv=D, chunk=chunk, dtype=dtype,
        packed=packed, varlen=varlen, scale=1.0 / float(np.sqrt(D)),
        q=q, k=k, v=v, g=g, beta=beta, S0=S0, dO=dO, dST=dST,
    )


# The five workloads. Sizes: tokens per sequence, key/value heads, head size.
CONFIG_SPECS = {
    0: dict(lens=[32], Hk=2, Hv=4, D=16, dtype="f32", chunk=16, gate="raw",
            with_S0=False, with_dST=False, packed=False, varlen=False,
            name="tiny B1 T32 Hk2 Hv4 D16 f32"),
    1: dict(lens=[256, 256], Hk=4, Hv=4, D=64, dtype="f32", chunk=16, gate="clamp09",
            with_S0=True, with_dST=True, packed=False, varlen=False,
            name="B2 T256 Hk4 Hv4 D64 f32 C16"),
    2: dict(lens=[2048], Hk=16, Hv=48, D=128, dtype="bf16", chunk=64, gate="clamp09",
            with_S0=True, with_dST=True, packed=True, varlen=False,
            name="strided B1 T2048 Hk16 Hv48 D128 bf16"),
    3: dict(lens=[4096] * 4, Hk=16, Hv=48, D=128, dtype="bf16", chunk=64, gate="clamp09",
            with_S0=False, with_dST=True, packed=True, varlen=False,
            name="training B4 T4096 Hk16 Hv48 D128 bf16"),
    4: dict(lens=[], Hk=16, Hv=48, D=128, dtype="bf16", chunk=64, gate="affine08",
            with_S0=True, with_dST=True, packed=True, varlen=True, draw_lens=(8, 256, 8192),
            name="varlen 8 seqs U[256,8192] Hk16 Hv48 D128 bf16"),
}


def config_case(i: int, **overrides) -> GdnCase:
    """Workload ``i`` (0..4), seeded with 1000 + i. ``overrides`` may shrink it
    (e.g. ``lens=[300]`` or ``Hk=2, Hv=6``) for tests that need a smaller run of the
    same recipe; a different shape then also uses a different seed offset only if
    ``seed`` is given explicitly."""
    spec = dict(CONFIG_SPECS[i])
    seed = overrides.pop("seed", 1000 + i)
    spec.update(overrides)
    lens = spec.pop("lens")
    Hk, Hv, D = spec.pop("Hk"), spec.pop("Hv"), spec.pop("D")
    return make_case(seed, lens, Hk, Hv, D, **spec)
