"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Forward agreement is checked before gradients (the dormouse KDA log's rule: make sure
both sides computed the same function before comparing derivatives). Bars: 2e-4
normwise for float32 inputs, 2e-2 for bfloat16 inputs with float32 state.
The full-size workloads (strided v_repeat 3, the training shape, varlen) are compared
element by element over every sequence and head.
"""
import sys

import numpy as np
import pytest

import dataclasses

import oracle
from synth import config_case, make_case, round_f32
from gdn_gpu import GRAD_NAMES, OUT_NAMES, compare, run_gpu

pytestmark = pytest.mark.gpu


def _check(case, seqs=None, key_heads=None, chunk=None, backward=True):
    print(f"[parity] {case.name} lens={case.lens[:8]} chunk={chunk or case.chunk}", flush=True)
    gpu = run_gpu(case, backward=backward, chunk=chunk)
    ref = oracle.run_case(case, backward=backward, seqs=seqs, key_heads=key_heads)
    rep = {}
    compare(case, gpu, ref, OUT_NAMES, report=rep)
    if backward:
        compare(case, gpu, ref, GRAD_NAMES, report=rep)
    print("   ", {k: f"{v:.2e}" for k, v in rep.items()}, flush=True)
    for name, a in gpu.items():
        assert np.all(np.isfinite(a)), name
    return gpu


def test_config0_tiny_f32():
    _check(config_case(0))


def test_config1_f32_chunk16():
    _check(config_case(1))


@pytest.mark.parametrize("chunk,D", [(16, 64), (64, 32)])
def test_config1_recipe_both_chunks(chunk, D):
    # float32 with chunk 64 is built for head sizes up to 32 (LDS budget)
    _check(config_case(1, lens=[130, 130], D=D), chunk=chunk)


SMALL = [
    # name, lens, Hk, Hv, D, dtype, chunk, varlen
    ("bf16_ragged_r3_D128", [200], 2, 6, 128, "bf16", 64, False),
    ("bf16_two_seqs_D64_C16", [77, 77], 1, 2, 64, "bf16", 16, False),
    ("f32_D32_C64_ragged", [150], 2, 4, 32, "f32", 64, False),
    ("f32_D16_C64", [70, 70, 70], 1, 3, 16, "f32", 64, False),
    ("f32_D128_C16", [40], 1, 1, 128, "f32", 16, False),
    ("bf16_varlen_zero_len", [0, 65, 1, 128, 0, 63], 2, 4, 64, "bf16", 64, True),
    ("f32_varlen_ragged_C16", [17, 0, 33, 5], 2, 2, 32, "f32", 16, True),
    # more value heads per key head than the kernels keep per-head state for at once (gate
    # records are formed four heads at a time, dg and dbeta staged for up to four heads)
    ("bf16_r8_D64", [150], 1, 8, 64, "bf16", 64, False),
    ("f32_r5_D32_C16", [70], 1, 5, 32, "f32", 16, False),
    # bf16 chunk 64 at the small head sizes (one and two MFMA steps over d in prep's Gram)
    ("bf16_D16_C64_ragged", [90, 90], 2, 2, 16, "bf16", 64, False),
    ("bf16_D32_C64", [128, 128], 1, 3, 32, "bf16", 64, False),
]


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes(spec):
    name, lens, Hk, Hv, D, dtype, chunk, varlen = spec
    case = make_case(500 + len(name), lens, Hk, Hv, D, dtype=dtype, chunk=chunk, gate="clamp09",
                     with_S0=True, with_dST=True, packed=(dtype == "bf16"), varlen=varlen, name=name)
    _check(case)


DEGENERATE = [
    # name, gate rule, beta rule, dtype, chunk, D
    ("g1_beta0_bf16", "one", "zero", "bf16", 64, 128),    # state carried unchanged: T = I
    ("g1_beta1_bf16", "one", "one", "bf16", 64, 128),     # no decay, full delta-rule write
    ("g_pow6_bf16", "pow6", "keep", "bf16", 64, 128),     # strong decay: 2^gamma underflows within a chunk
    ("g1_beta0_f32_C16", "one", "zero", "f32", 16, 32),
]


@pytest.mark.parametrize("spec", DEGENERATE, ids=[s[0] for s in DEGENERATE])
def test_degenerate_gates(spec):
    """Boundary values of the gates: g = 1 (log g = 0), beta = 0 and 1, and gates so small
    that the cumulative decay of a chunk falls below the float32 range (g ~ 1e-8 .. 0.8)."""
    name, gr, br, dtype, chunk, D = spec
    case = make_case(900 + len(name), [150, 37], 2, 6, D, dtype=dtype, chunk=chunk, gate="raw",
                     with_S0=True, with_dST=True, packed=(dtype == "bf16"), varlen=True, name=name)
    g = {"one": np.ones_like(case.g), "pow6": round_f32(case.g ** 6)}[gr]
    beta = {"zero": np.zeros_like(case.beta), "one": np.ones_like(case.beta), "keep": case.beta}[br]
    _check(dataclasses.replace(case, g=g, beta=beta))


def test_config2_strided_vrepeat3():
    """Every sequence, head and element of the strided v_repeat 3 workload."""
    _check(config_case(2))


def test_config3_training_shape_full():
    """The 27B-layer training shape (4 x 4096 tokens, Hk 16, Hv 48, D 128): every output and
    gradient element against the oracle's whole-batch run."""
    _check(config_case(3))


def test_config4_varlen_full():
    """The varlen workload (8 sequences of U[256, 8192] tokens, S0 and dS0): every element."""
    _check(config_case(4))
