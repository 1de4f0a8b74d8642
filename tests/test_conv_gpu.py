"""GPU parity of the causal depthwise conv1d + SiLU (gdn_conv1d_silu_fwd / _bwd) against
the float64 oracle (oracle/conv.py).

Inputs (seeded): x and dy standard normal, w uniform in [-0.8, 0.8]. bf16 inputs are
rounded on the host first so that the oracle sees the device's values. Tolerance:
normwise 2e-2 (bf16) / 2e-4 (float32). Shapes cover every kernel size, sequence
boundaries inside a thread's 32-row run, an empty sequence, a one-row sequence, a
channel count that leaves the last workgroup partly idle, and the packed projection of
the training shape (16384 rows x 10240 channels).
"""
import numpy as np
import pytest

from gdn_gpu import normwise

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 2e-4}


def _round(a, dtype):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a)).float()
    return (t.to(torch.bfloat16).float() if dtype == "bf16" else t).double().numpy()


def _run(dtype, lens, ch, K, seed, varlen=True, x_pad=0):
    """Forward and input gradient on the GPU; returns (cu, x, w, dy, y, dx) as float64."""
    import torch
    import gated_delta_rule_34_amd as G

    rng = np.random.default_rng(seed)
    rows = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = _round(rng.standard_normal((rows, ch)), dtype)
    dy = _round(rng.standard_normal((rows, ch)), dtype)
    w = rng.uniform(-0.8, 0.8, (ch, K)).astype(np.float32).astype(np.float64)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = "cuda"
    xb = torch.zeros(rows, ch + x_pad, dtype=dt, device=dev)  # x as a row view of a wider buffer
    xb[:, :ch] = torch.from_numpy(x).to(dt)
    tx = xb[:, :ch]
    tdy = torch.from_numpy(dy).to(dt).to(dev)
    tw = torch.from_numpy(w).float().to(dev)
    y = torch.empty(rows, ch, dtype=dt, device=dev)
    dx = torch.empty(rows, ch, dtype=dt, device=dev)
    tcu = torch.from_numpy(cu.astype(np.int32)).to(dev) if varlen else None
    p = G.make_conv_problem(len(lens), rows, ch, K, cu_seqlens=tcu, dtype=dtype,
                            T=None if varlen else lens[0])
    G.gdn_conv1d_silu_fwd(p, tx, tw, y)
    G.gdn_conv1d_silu_bwd(p, tx, tw, tdy, dx)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return cu, x, w, dy, f(y), f(dx)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_parity_varlen(dtype, K):
    from oracle.conv import conv1d_silu_bwd, conv1d_silu_fwd

    cu, x, w, dy, y, dx = _run(dtype, [1, 5, 70, 0, 33, 31], 296, K, seed=40 + K, x_pad=8)
    assert normwise(y, conv1d_silu_fwd(cu, x, w)) < TOL[dtype]
    assert normwise(dx, conv1d_silu_bwd(cu, x, w, dy)) < TOL[dtype]


def test_conv_parity_equal_length():
    from oracle.conv import conv1d_silu_bwd, conv1d_silu_fwd

    cu, x, w, dy, y, dx = _run("bf16", [50, 50, 50], 2056, 4, seed=5, varlen=False)
    assert normwise(y, conv1d_silu_fwd(cu, x, w)) < TOL["bf16"]
    assert normwise(dx, conv1d_silu_bwd(cu, x, w, dy)) < TOL["bf16"]


def test_conv_first_rows_see_an_empty_buffer():
    """Row 0 of each sequence depends on its own input only: y = SiLU(w[K-1] x), bit for bit
    against the same formula evaluated by the kernel for a one-row sequence."""
    cu, x, w, dy, y, dx = _run("f32", [1, 1, 1], 64, 4, seed=8)
    z = w[:, 3] * x
    assert normwise(y, z / (1 + np.exp(-z))) < 1e-6


def test_conv_training_projection_sampled_channels():
    """16384 rows x 10240 channels (4 sequences of 4096), K = 4, bf16: the conv of the
    training shape's packed projection. Channels are independent, so the oracle runs on
    every seventh 8-channel group (all rows) and that restriction is exact."""
    from oracle.conv import conv1d_silu_bwd, conv1d_silu_fwd

    cu, x, w, dy, y, dx = _run("bf16", [4096] * 4, 10240, 4, seed=77, varlen=False)
    sel = np.concatenate([np.arange(g * 8, g * 8 + 8) for g in range(0, 10240 // 8, 7)])
    assert normwise(y[:, sel], conv1d_silu_fwd(cu, x[:, sel], w[sel])) < TOL["bf16"]
    assert normwise(dx[:, sel], conv1d_silu_bwd(cu, x[:, sel], w[sel], dy[:, sel])) < TOL["bf16"]


@pytest.mark.parametrize("K", [2, 4])
def test_conv_sequence_starts_on_run_boundaries(K):
    """Sequence starts at rows 32, 96 and 128 (each the first row of a thread's 32-row run),
    empty sequences at a run start, and a one-row last sequence: the rows a run reads before
    its start (forward window) and past its end (backward halo) belong to other sequences
    and must not enter its sums."""
    from oracle.conv import conv1d_silu_bwd, conv1d_silu_fwd

    cu, x, w, dy, y, dx = _run("bf16", [32, 64, 0, 32, 0, 1], 520, K, seed=90 + K)
    assert normwise(y, conv1d_silu_fwd(cu, x, w)) < TOL["bf16"]
    assert normwise(dx, conv1d_silu_bwd(cu, x, w, dy)) < TOL["bf16"]
