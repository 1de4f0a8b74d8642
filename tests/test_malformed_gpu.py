"""GPU: a malformed device cu_seqlens table never makes a kernel touch rows outside the
caller's buffers.

include/gdn.h promises that device-side sequence offsets are clamped into [0, T_total], so a
table with a negative or decreasing entry gives wrong sequence boundaries but no access out
of bounds. Each buffer here is the middle of a larger allocation: input guard rows before and
after hold NaN (a read of them would reach the outputs as NaN) and output guard rows hold a
sentinel (a write to them would change it). The kernels' own clamps keep every access inside
the middle rows; the guards only turn a broken clamp into a failed assertion.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

GUARD = 8
SENT = 7.0


def _guarded(torch, rows, width, dtype, fill):
    full = torch.full((rows + 2 * GUARD, width), fill, dtype=dtype, device="cuda")
    return full, full[GUARD: GUARD + rows]


def _guards_hold(full, value):
    g = np.concatenate([full[:GUARD].float().cpu().numpy(), full[-GUARD:].float().cpu().numpy()])
    return bool(np.all(g == value))


BAD_TABLES = [[0, -5, 40, 30, 100], [0, 60, 20, 100, 100], [3, 50, 150, 70, 99]]


@pytest.mark.parametrize("cu", BAD_TABLES, ids=["negative", "decreasing", "past_end"])
@pytest.mark.parametrize("K", [2, 4])
def test_conv_malformed_table_stays_in_bounds(cu, K):
    import torch
    import gated_delta_rule_34_amd as G

    print(f"[malformed] conv cu={cu} K={K}", flush=True)
    T, ch = 100, 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    xf, x = _guarded(torch, T, ch, torch.bfloat16, float("nan"))
    x.copy_(torch.randn(T, ch, device="cuda", generator=gen))
    dyf, dy = _guarded(torch, T, ch, torch.bfloat16, float("nan"))
    dy.copy_(torch.randn(T, ch, device="cuda", generator=gen))
    yf, y = _guarded(torch, T, ch, torch.bfloat16, SENT)
    dxf, dx = _guarded(torch, T, ch, torch.bfloat16, SENT)
    w = torch.rand(ch, K, device="cuda", generator=gen) - 0.5
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    p = G.make_conv_problem(len(cu) - 1, T, ch, K, cu_seqlens=cu_d)
    G.gdn_conv1d_silu_fwd(p, x, w, y)
    G.gdn_conv1d_silu_bwd(p, x, w, dy, dx)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all() and torch.isfinite(dx.float()).all()
    assert _guards_hold(yf, SENT) and _guards_hold(dxf, SENT)


@pytest.mark.parametrize("cu", BAD_TABLES, ids=["negative", "decreasing", "past_end"])
def test_recurrence_malformed_table_stays_in_bounds(cu):
    import torch
    import gated_delta_rule_34_amd as G

    print(f"[malformed] recurrence cu={cu}", flush=True)
    T, Hk, Hv, D = 100, 2, 6, 64
    N = len(cu) - 1
    width = 2 * Hk * D + Hv * D
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    pf, packed = _guarded(torch, T, width, torch.bfloat16, float("nan"))
    packed.copy_(0.1 * torch.randn(T, width, device="cuda", generator=gen))
    q, k, v = packed[:, : Hk * D], packed[:, Hk * D: 2 * Hk * D], packed[:, 2 * Hk * D:]
    gf, g = _guarded(torch, T, Hv, torch.float32, float("nan"))
    g.copy_(0.9 + 0.1 * torch.rand(T, Hv, device="cuda", generator=gen))
    bf, beta = _guarded(torch, T, Hv, torch.float32, float("nan"))
    beta.copy_(torch.rand(T, Hv, device="cuda", generator=gen))
    dof, dO = _guarded(torch, T, Hv * D, torch.bfloat16, float("nan"))
    dO.copy_(torch.randn(T, Hv * D, device="cuda", generator=gen))
    of, o = _guarded(torch, T, Hv * D, torch.bfloat16, SENT)
    gbf, gb = _guarded(torch, T, width, torch.bfloat16, SENT)
    dq, dk, dv = gb[:, : Hk * D], gb[:, Hk * D: 2 * Hk * D], gb[:, 2 * Hk * D:]
    dgf, dg = _guarded(torch, T, Hv, torch.float32, SENT)
    dbf, dbeta = _guarded(torch, T, Hv, torch.float32, SENT)
    S_T = torch.empty(N, Hv, D, D, device="cuda")
    dS0 = torch.empty(N, Hv, D, D, device="cuda")
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
    p = G.make_problem(N, T, Hk, Hv, D, cu_seqlens=cu_d, chunk=64, dtype="bf16")
    # zero the buffers' contents first: the clamped table may leave some rows unwritten
    for t in (o, dq, dk, dv, dg, dbeta):
        t.zero_()
    states = torch.empty(G.gdn_chunk_state_bytes(p), dtype=torch.uint8, device="cuda")
    ws = torch.empty(G.gdn_bwd_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    G.gdn_fwd(p, q, k, v, g, beta, None, o, S_T, states, None)
    G.gdn_bwd(p, q, k, v, g, beta, None, states, dO, None, dq, dk, dv, dg, dbeta, dS0, ws)
    torch.cuda.synchronize()
    for t in (o, dq, dk, dv, dg, dbeta, S_T, dS0):
        assert torch.isfinite(t.float()).all()
    for full in (of, gbf, dgf, dbf):
        assert _guards_hold(full, SENT)
