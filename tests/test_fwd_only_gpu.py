"""GPU: the forward-only call (chunk_states NULL, a workspace instead).

It is the op that returns (o, S_T) and saves nothing for a backward. Its kernels are the
saving forward's with the saves switched off, so o and S_T must be bit-identical to the
saving forward's; they are also compared with the float64 oracle at the strided v_repeat 3
workload, and must not depend on what the workspace holds on entry.
"""
import numpy as np
import pytest

import oracle
from synth import config_case, make_case
from gdn_gpu import OUT_NAMES, compare, problem, to_device

pytestmark = pytest.mark.gpu


def _fwd(G, torch, case, d, p, save, ws_fill=None):
    T, Hv, D = case.T_total, case.Hv, case.Dk
    o = torch.empty(T, Hv, D, dtype=d["v"].dtype, device=d["v"].device)
    ws = None
    if not save:
        ws = torch.empty(max(G.gdn_fwd_workspace_bytes(p), 1), dtype=torch.uint8, device=o.device)
        if ws_fill is not None:
            ws.fill_(ws_fill)
    o, S_T, states = G.forward(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o=o, workspace=ws, save=save)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S_T.cpu().numpy()


CASES = [
    # name, lens, Hk, Hv, D, dtype, chunk, varlen
    ("bf16_varlen_r3_D128", [200, 0, 64, 1, 130], 2, 6, 128, "bf16", 64, True),
    ("bf16_D64_C16", [77, 77], 1, 2, 64, "bf16", 16, False),
    ("f32_D32_C64", [150], 2, 4, 32, "f32", 64, False),
    ("f32_D128_C16", [40, 40], 1, 1, 128, "f32", 16, False),
]


@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
def test_fwd_only_equals_saving_forward(spec):
    import torch
    import gated_delta_rule_34_amd as G

    name, lens, Hk, Hv, D, dtype, chunk, varlen = spec
    print(f"[fwd-only] {name}", flush=True)
    case = make_case(1300 + len(name), lens, Hk, Hv, D, dtype=dtype, chunk=chunk, gate="clamp09", with_S0=True,
                     packed=(dtype == "bf16"), varlen=varlen, name=name)
    d = to_device(case)
    p = problem(case, d)
    o_s, st_s = _fwd(G, torch, case, d, p, save=True)
    o_f, st_f = _fwd(G, torch, case, d, p, save=False, ws_fill=0xFF)  # NaN bytes in the workspace
    o_g, st_g = _fwd(G, torch, case, d, p, save=False, ws_fill=0x00)
    assert np.array_equal(o_s, o_f) and np.array_equal(st_s, st_f)
    assert np.array_equal(o_f, o_g) and np.array_equal(st_f, st_g)


def test_fwd_only_with_fused_norm_and_gate_chain():
    """Forward-only with the q/k L2 norm and the gate chain fused (the normalised rows then
    live in the workspace): bit-identical to the saving forward of the same problem."""
    import torch
    import gated_delta_rule_34_amd as G

    case = make_case(1401, [130, 70], 2, 6, 64, dtype="bf16", chunk=64, gate="clamp09", with_S0=True, packed=True,
                     varlen=True, name="fused")
    d = to_device(case)
    p = problem(case, d)
    dev = d["v"].device
    p.qk_l2norm = 1
    a_log = torch.linspace(-1.0, 0.0, case.Hv, device=dev)
    dt_bias = torch.full((case.Hv,), 0.5, device=dev)
    p.a_log, p.dt_bias = a_log.data_ptr(), dt_bias.data_ptr()
    d["q"].mul_(3.0)  # raw rows: not unit norm
    o_s, st_s = _fwd(G, torch, case, d, p, save=True)
    o_f, st_f = _fwd(G, torch, case, d, p, save=False, ws_fill=0xFF)
    assert np.array_equal(o_s, o_f) and np.array_equal(st_s, st_f)


@pytest.mark.parametrize("cfg", [2, 3])
def test_fwd_only_full_shape_against_oracle(cfg):
    """The strided v_repeat 3 workload (one sequence of 2048 tokens) and the training shape (4 x
    4096 tokens), Hk 16, Hv 48, D 128, packed bf16 rows, every head, against the float64 oracle
    at the bf16 bar."""
    import torch
    import gated_delta_rule_34_amd as G

    case = config_case(cfg)
    print(f"[fwd-only] {case.name}", flush=True)
    d = to_device(case)
    p = problem(case, d)
    o, st = _fwd(G, torch, case, d, p, save=False)
    gpu = {"o": o.astype(np.float64).reshape(case.T_total, case.Hv, case.Dk), "S_T": st.astype(np.float64)}
    ref = oracle.run_case(case, backward=False)
    errs = compare(case, gpu, ref, OUT_NAMES)
    print("   ", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
