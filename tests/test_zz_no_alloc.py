"""GPU: gdn_fwd_noalloc (forward-only, workspace in the library's fixed per-GPU scratch array)
against gdn_fwd forward-only with a caller workspace, through the C ABI: bit-identical o and
S_T on two calls in a row, the second with a smaller problem (the scratch keeps the first
call's contents, which the second must not depend on)."""
import numpy as np
import pytest

from synth import make_case
from gdn_gpu import problem, to_device

pytestmark = pytest.mark.gpu


def _run(G, torch, case, noalloc):
    d = to_device(case)
    p = problem(case, d)
    T, Hv, D = case.T_total, case.Hv, case.Dk
    o = torch.empty(T, Hv, D, dtype=d["v"].dtype, device=d["v"].device)
    S_T = torch.empty(case.N, Hv, D, D, dtype=torch.float32, device=o.device)
    if noalloc:
        assert G.gdn_fwd_workspace_bytes(p) <= G.GDN_NOALLOC_SCRATCH_BYTES
        G.gdn_fwd_noalloc(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, S_T)
    else:
        ws = torch.full((G.gdn_fwd_workspace_bytes(p),), 0xAB, dtype=torch.uint8, device=o.device)
        G.gdn_fwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, S_T, None, ws)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S_T.cpu().numpy()


def test_fwd_noalloc_equals_fwd_only_twice():
    import torch
    import gated_delta_rule_34_amd as G

    big = make_case(1700, [2500, 700, 0, 33], 16, 48, 128, dtype="bf16", chunk=64, gate="clamp09", with_S0=True,
                    packed=True, varlen=True, name="noalloc-big")
    small = make_case(1701, [90, 40], 2, 6, 64, dtype="bf16", chunk=64, gate="clamp09", with_S0=True,
                      packed=True, varlen=True, name="noalloc-small")
    for case in (big, small):  # the second call is smaller: stale scratch contents must not matter
        print(f"[noalloc] {case.name} lens={case.lens}", flush=True)
        o_n, st_n = _run(G, torch, case, noalloc=True)
        o_w, st_w = _run(G, torch, case, noalloc=False)
        assert np.array_equal(o_n, o_w) and np.array_equal(st_n, st_w), case.name
        assert np.isfinite(o_n).all()
