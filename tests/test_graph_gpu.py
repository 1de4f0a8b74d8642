"""GPU: the forward + backward step captured in a HIP graph (torch.cuda.graph; the library
enqueues on torch's current stream, which is the capture stream) and replayed. Each replay,
with the program's own eager work and synchronisations between replays, must equal the eager
result bit for bit (the kernels are deterministic and the library records nothing but kernel
launches: no memset nodes)."""
import numpy as np
import pytest

from synth import make_case
from gdn_gpu import problem, to_device

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager():
    import torch
    import gated_delta_rule_34_amd as G

    case = make_case(1800, [300, 77, 0, 129], 2, 6, 128, dtype="bf16", chunk=64, gate="clamp09", with_S0=True,
                     with_dST=True, packed=True, varlen=True, name="graph")
    print(f"[graph] {case.name} lens={case.lens}", flush=True)
    d = to_device(case)
    p = problem(case, d)
    T, Hv, D, dev = case.T_total, case.Hv, case.Dk, d["v"].device
    o = torch.empty(T, Hv, D, dtype=torch.bfloat16, device=dev)
    S_T = torch.empty(case.N, Hv, D, D, device=dev)
    states = torch.empty(G.gdn_chunk_state_bytes(p), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(G.gdn_bwd_workspace_bytes(p), G.gdn_fwd_workspace_bytes(p)), dtype=torch.uint8, device=dev)
    dg = torch.empty(T, Hv, device=dev)
    dbeta = torch.empty(T, Hv, device=dev)
    dS0 = torch.empty(case.N, Hv, D, D, device=dev)

    def step():
        G.gdn_fwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], o, S_T, states, None)
        G.gdn_bwd(p, d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], states, d["dO"], d["dST"], d["dq"],
                  d["dk"], d["dv"], dg, dbeta, dS0, ws)

    def outs():
        return [t.clone() for t in (o, S_T, d["dq"], d["dk"], d["dv"], dg, dbeta, dS0)]

    step()
    torch.cuda.synchronize()
    eager = outs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (o, S_T, d["dq"], d["dk"], d["dv"], dg, dbeta, dS0):
            t.fill_(float("nan"))  # eager work between replays; the replay must rewrite everything
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(), eager):
            assert torch.equal(a, b), rep
        step()  # an eager step between replays
        torch.cuda.synchronize()
