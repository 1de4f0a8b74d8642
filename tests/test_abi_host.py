"""C ABI host-side contract (CPU only: no kernel is ever launched here).

The library loads, exports every function include/gdn.h declares, sizes its
workspaces, and rejects bad arguments with the documented status before it touches
the GPU. Every call below fails validation by construction; none reaches a launch.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def G():
    lib = os.path.join(ROOT, "gated_delta_rule_34_amd", "libgdn.so")
    if not os.path.exists(lib):
        import importlib.util

        spec = importlib.util.spec_from_file_location("_gdn_build", os.path.join(ROOT, "gated_delta_rule_34_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import gated_delta_rule_34_amd as G

    return G


def header_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(G):
    names = header_functions()
    assert set(names) == set(G.EXPORTED), names
    lib = ctypes.CDLL(G.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", G.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not exported as a text symbol"


def prob(G, **kw):
    base = dict(N=2, T_total=256, Hk=16, Hv=48, D=128, T=128, chunk=64, dtype="bf16")
    base.update(kw)
    N, T_total, Hk, Hv, D = (base.pop(k) for k in ("N", "T_total", "Hk", "Hv", "D"))
    return G.make_problem(N, T_total, Hk, Hv, D, **base)


def test_workspace_queries(G):
    p = prob(G)
    # forward-only calls keep T, M, the gate record and the chunk table in the workspace, but
    # not the chunk-start states and Delta that the saved buffer also holds
    nc, Hv, C = 2 * 2, 48, 64  # two sequences of two chunks
    assert G.gdn_fwd_workspace_bytes(p) >= nc * Hv * 2 * C * C * 2
    assert G.gdn_fwd_workspace_bytes(p) < G.gdn_chunk_state_bytes(p) - nc * Hv * 128 * 128 * 2
    assert G.gdn_bwd_workspace_bytes(p) > 0
    assert G.gdn_chunk_state_bytes(p) >= nc * Hv * 128 * 128 * 2
    bigger = prob(G, T_total=512, T=256)
    assert G.gdn_bwd_workspace_bytes(bigger) > G.gdn_bwd_workspace_bytes(p)
    bad = prob(G, Hv=47)
    assert G.gdn_fwd_workspace_bytes(bad) == 0
    assert G.gdn_bwd_workspace_bytes(bad) == 0
    assert G.gdn_chunk_state_bytes(bad) == 0


def test_strerror(G):
    for code in (0, -1, -2, -3, -4, -5):
        assert G.gdn_strerror(code)
    assert "unknown" in G.gdn_strerror(7)


class FakeTensor:
    """Stands in for a device tensor: a fixed address and 2-D row-view strides. It is
    never dereferenced, since every call below is rejected on the host."""

    def __init__(self, addr, rows, width, rs=None, nbytes=None):
        self.addr, self.shape, self._rs = addr, (rows, width), rs or width
        self._nbytes = nbytes

    def data_ptr(self):
        return self.addr

    def dim(self):
        return 2

    def stride(self, i):
        return (self._rs, 1)[i]

    def numel(self):
        return self._nbytes or 0

    def element_size(self):
        return 1


def fwd_args(G, p, **over):
    T = p.T_total
    a = dict(q=FakeTensor(0x10000, T, p.Hk * p.Dk, 10240), k=FakeTensor(0x20000, T, p.Hk * p.Dk, 10240),
             v=FakeTensor(0x30000, T, p.Hv * p.Dv, 10240), g=FakeTensor(0x40000, T, p.Hv),
             beta=FakeTensor(0x50000, T, p.Hv), S0=None, o=FakeTensor(0x60000, T, p.Hv * p.Dv),
             S_T=None, chunk_states=FakeTensor(0x70000, 1, 1), workspace=FakeTensor(0x80000, 1, 1, nbytes=16))
    a.update(over)
    return a


def status_of(G, p, **over):
    a = fwd_args(G, p, **over)
    with pytest.raises(G.GdnError) as e:
        G.gdn_fwd(p, a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["o"], a["S_T"], a["chunk_states"],
                  a["workspace"], stream=0)
    return e.value.status


def bwd_status_of(G, p, **over):
    a = fwd_args(G, p, **over)
    T = p.T_total
    qk = lambda base: FakeTensor(base, T, p.Hk * p.Dk, 10240)
    vv = lambda base: FakeTensor(base, T, p.Hv * p.Dv)
    with pytest.raises(G.GdnError) as e:
        G.gdn_bwd(p, a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["chunk_states"], vv(0x90000), None,
                  qk(0xA0000), qk(0xB0000), vv(0xC0000), FakeTensor(0xD0000, T, p.Hv), FakeTensor(0xE0000, T, p.Hv),
                  None, a["workspace"], stream=0)
    return e.value.status


def test_rejects_bad_problems(G):
    assert status_of(G, prob(G, Hv=47)) == G.GDN_EINVAL
    assert status_of(G, prob(G, D=96)) == G.GDN_EUNSUPPORTED
    assert status_of(G, prob(G, chunk=32)) == G.GDN_EUNSUPPORTED
    assert status_of(G, prob(G, dtype=5)) == G.GDN_EUNSUPPORTED
    assert status_of(G, prob(G, dtype="f32", D=64)) == G.GDN_EUNSUPPORTED  # f32 + chunk 64 needs D <= 32
    assert status_of(G, prob(G, T_total=255)) == G.GDN_EINVAL  # != N * T
    p = prob(G)
    p.Dv = 64
    assert status_of(G, p) == G.GDN_EUNSUPPORTED
    p = prob(G)
    p.scale = float("nan")
    assert status_of(G, p) == G.GDN_EINVAL


def test_l2norm_keeps_the_normalised_rows(G):
    p = prob(G)
    base = G.gdn_chunk_state_bytes(p)
    p.qk_l2norm = 1
    extra = 2 * p.T_total * p.Hk * p.Dk * 2 + p.T_total * p.Hk * 8  # q_hat, k_hat (bf16), two factors per head row
    assert G.gdn_chunk_state_bytes(p) >= base + extra
    assert G.gdn_chunk_state_bytes(p) < base + extra + 3 * 256  # each region rounded up to 256 bytes


def test_gate_chain_needs_both_parameters(G):
    p = prob(G)
    p.a_log = 0x88000  # dt_bias left NULL
    assert status_of(G, p) == G.GDN_EINVAL
    p.dt_bias = 0x88102  # misaligned
    assert status_of(G, p) == G.GDN_EALIGN


def test_rejects_bad_views(G):
    p = prob(G)
    T = p.T_total
    assert status_of(G, p, q=FakeTensor(0x10000, T, 2048, 1000)) == G.GDN_EINVAL  # row stride < width
    assert status_of(G, p, q=FakeTensor(0x10002, T, 2048, 10240)) == G.GDN_EALIGN
    assert status_of(G, p, v=FakeTensor(0x30000, T, 6144, 10241)) == G.GDN_EALIGN  # stride * 2 B % 16
    assert status_of(G, p, g=FakeTensor(0x40002, T, 48)) == G.GDN_EALIGN
    assert status_of(G, p, beta=None) == G.GDN_EINVAL
    # forward-only (no chunk states): the workspace must hold gdn_fwd_workspace_bytes
    assert status_of(G, p, chunk_states=None) == G.GDN_EWORKSPACE
    assert status_of(G, p, chunk_states=None, workspace=None) == G.GDN_EWORKSPACE
    big = G.gdn_fwd_workspace_bytes(p)
    assert status_of(G, p, chunk_states=None, workspace=FakeTensor(0x80010, 1, 1, nbytes=big)) == G.GDN_EALIGN
    assert status_of(G, p, chunk_states=FakeTensor(0x70008, 1, 1)) == G.GDN_EALIGN


def decode_status_of(G, p, n_slots=None, **over):
    N = p.N
    a = dict(q=FakeTensor(0x10000, N, p.Hk * p.Dk, 10240), k=FakeTensor(0x20000, N, p.Hk * p.Dk, 10240),
             v=FakeTensor(0x30000, N, p.Hv * p.Dv, 10240), g=FakeTensor(0x40000, N, p.Hv),
             beta=FakeTensor(0x50000, N, p.Hv), state=FakeTensor(0x70000, N if n_slots is None else n_slots, 1),
             slot_idx=None, o=FakeTensor(0x60000, N, p.Hv * p.Dv))
    a.update(over)
    with pytest.raises(G.GdnError) as e:
        G.gdn_decode(p, a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], a["slot_idx"], a["o"], stream=0)
    return e.value.status


def test_decode_rejects_bad_arguments(G):
    one = dict(N=4, T_total=4, T=1)
    assert decode_status_of(G, prob(G, N=4, T_total=8, T=2)) == G.GDN_EINVAL  # one token per row
    assert decode_status_of(G, prob(G, **one), n_slots=3) == G.GDN_EINVAL  # no slot map: slots >= rows
    assert decode_status_of(G, prob(G, **one, D=96)) == G.GDN_EUNSUPPORTED
    assert decode_status_of(G, prob(G, **one, Hv=47)) == G.GDN_EINVAL
    assert decode_status_of(G, prob(G, **one), state=FakeTensor(0x70004, 4, 1)) == G.GDN_EALIGN
    assert decode_status_of(G, prob(G, **one), state=None) == G.GDN_EINVAL
    assert decode_status_of(G, prob(G, **one), o=FakeTensor(0x60002, 4, 6144)) == G.GDN_EALIGN
    p = prob(G, **one)
    p.cu_seqlens = 0x90000
    assert decode_status_of(G, p) == G.GDN_EINVAL


def conv_status_of(G, p, backward=False, **over):
    R = p.T_total
    a = dict(x=FakeTensor(0x10000, R, p.channels, 10240), w=FakeTensor(0x20000, p.channels, p.kernel_size),
             y=FakeTensor(0x30000, R, p.channels, 10240), dy=FakeTensor(0x40000, R, p.channels, 10240),
             dx=FakeTensor(0x50000, R, p.channels, 10240))
    a.update(over)
    with pytest.raises(G.GdnError) as e:
        if backward:
            G.gdn_conv1d_silu_bwd(p, a["x"], a["w"], a["dy"], a["dx"], stream=0)
        else:
            G.gdn_conv1d_silu_fwd(p, a["x"], a["w"], a["y"], stream=0)
    return e.value.status


def test_conv_rejects_bad_arguments(G):
    cp = lambda **kw: G.make_conv_problem(**{**dict(N=2, T_total=64, channels=10240, kernel_size=4, T=32), **kw})
    assert conv_status_of(G, cp(kernel_size=5)) == G.GDN_EUNSUPPORTED
    assert conv_status_of(G, cp(kernel_size=0)) == G.GDN_EUNSUPPORTED
    assert conv_status_of(G, cp(channels=10236)) == G.GDN_EINVAL  # not a multiple of 8
    assert conv_status_of(G, cp(T=31)) == G.GDN_EINVAL  # N * T != T_total
    assert conv_status_of(G, cp(dtype=7)) == G.GDN_EUNSUPPORTED
    assert conv_status_of(G, cp(), x=FakeTensor(0x10002, 64, 10240, 10240)) == G.GDN_EALIGN
    assert conv_status_of(G, cp(), w=None) == G.GDN_EINVAL
    assert conv_status_of(G, cp(), y=FakeTensor(0x30000, 64, 10240, 1000)) == G.GDN_EINVAL  # stride < width
    assert conv_status_of(G, cp(), backward=True, dy=None) == G.GDN_EINVAL
    assert conv_status_of(G, cp(), backward=True, dx=FakeTensor(0x50004, 64, 10240, 10240)) == G.GDN_EALIGN


def test_rejects_small_workspace(G):
    p = prob(G)
    assert bwd_status_of(G, p) == G.GDN_EWORKSPACE
    assert bwd_status_of(G, p, workspace=None) == G.GDN_EWORKSPACE


def test_rejects_varlen_inconsistency(G):
    p = prob(G)
    p.N = 0
    p.cu_seqlens = 0x90000
    assert status_of(G, p) == G.GDN_EINVAL  # no sequences but rows


def test_fwd_noalloc_rejects_on_the_host(G):
    """gdn_fwd_noalloc checks its arguments like gdn_fwd, and a problem whose forward-only
    workspace exceeds the library's fixed scratch is rejected before anything runs."""
    def st(p, **over):
        a = fwd_args(G, p, **over)
        with pytest.raises(G.GdnError) as e:
            G.gdn_fwd_noalloc(p, a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["o"], a["S_T"], stream=0)
        return e.value.status

    big = prob(G, N=4, T_total=4 * 4096, T=4096)
    assert G.gdn_fwd_workspace_bytes(big) > G.GDN_NOALLOC_SCRATCH_BYTES
    assert st(big) == G.GDN_EWORKSPACE
    small = prob(G)
    assert G.gdn_fwd_workspace_bytes(small) <= G.GDN_NOALLOC_SCRATCH_BYTES
    assert st(small, beta=None) == G.GDN_EINVAL
    assert st(small, q=FakeTensor(0x10002, 256, 2048, 10240)) == G.GDN_EALIGN
    assert st(prob(G, Hv=47)) == G.GDN_EINVAL


def test_row_stride_of_empty_views(G):
    """A view with no rows has no layout to check (torch gives empty views arbitrary strides):
    the binding passes the row width as its stride; views with rows still need contiguous
    heads."""
    import torch

    empty = torch.empty(4, 3, 2, 32)[:0, 1]  # zero rows, strides of the parent
    assert G._rs(empty, 64) == 64
    assert G._rs(torch.empty(0, 64), 64) == 64
    with pytest.raises(ValueError):
        G._rs(torch.empty(3, 2, 32).transpose(1, 2), 64)
