"""gated_delta_rule_34_amd -- gated delta-net forward/backward on MI355X (gfx950).

Thin ctypes binding over the C ABI of ``include/gdn.h`` (``libgdn.so``, built in-tree
by ``gated_delta_rule_34_amd.build``). Functions keep the C names; this layer only
marshals arguments: PyTorch provides device memory and the current HIP stream, every
step of the computation runs in the library's HIP kernels. There is no CPU fallback:
importing fails loudly when the library has not been built.

Convenience wrappers ``forward`` / ``backward`` allocate outputs, the saved chunk
states and the workspace with torch and call ``gdn_fwd`` / ``gdn_bwd``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY may name another build of the same C ABI (the host-only sanitizer build of the
# argument checks, for instance); by default the in-tree libgdn.so is loaded.
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(_PKG, "libgdn.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EALIGN, GDN_EWORKSPACE, GDN_EHIP = 0, -1, -2, -3, -4, -5
GDN_F32, GDN_BF16 = 0, 1

EXPORTED = ("gdn_fwd", "gdn_fwd_noalloc", "gdn_bwd", "gdn_decode", "gdn_conv1d_silu_fwd", "gdn_conv1d_silu_bwd",
            "gdn_fwd_workspace_bytes", "gdn_bwd_workspace_bytes", "gdn_chunk_state_bytes", "gdn_strerror",
            "gdn_trace_enable", "gdn_trace_collect")


class gdn_trace_entry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("total_ms", ctypes.c_double), ("launches", ctypes.c_int64)]


class gdn_problem(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32),
        ("T", ctypes.c_int32),
        ("T_total", ctypes.c_int64),
        ("cu_seqlens", ctypes.c_void_p),
        ("Hk", ctypes.c_int32),
        ("Hv", ctypes.c_int32),
        ("Dk", ctypes.c_int32),
        ("Dv", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("a_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("qk_l2norm", ctypes.c_int32),
    ]


class gdn_conv_problem(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32),
        ("T", ctypes.c_int32),
        ("T_total", ctypes.c_int64),
        ("cu_seqlens", ctypes.c_void_p),
        ("channels", ctypes.c_int32),
        ("kernel_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python gated_delta_rule_34_amd/build.py, or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    prob = ctypes.POINTER(gdn_problem)
    for name in ("gdn_fwd_workspace_bytes", "gdn_bwd_workspace_bytes", "gdn_chunk_state_bytes"):
        fn = getattr(lib, name)
        fn.argtypes = [prob]
        fn.restype = SZ
    lib.gdn_fwd.argtypes = [prob, P, I64, P, I64, P, I64, P, P, P, P, I64, P, P, P, SZ, P]
    lib.gdn_fwd.restype = ctypes.c_int
    lib.gdn_fwd_noalloc.argtypes = [prob, P, I64, P, I64, P, I64, P, P, P, P, I64, P, P]
    lib.gdn_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_bwd.argtypes = [prob, P, I64, P, I64, P, I64, P, P, P, P, P, I64, P,
                            P, I64, P, I64, P, I64, P, P, P, P, SZ, P]
    lib.gdn_bwd.restype = ctypes.c_int
    lib.gdn_decode.argtypes = [prob, P, I64, P, I64, P, I64, P, P, P, ctypes.c_int32, P, P, I64, P]
    lib.gdn_decode.restype = ctypes.c_int
    cprob = ctypes.POINTER(gdn_conv_problem)
    lib.gdn_conv1d_silu_fwd.argtypes = [cprob, P, I64, P, P, I64, P]
    lib.gdn_conv1d_silu_fwd.restype = ctypes.c_int
    lib.gdn_conv1d_silu_bwd.argtypes = [cprob, P, I64, P, P, I64, P, I64, P]
    lib.gdn_conv1d_silu_bwd.restype = ctypes.c_int
    lib.gdn_trace_enable.argtypes = [ctypes.c_int]
    lib.gdn_trace_enable.restype = ctypes.c_int
    lib.gdn_trace_collect.argtypes = [ctypes.POINTER(gdn_trace_entry), ctypes.c_int]
    lib.gdn_trace_collect.restype = ctypes.c_int
    lib.gdn_strerror.argtypes = [ctypes.c_int]
    lib.gdn_strerror.restype = ctypes.c_char_p
    return lib


_lib = _load()


def gdn_strerror(status: int) -> str:
    return _lib.gdn_strerror(int(status)).decode()


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {gdn_strerror(status)} ({status})")
        self.status = status


def make_problem(N, T_total, Hk, Hv, D, *, T=None, cu_seqlens=None, chunk=64, scale=None, dtype="bf16",
                 a_log=None, dt_bias=None, qk_l2norm=False):
    """Build a gdn_problem. ``cu_seqlens``: device int32 tensor [N + 1] or None. ``a_log``,
    ``dt_bias``: device float32 tensors [Hv] (the fused gate chain: g and beta arguments then
    carry alpha and beta_raw) or None."""
    p = gdn_problem()
    p.N = int(N)
    p.T_total = int(T_total)
    p.T = int(T if T is not None else (T_total // N if (cu_seqlens is None and N) else 0))
    p.cu_seqlens = None if cu_seqlens is None else cu_seqlens.data_ptr()
    p.Hk, p.Hv, p.Dk, p.Dv = int(Hk), int(Hv), int(D), int(D)
    p.chunk = int(chunk)
    p.scale = float(scale if scale is not None else D ** -0.5)
    p.dtype = {"f32": GDN_F32, "bf16": GDN_BF16}[dtype] if isinstance(dtype, str) else int(dtype)
    p.a_log = None if a_log is None else a_log.data_ptr()
    p.dt_bias = None if dt_bias is None else dt_bias.data_ptr()
    p.qk_l2norm = 1 if qk_l2norm else 0
    return p


def gdn_trace_enable(on: bool) -> None:
    _lib.gdn_trace_enable(1 if on else 0)


def gdn_trace_collect(max_entries: int = 64) -> dict:
    """{kernel name: (total milliseconds, launches)} since the last collect."""
    buf = (gdn_trace_entry * max_entries)()
    n = _lib.gdn_trace_collect(buf, max_entries)
    return {buf[i].name.decode(): (buf[i].total_ms, int(buf[i].launches)) for i in range(n)}


def gdn_fwd_workspace_bytes(p: gdn_problem) -> int:
    return int(_lib.gdn_fwd_workspace_bytes(ctypes.byref(p)))


def gdn_bwd_workspace_bytes(p: gdn_problem) -> int:
    return int(_lib.gdn_bwd_workspace_bytes(ctypes.byref(p)))


def gdn_chunk_state_bytes(p: gdn_problem) -> int:
    return int(_lib.gdn_chunk_state_bytes(ctypes.byref(p)))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _rs(t, width):
    """Row stride (elements) of a [rows, width] or [rows, heads, D] view whose rows hold
    contiguous heads; the ABI requires exactly that inner layout."""
    if t is None:
        return 0
    if t.dim() in (2, 3) and t.shape[0] == 0:
        return width  # no row to address: any layout (torch gives empty views arbitrary strides)
    if t.dim() == 3:
        if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError("inner head layout must be contiguous")
    elif t.dim() == 2:
        if t.stride(1) != 1 or t.shape[1] != width:
            raise ValueError("rows must be contiguous")
    else:
        raise ValueError("expected a 2-D or 3-D row view")
    return t.stride(0)


def _stream(stream):
    import torch

    return stream if stream is not None else torch.cuda.current_stream().cuda_stream


def gdn_fwd(p, q, k, v, g, beta, S0, o, S_T, chunk_states, workspace, stream=None):
    """Call gdn_fwd on torch tensors (views). Raises GdnError on a non-OK status."""
    qk, vw = p.Hk * p.Dk, p.Hv * p.Dv
    st = _lib.gdn_fwd(ctypes.byref(p), _ptr(q), _rs(q, qk), _ptr(k), _rs(k, qk), _ptr(v), _rs(v, vw),
                      _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _rs(o, vw), _ptr(S_T), _ptr(chunk_states),
                      _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
                      _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_fwd")


GDN_NOALLOC_SCRATCH_BYTES = 64 << 20


def gdn_fwd_noalloc(p, q, k, v, g, beta, S0, o, S_T, stream=None):
    """Call gdn_fwd_noalloc (forward-only, workspace in the library's fixed per-GPU scratch)."""
    qk, vw = p.Hk * p.Dk, p.Hv * p.Dv
    st = _lib.gdn_fwd_noalloc(ctypes.byref(p), _ptr(q), _rs(q, qk), _ptr(k), _rs(k, qk), _ptr(v), _rs(v, vw),
                              _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _rs(o, vw), _ptr(S_T), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_fwd_noalloc")


def gdn_bwd(p, q, k, v, g, beta, S0, chunk_states, dO, dS_T, dq, dk, dv, dg, dbeta, dS0, workspace,
            stream=None):
    qk, vw = p.Hk * p.Dk, p.Hv * p.Dv
    st = _lib.gdn_bwd(ctypes.byref(p), _ptr(q), _rs(q, qk), _ptr(k), _rs(k, qk), _ptr(v), _rs(v, vw),
                      _ptr(g), _ptr(beta), _ptr(S0), _ptr(chunk_states), _ptr(dO), _rs(dO, vw), _ptr(dS_T),
                      _ptr(dq), _rs(dq, qk), _ptr(dk), _rs(dk, qk), _ptr(dv), _rs(dv, vw),
                      _ptr(dg), _ptr(dbeta), _ptr(dS0),
                      _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
                      _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_bwd")


def make_conv_problem(N, T_total, channels, kernel_size, *, T=None, cu_seqlens=None, dtype="bf16"):
    """Build a gdn_conv_problem. ``cu_seqlens``: device int32 tensor [N + 1] or None."""
    p = gdn_conv_problem()
    p.N, p.T_total = int(N), int(T_total)
    p.T = int(T if T is not None else (T_total // N if (cu_seqlens is None and N) else 0))
    p.cu_seqlens = None if cu_seqlens is None else cu_seqlens.data_ptr()
    p.channels, p.kernel_size = int(channels), int(kernel_size)
    p.dtype = {"f32": GDN_F32, "bf16": GDN_BF16}[dtype] if isinstance(dtype, str) else int(dtype)
    return p


def _rows(t):
    """Row stride (elements) of a [rows, channels] view with contiguous rows."""
    if t is None:
        return 0
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a [rows, channels] view with contiguous rows")
    return t.stride(0)


def gdn_conv1d_silu_fwd(p, x, w, y, stream=None):
    """Call gdn_conv1d_silu_fwd: y = SiLU(causal depthwise conv1d(x, w)) per sequence."""
    st = _lib.gdn_conv1d_silu_fwd(ctypes.byref(p), _ptr(x), _rows(x), _ptr(w), _ptr(y), _rows(y), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_conv1d_silu_fwd")


def gdn_conv1d_silu_bwd(p, x, w, dy, dx, stream=None):
    """Call gdn_conv1d_silu_bwd: dx from dy (the input gradient; the weights are fixed)."""
    st = _lib.gdn_conv1d_silu_bwd(ctypes.byref(p), _ptr(x), _rows(x), _ptr(w), _ptr(dy), _rows(dy), _ptr(dx),
                                  _rows(dx), _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_conv1d_silu_bwd")


def gdn_decode(p, q, k, v, g, beta, state, slot_idx, o, stream=None):
    """Call gdn_decode: one token per row (p.T == 1, p.T_total == p.N); ``state`` is the
    float32 [n_slots, Hv, Dk, Dv] pool updated in place, ``slot_idx`` an int32 [N] device
    tensor of slots or None (row n -> slot n). Raises GdnError on a non-OK status."""
    qk, vw = p.Hk * p.Dk, p.Hv * p.Dv
    n_slots = 0 if state is None else int(state.shape[0])
    st = _lib.gdn_decode(ctypes.byref(p), _ptr(q), _rs(q, qk), _ptr(k), _rs(k, qk), _ptr(v), _rs(v, vw),
                         _ptr(g), _ptr(beta), _ptr(state), n_slots, _ptr(slot_idx), _ptr(o), _rs(o, vw),
                         _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_decode")


def _empty_bytes(n, device):
    import torch

    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def forward(p, q, k, v, g, beta, S0=None, o=None, want_final=True, workspace=None, stream=None, save=True):
    """Allocate o, S_T and (``save``) the saved chunk states, run gdn_fwd; returns
    (o, S_T, states). With ``save=False`` the call is forward-only: nothing is saved for a
    backward (states is None) and the forward's factors live in a workspace."""
    import torch

    dev = v.device
    T = p.T_total
    if o is None:
        o = torch.empty(T, p.Hv, p.Dv, dtype=v.dtype, device=dev)
    S_T = torch.empty(p.N, p.Hv, p.Dk, p.Dv, dtype=torch.float32, device=dev) if want_final else None
    states = _empty_bytes(gdn_chunk_state_bytes(p), dev) if save else None
    if workspace is None and not save:
        workspace = _empty_bytes(gdn_fwd_workspace_bytes(p), dev)
    gdn_fwd(p, q, k, v, g, beta, S0, o, S_T, states, workspace, stream)
    return o, S_T, states


def backward(p, q, k, v, g, beta, S0, states, dO, dS_T=None, grads=None, want_dS0=True, workspace=None,
             stream=None):
    """Allocate gradients, run gdn_bwd; returns dict dq, dk, dv, dg, dbeta, dS0."""
    import torch

    dev = v.device
    T = p.T_total
    if grads is None:
        grads = dict(
            dq=torch.empty(T, p.Hk, p.Dk, dtype=v.dtype, device=dev),
            dk=torch.empty(T, p.Hk, p.Dk, dtype=v.dtype, device=dev),
            dv=torch.empty(T, p.Hv, p.Dv, dtype=v.dtype, device=dev),
            dg=torch.empty(T, p.Hv, dtype=torch.float32, device=dev),
            dbeta=torch.empty(T, p.Hv, dtype=torch.float32, device=dev),
            dS0=torch.empty(p.N, p.Hv, p.Dk, p.Dv, dtype=torch.float32, device=dev) if want_dS0 else None,
        )
    if workspace is None:
        workspace = _empty_bytes(gdn_bwd_workspace_bytes(p), dev)
    gdn_bwd(p, q, k, v, g, beta, S0, states, dO, dS_T, grads["dq"], grads["dk"], grads["dv"], grads["dg"],
            grads["dbeta"], grads["dS0"], workspace, stream)
    return grads
