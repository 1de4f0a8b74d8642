"""Float64 CPU oracle of the causal depthwise conv1d + SiLU (forward and input gradient).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: used by ``tests/`` and
``bench.py``'s CPU leg, never by the product package; it shares no code with the HIP path.

What it computes (the lattice-inference gdn_backward.rs page: conv1d_silu_fwd in
gdn_forward_save, and step 5 of gdn_backward, "Backward through conv1d + SiLU"): per
sequence (row range [a, b)), channel c and row t, with the rows before the sequence's
first taken as zero (the conv buffer starts empty),
    pre[t] = sum_{j < K} w[c, j] x[t - (K - 1) + j]          y[t] = pre[t] sigmoid(pre[t])
    dpre[t] = dy[t] sigmoid(pre[t]) (1 + pre[t] (1 - sigmoid(pre[t])))
    dx[t] = sum_{l < K} w[c, K - 1 - l] dpre[t + l]           (t + l < b)
Each sum is written over the lag l = K - 1 - j as a shifted copy of whole sequences.

Pins (tests/test_oracle.py): torch's conv1d (groups = channels, K - 1 zeros of left
padding) followed by silu, and torch autograd of it, on float64 CPU tensors; central
finite differences of ``conv1d_silu_fwd`` for the input gradient.
"""
from __future__ import annotations

import numpy as np


def _pre(cu, x, w):
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    K = w.shape[1]
    pre = np.zeros_like(x)
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        for j in range(K):
            lag = K - 1 - j  # x[t - lag] feeds pre[t] with weight w[:, j]
            if b - a > lag:
                pre[a + lag:b] += w[:, j] * x[a:b - lag]
    return pre


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def conv1d_silu_fwd(cu, x, w):
    """x [rows, channels], w [channels, K], cu row offsets [N + 1] -> y [rows, channels]."""
    pre = _pre(cu, x, w)
    return pre * _sigmoid(pre)


def conv1d_silu_bwd(cu, x, w, dy):
    """Input gradient dx [rows, channels] of the forward above for upstream dy."""
    w = np.asarray(w, np.float64)
    K = w.shape[1]
    pre = _pre(cu, x, w)
    sg = _sigmoid(pre)
    dpre = np.asarray(dy, np.float64) * sg * (1.0 + pre * (1.0 - sg))
    dx = np.zeros_like(pre)
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        for lag in range(K):
            if b - a > lag:
                dx[a:b - lag] += w[:, K - 1 - lag] * dpre[a + lag:b]
    return dx
