"""ORACLE — test infrastructure only (see oracle/__init__.py).

Short causal depthwise convolution + SiLU with its rolling input history, in
fp64 ("Qwen3.5-397B-A17B" trace page, Decode-GDN node 6,
qkvzba_unpack_causal_conv1d_silu: x~_{t,c} = SiLU(sum_l w_{c,l} x_{t-l,c} + b_c),
no bias = 0; "Kestrel_VLLM - 24" page, section 三: the window is ordered oldest
first, [s_0, .., s_{K-2}, x_t], and the history keeps the convolution's raw
inputs, shifted by one each token).

Weights w [C, K] are indexed oldest first: w[c, K-1] multiplies the current
input, w[c, K-1-l] the input l tokens back.  The history ("conv state") of a
sequence is [K-1, C], row 0 the oldest input.
"""
from __future__ import annotations

import numpy as np


def _silu(x):
    return x / (1.0 + np.exp(-x))


def conv_silu_varlen(x, cu_seqlens, w, bias=None, initial_state=None):
    """x [T, C]; cu_seqlens [N+1]; w [C, K]; bias [C] or None;
    initial_state [N, K-1, C] or None (zeros).  Returns (y [T, C], final_state
    [N, K-1, C]) in fp64; final_state holds each sequence's last K-1 inputs
    (reaching into its initial state when the sequence is shorter)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, C = x.shape
    K = w.shape[1]
    N = len(cu_seqlens) - 1
    b = np.zeros(C) if bias is None else np.asarray(bias, dtype=np.float64)
    y = np.zeros((T, C))
    fin = np.zeros((N, K - 1, C))
    for n in range(N):
        t0, t1 = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        hist = np.zeros((K - 1, C)) if initial_state is None else np.asarray(initial_state[n], dtype=np.float64)
        seq = np.concatenate([hist, x[t0:t1]], axis=0)  # oldest first
        for t in range(t1 - t0):
            window = seq[t:t + K]                        # [K, C], row K-1 = current input
            y[t0 + t] = _silu(np.sum(window * w.T, axis=0) + b)
        fin[n] = seq[len(seq) - (K - 1):] if K > 1 else np.zeros((0, C))
    return y, fin


def conv_silu_step(x, w, bias, state):
    """One decode token for N sequences: x [N, C]; state [N, K-1, C] float64,
    updated in place (shift, append x).  Returns y [N, C] fp64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    C = x.shape[1]
    b = np.zeros(C) if bias is None else np.asarray(bias, dtype=np.float64)
    window = np.concatenate([state, x[:, None, :]], axis=1)  # [N, K, C]
    y = _silu(np.sum(window * w.T[None], axis=1) + b)
    state[:] = window[:, 1:]
    return y
