"""ORACLE — test infrastructure only (see oracle/__init__.py).

Front end of the chunked prefill ("Qwen3.5-397B-A17B" trace page, section 1,
Prefill-GDN graph: node 8 gdn_gating turns the projections a, b into the gate
and beta; nodes 9 and 10 L2-normalise q and k), in fp64:

    q_bar = q / sqrt(sum_j q_j^2 + 1e-6)       (per token and head, over d_k)
    k_bar = k / sqrt(sum_j k_j^2 + 1e-6)
    g     = -exp(A_log[h]) * softplus(a[t, h] + dt_bias[h]),  softplus(x) = ln(1 + e^x)
    beta  = sigmoid(b[t, h])

The normalisation and gating nodes hand their results to the chunk kernels in
the activation dtype, so with ``round_to_bf16`` q_bar, k_bar and beta are
rounded to bf16 (round to nearest even); beta's sigmoid is first rounded to
fp32, the precision the page's kernels compute it in.  g stays fp64.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x):
    """fp64 -> fp32 -> bf16 (nearest even) -> fp64, elementwise (finite inputs)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def softplus(x):
    """ln(1 + e^x), elementwise, as max(x, 0) + ln(1 + e^-|x|) so that nothing overflows."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def l2_normalise(x):
    """x [..., d]: each row over the last axis divided by sqrt(sum x^2 + 1e-6)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)


def prefill_front_end(q, k, a, b, A_log, dt_bias, round_to_bf16):
    """q, k: [T, H_q, d_k] raw; a, b: [T, H_v]; A_log, dt_bias: [H_v].
    Returns (q_bar, k_bar, g, beta), fp64, with the dtype roundings above."""
    qn, kn = l2_normalise(q), l2_normalise(k)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    g = -np.exp(A_log)[None, :] * softplus(a + dt_bias[None, :])
    sig = (1.0 / (1.0 + np.exp(-b))).astype(np.float32).astype(np.float64)
    if round_to_bf16:
        return round_bf16(qn), round_bf16(kn), g, round_bf16(sig)
    return qn, kn, g, sig
