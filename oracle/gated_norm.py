"""ORACLE — test infrastructure only (see oracle/__init__.py).

Head-wise gated RMSNorm of the GDN read-out ("Qwen3.5-397B-A17B" trace page,
Decode-GDN node 8, output_rmsnorm_silu_gate; the same operation sits after
chunk_output in the prefill graph, node 18), in fp64:

    y = o / sqrt(mean_j o_j^2 + eps) * weight * silu(z),   silu(z) = z * sigmoid(z)

The mean runs over the d_v channels of one value head (not the whole hidden
vector); the norm comes before the gate; weight multiplies directly (it is not
the 1 + w parameterisation of the outer norms on that page).  The page leaves
eps to the model configuration: it is an argument here.
"""
from __future__ import annotations

import numpy as np


def gated_rmsnorm(o, z, weight, eps):
    """o, z: [..., d_v]; weight: [d_v].  Returns fp64 [..., d_v]."""
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    rstd = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + float(eps))
    silu = z / (1.0 + np.exp(-z))
    return o * rstd * w * silu
