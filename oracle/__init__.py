"""ORACLE — test infrastructure only.

Plain CPU reference implementations of the Gated DeltaNet forward pass:

* ``forward`` / ``decode_step``: fp64 token-by-token recurrence (C, OpenMP),
  oracle/gdn_recurrence.c.  This is the definition the GPU path is judged against.
* ``chunk_form.chunk_forward``: an independent fp64 chunk-wise implementation
  (numpy, general dense inverse) exposing the per-chunk intermediates
  (cumulative gate, A, W, U, chunk-start state, U - W S).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and never imports it.

Pins (tests/test_oracle.py, run without a GPU): the recurrence and the chunk
form agree for C in {1, 2, 3, 16, 64, >= L} including ragged tails; beta = 0
reduces to pure decay (closed form); alpha = beta = 1 with unit keys makes
k_t S_t = v_t exactly and q_t = k_t reads back v_t; orthonormal keys with
alpha = beta = 1 give S = sum_t k_t^T v_t; the delta write equals one gradient
step on 1/2 ||k S - v||^2 (checked with torch autograd); the two algebraic
forms of the update agree; alpha = 1 reduces to DeltaNet; outputs are affine
in the initial state and linear in V when S0 = 0; GVA equals explicit head
repetition; splitting a sequence and passing the state equals running it whole;
a hand-derived d = 2 worked example (tests/golden/).

``decode_step_fused`` adds the decode front end (q/k L2 norm, gate from a,
A_log, dt_bias, beta from b).  Pins: softplus(x) - softplus(-x) = x and
softplus(0) = ln 2 through the returned gate (over |x| up to 60, where a
naive exponential would overflow), softplus(x) -> x and -> e^x in its tails, sigmoid's logit identity and exact bf16 representability
of the rounded beta, invariance of the step under scaling q or k (L2 norm),
zero keys reducing to pure decay, and the page's merged update
S' = alpha (I - beta k^T k) S + beta k^T v evaluated with numpy matrices.

``gated_rmsnorm`` is the read-out epilogue (oracle/gated_norm.py).  Pins:
invariance under scaling o (eps = 0), zero gate gives zero, the unit RMS of
the normalised read-out under a saturated gate, silu(z) - silu(-z) = z, and
linearity in the weight.

``prefill_front_end`` / ``forward_fused`` add the prefill front end (q/k L2
norm, gate and beta from the raw projections; oracle/front_end.py) before
``forward``.  Pins: the gate and beta equal those of the independent C decode
oracle (``decode_step_fused``) over gate inputs from -60 to 60; with fp32 inputs
``forward_fused`` over a sequence equals the C fused decode step applied token
by token; normalised rows have unit norm, are invariant under scaling the raw
row and keep zero rows zero; bf16-rounded results are exactly representable.

``conv_silu_varlen`` / ``conv_silu_step`` are the short causal convolution +
SiLU with its input history (oracle/conv.py).  Pins: numpy's convolve and
torch's grouped conv1d per channel, SiLU alone under the identity kernel,
splitting a sequence and passing the history, and the decode step against the
prefill of the same tokens.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import chunk_form  # noqa: F401
from .gated_norm import gated_rmsnorm  # noqa: F401
from .conv import conv_silu_step, conv_silu_varlen  # noqa: F401
from .front_end import prefill_front_end  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b

        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.gdn_oracle_forward.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, ctypes.c_double, P, P, P, P, I64,
                                       P, ctypes.c_int]
    lib.gdn_oracle_forward.restype = ctypes.c_int
    lib.gdn_oracle_decode_step.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, ctypes.c_double, P, P, P, I64,
                                           ctypes.c_int]
    lib.gdn_oracle_decode_step.restype = ctypes.c_int
    lib.gdn_oracle_decode_step_fused.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, I64, I64, I64, I64, I64,
                                                 ctypes.c_double, P, P, P, P, P, I64, ctypes.c_int]
    lib.gdn_oracle_decode_step_fused.restype = ctypes.c_int
    lib.gdn_oracle_max_threads.argtypes = []
    lib.gdn_oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


def forward(q, k, v, g, beta, cu_seqlens, H_q, H_v, scale, initial_state=None, heads=None,
            want_out=True, want_delta=False, num_threads=0):
    """fp64 recurrence over a packed batch.

    q, k: [T, H_q, d_k]; v: [T, H_v, d_v]; g, beta: [T, H_v] — any float arrays,
    converted to float32 (pass exact float32 / bf16-upcast values).
    initial_state: [N, H_v, d_k, d_v] (float64 after conversion) or None.
    heads: optional list of value heads to compute (others left zero).
    Returns (out [T, H_v, d_v] float64 or None, final [N, H_v, d_k, d_v] float64[, delta]).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    T, _, d_k = k.shape
    d_v = v.shape[2]
    N = len(cu) - 1
    s0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    out = np.zeros((T, H_v, d_v)) if want_out else None
    fin = np.zeros((N, H_v, d_k, d_v))
    hs = None if heads is None else np.ascontiguousarray(heads, dtype=np.int32)
    delta = np.zeros((T, H_v, d_v)) if want_delta else None
    rc = lib.gdn_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu), N, H_q, H_v, d_k, d_v,
                                float(scale), _ptr(s0), _ptr(out), _ptr(fin), _ptr(hs),
                                0 if hs is None else len(hs), _ptr(delta), int(num_threads))
    if rc != 0:
        raise ValueError("gdn_oracle_forward: bad arguments")
    if want_delta:
        return out, fin, delta
    return out, fin


def forward_fused(q, k, v, a, b, A_log, dt_bias, cu_seqlens, H_q, H_v, scale, round_to_bf16, initial_state=None,
                  heads=None, num_threads=0):
    """Prefill from the raw inputs: prefill_front_end, then forward (which takes
    its inputs as fp32, so q_bar, k_bar and g pass through one fp32 rounding).
    Returns (out, final) as forward does."""
    qn, kn, g, beta = prefill_front_end(q, k, a, b, A_log, dt_bias, round_to_bf16)
    return forward(qn, kn, v, g, beta, cu_seqlens, H_q, H_v, scale, initial_state=initial_state, heads=heads,
                   num_threads=num_threads)


def decode_step_fused(q, k, v, a, b, A_log, dt_bias, state, H_q, H_v, scale, beta_round_bf16, heads=None,
                      num_threads=0):
    """Decode step with the gate / beta / q-k normalisation front end
    (gdn_oracle_decode_step_fused).  q, k raw [N, H_q, d_k]; v [N, H_v, d_v];
    a, b [N, H_v]; A_log, dt_bias [H_v]; ``state`` float64 [N, H_v, d_k, d_v]
    updated in place.  Returns (out [N, H_v, d_v], g [N, H_v], beta [N, H_v])."""
    lib = _load()
    f32 = lambda x: np.ascontiguousarray(x, dtype=np.float32)
    q, k, v, a, b, A_log, dt_bias = map(f32, (q, k, v, a, b, A_log, dt_bias))
    if state.dtype != np.float64 or not state.flags["C_CONTIGUOUS"]:
        raise ValueError("state must be C-contiguous float64")
    N, _, d_k = k.shape
    d_v = v.shape[2]
    out = np.zeros((N, H_v, d_v))
    g = np.zeros((N, H_v))
    beta = np.zeros((N, H_v))
    hs = None if heads is None else np.ascontiguousarray(heads, dtype=np.int32)
    rc = lib.gdn_oracle_decode_step_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                                          int(bool(beta_round_bf16)), N, H_q, H_v, d_k, d_v, float(scale),
                                          _ptr(state), _ptr(out), _ptr(g), _ptr(beta), _ptr(hs),
                                          0 if hs is None else len(hs), int(num_threads))
    if rc != 0:
        raise ValueError("gdn_oracle_decode_step_fused: bad arguments")
    return out, g, beta


def decode_step(q, k, v, g, beta, state, H_q, H_v, scale, heads=None, num_threads=0):
    """One recurrent step for N sequences; ``state`` (float64 [N, H_v, d_k, d_v],
    C-contiguous) is updated in place.  Returns out [N, H_v, d_v] float64."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    if state.dtype != np.float64 or not state.flags["C_CONTIGUOUS"]:
        raise ValueError("state must be C-contiguous float64")
    N, _, d_k = k.shape
    d_v = v.shape[2]
    out = np.zeros((N, H_v, d_v))
    hs = None if heads is None else np.ascontiguousarray(heads, dtype=np.int32)
    rc = lib.gdn_oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), N, H_q, H_v, d_k, d_v,
                                    float(scale), _ptr(state), _ptr(out), _ptr(hs), 0 if hs is None else len(hs),
                                    int(num_threads))
    if rc != 0:
        raise ValueError("gdn_oracle_decode_step: bad arguments")
    return out
