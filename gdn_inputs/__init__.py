"""Seeded synthetic inputs for the Gated DeltaNet forward pass.

This module is shared by the oracle-side tests and the HIP-side tests and
bench.  It draws random numbers and rounds them to the storage types; it holds
none of the method's arithmetic (no decay, no delta rule, no chunking).

Shapes and distributions follow the workloads the GDN prefill lab page
("实验三：GDN Prefill 前向优化", section 输入输出定义) fixes for the operator:
q, k are L2-normalised per (token, head) before they reach the operator, v is
given per value head, the gate arrives as log-decay g = ln(alpha) per token and
value head, beta is the write strength in (0, 1), and the optional initial state
has shape [N, H_v, d_k, d_v] (d_v contiguous).

Recipe (every config):
  * numpy ``default_rng(seed)`` (PCG64); fixed draw order
    lengths -> q -> k -> v -> alpha -> beta-logits -> initial state.
  * q, k ~ N(0, 1) drawn in float32, L2-normalised per (token, head) in float64,
    then rounded to the storage dtype (RNE to bf16, or float32).
  * v ~ N(0, 1), rounded to the storage dtype.
  * alpha ~ U(lo, hi); g = ln(alpha) stored float32.
  * beta = sigmoid(x), x ~ N(0, 1), stored float32.
  * initial state ~ N(0, std^2) stored float32 (std = 0.02), or zeros.

Every array handed to the GPU is also returned upcast exactly to float32 /
float64, so that both sides see identical values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# --------------------------------------------------------------------------
# bf16 helpers (storage rounding only)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return raw uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = (b + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact upcast of raw bfloat16 bits to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage dtype; returns uint16 bits for bf16, float32 otherwise."""
    if dtype == "bf16":
        return f32_to_bf16_bits(x.astype(np.float32))
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _l2_normalise_rows(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    n = np.sqrt(np.sum(x64 * x64, axis=-1, keepdims=True))
    n[n == 0] = 1.0
    return x64 / n


# --------------------------------------------------------------------------
# Prefill inputs
# --------------------------------------------------------------------------


@dataclasses.dataclass
class PrefillInputs:
    """One packed variable-length prefill batch.

    q, k: [T, H_q, d_k]; v: [T, H_v, d_v] in storage form (uint16 bf16 bits or
    float32); g, beta: [T, H_v] float32; cu_seqlens: int32 [N+1];
    initial_state: float32 [N, H_v, d_k, d_v] or None.
    """

    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    cu_seqlens: np.ndarray
    initial_state: Optional[np.ndarray]
    H_q: int
    H_v: int
    d_k: int
    d_v: int

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def N(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_k))

    # exact float32 views of what the GPU receives
    def q32(self) -> np.ndarray:
        return storage_to_f32(self.q, self.dtype)

    def k32(self) -> np.ndarray:
        return storage_to_f32(self.k, self.dtype)

    def v32(self) -> np.ndarray:
        return storage_to_f32(self.v, self.dtype)


def make_prefill(
    seed: int,
    seqlens,
    H_q: int,
    H_v: int,
    d_k: int,
    d_v: int,
    dtype: str = "bf16",
    alpha_range=(0.85, 0.999),
    state_std: Optional[float] = 0.02,
    beta_override: Optional[float] = None,
    g_override: Optional[float] = None,
    max_len: int = 8192,
) -> PrefillInputs:
    """Draw one prefill batch.  ``seqlens`` is a list of sequence lengths, or an int
    N meaning "draw N lengths uniform in [1, max_len]" (first draw of the stream)."""
    rng = np.random.default_rng(seed)
    if isinstance(seqlens, (int, np.integer)):
        seqlens = rng.integers(1, max_len + 1, size=int(seqlens))
    seqlens = np.asarray(seqlens, dtype=np.int64)
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    T = int(cu[-1])
    N = len(seqlens)

    q = rng.standard_normal((T, H_q, d_k), dtype=np.float32)
    q = round_to(_l2_normalise_rows(q), dtype)
    k = rng.standard_normal((T, H_q, d_k), dtype=np.float32)
    k = round_to(_l2_normalise_rows(k), dtype)
    v = round_to(rng.standard_normal((T, H_v, d_v), dtype=np.float32), dtype)
    alpha = rng.uniform(alpha_range[0], alpha_range[1], size=(T, H_v))
    g = np.log(alpha).astype(np.float32)
    blog = rng.standard_normal((T, H_v))
    beta = (1.0 / (1.0 + np.exp(-blog))).astype(np.float32)
    if state_std is None:
        s0 = None
    else:
        s0 = (rng.standard_normal((N, H_v, d_k, d_v), dtype=np.float32) * np.float32(state_std)).astype(np.float32)
    if beta_override is not None:
        beta[:] = np.float32(beta_override)
    if g_override is not None:
        g[:] = np.float32(g_override)
    return PrefillInputs(dtype, q, k, v, g, beta, cu, s0, H_q, H_v, d_k, d_v)


# --------------------------------------------------------------------------
# Decode inputs
# --------------------------------------------------------------------------


@dataclasses.dataclass
class DecodeToken:
    """One decode step for N sequences: q, k [N, H_q, d_k]; v [N, H_v, d_v];
    g, beta [N, H_v] float32."""

    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray

    def q32(self):
        return storage_to_f32(self.q, self.dtype)

    def k32(self):
        return storage_to_f32(self.k, self.dtype)

    def v32(self):
        return storage_to_f32(self.v, self.dtype)


def make_decode_token(seed: int, N: int, H_q: int, H_v: int, d_k: int, d_v: int,
                      dtype: str = "bf16", alpha_range=(0.85, 0.999)) -> DecodeToken:
    rng = np.random.default_rng(seed)
    q = round_to(_l2_normalise_rows(rng.standard_normal((N, H_q, d_k), dtype=np.float32)), dtype)
    k = round_to(_l2_normalise_rows(rng.standard_normal((N, H_q, d_k), dtype=np.float32)), dtype)
    v = round_to(rng.standard_normal((N, H_v, d_v), dtype=np.float32), dtype)
    alpha = rng.uniform(alpha_range[0], alpha_range[1], size=(N, H_v))
    g = np.log(alpha).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((N, H_v))))).astype(np.float32)
    return DecodeToken(dtype, q, k, v, g, beta)


@dataclasses.dataclass
class DecodeRawToken:
    """Raw inputs of one fused decode step: q, k [N, H_q, d_k] (not normalised),
    v [N, H_v, d_v], a, b [N, H_v] in the storage dtype; A_log, dt_bias [H_v] float32."""

    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    b: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray

    def f32(self, name):
        return storage_to_f32(getattr(self, name), self.dtype)


def make_decode_raw_token(seed: int, N: int, H_q: int, H_v: int, d_k: int, d_v: int,
                          dtype: str = "bf16") -> DecodeRawToken:
    """q, k, v, a, b ~ N(0, 1) (projection / convolution outputs, unnormalised);
    per value head A_log = ln U(1, 16) and dt_bias ~ U(-7, -2.3) (so the gate input
    a + dt_bias sits around the range of softplus used by decay rates)."""
    rng = np.random.default_rng(seed)
    q = round_to(rng.standard_normal((N, H_q, d_k), dtype=np.float32), dtype)
    k = round_to(rng.standard_normal((N, H_q, d_k), dtype=np.float32), dtype)
    v = round_to(rng.standard_normal((N, H_v, d_v), dtype=np.float32), dtype)
    a = round_to(rng.standard_normal((N, H_v), dtype=np.float32), dtype)
    b = round_to(rng.standard_normal((N, H_v), dtype=np.float32), dtype)
    A_log = np.log(rng.uniform(1.0, 16.0, size=H_v)).astype(np.float32)
    dt_bias = rng.uniform(-7.0, -2.3, size=H_v).astype(np.float32)
    return DecodeRawToken(dtype, q, k, v, a, b, A_log, dt_bias)


@dataclasses.dataclass
class PrefillRawInputs:
    """Raw inputs of the prefill with its front end: q, k [T, H_q, d_k] (not
    normalised), v [T, H_v, d_v], a, b [T, H_v] in the storage dtype; A_log,
    dt_bias [H_v] float32; cu_seqlens int32 [N+1]; initial_state float32
    [N, H_v, d_k, d_v] or None."""

    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    b: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    cu_seqlens: np.ndarray
    initial_state: Optional[np.ndarray]
    H_q: int
    H_v: int
    d_k: int
    d_v: int

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def N(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_k))

    def f32(self, name):
        return storage_to_f32(getattr(self, name), self.dtype)


def make_prefill_raw(seed: int, seqlens, H_q: int, H_v: int, d_k: int, d_v: int, dtype: str = "bf16",
                     state_std: Optional[float] = 0.02) -> PrefillRawInputs:
    """The decode raw-token recipe over a packed batch: q, k, v, a, b ~ N(0, 1)
    rounded to the storage dtype, A_log = ln U(1, 16), dt_bias ~ U(-7, -2.3) per
    value head, initial states ~ N(0, state_std^2)."""
    rng = np.random.default_rng(seed)
    seqlens = np.asarray(seqlens, dtype=np.int64)
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    T, N = int(cu[-1]), len(seqlens)
    q = round_to(rng.standard_normal((T, H_q, d_k), dtype=np.float32), dtype)
    k = round_to(rng.standard_normal((T, H_q, d_k), dtype=np.float32), dtype)
    v = round_to(rng.standard_normal((T, H_v, d_v), dtype=np.float32), dtype)
    a = round_to(rng.standard_normal((T, H_v), dtype=np.float32), dtype)
    b = round_to(rng.standard_normal((T, H_v), dtype=np.float32), dtype)
    A_log = np.log(rng.uniform(1.0, 16.0, size=H_v)).astype(np.float32)
    dt_bias = rng.uniform(-7.0, -2.3, size=H_v).astype(np.float32)
    s0 = None
    if state_std is not None:
        s0 = (rng.standard_normal((N, H_v, d_k, d_v), dtype=np.float32) * np.float32(state_std)).astype(np.float32)
    return PrefillRawInputs(dtype, q, k, v, a, b, A_log, dt_bias, cu, s0, H_q, H_v, d_k, d_v)


def make_gate(seed: int, rows: int, H_v: int, d_v: int, dtype: str = "bf16"):
    """Inputs of the gated RMSNorm read-out: z [rows, H_v, d_v] ~ N(0, 1) in the
    storage dtype, weight [d_v] ~ U(0.5, 1.5) float32."""
    rng = np.random.default_rng(seed)
    z = round_to(rng.standard_normal((rows, H_v, d_v), dtype=np.float32), dtype)
    w = rng.uniform(0.5, 1.5, size=d_v).astype(np.float32)
    return z, w


def make_conv(seed: int, T: int, C: int, K: int, N: int, dtype: str = "bf16", with_state: bool = True):
    """Inputs of the short causal convolution: x [T, C] ~ N(0, 1) and, if asked,
    histories [N, K-1, C] ~ N(0, 1) in the storage dtype; weight [C, K] ~ N(0, 1/K)
    and bias [C] ~ N(0, 0.1^2) float32."""
    rng = np.random.default_rng(seed)
    x = round_to(rng.standard_normal((T, C), dtype=np.float32), dtype)
    s0 = round_to(rng.standard_normal((N, K - 1, C), dtype=np.float32), dtype) if with_state else None
    w = (rng.standard_normal((C, K)) / np.sqrt(K)).astype(np.float32)
    b = (0.1 * rng.standard_normal(C)).astype(np.float32)
    return x, s0, w, b


def make_decode_state(seed: int, N: int, H_v: int, d_k: int, d_v: int, std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, H_v, d_k, d_v), dtype=np.float32) * np.float32(std)).astype(np.float32)


# --------------------------------------------------------------------------
# The named workloads (small parity case, headline prefill, packed varlen,
# long context, batched decode)
# --------------------------------------------------------------------------

WORKLOADS = {
    "tiny_f32_T100": dict(seed=1, seqlens=[100], H_q=2, H_v=2, d_k=64, d_v=64, dtype="f32",
                          alpha_range=(0.85, 0.999), state_std=None),
    "prefill_T4096": dict(seed=2, seqlens=[4096], H_q=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
                          alpha_range=(0.85, 0.999), state_std=0.02),
    "varlen_8seq": dict(seed=3, seqlens=8, H_q=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
                        alpha_range=(0.85, 0.999), state_std=0.02),
    "long_T65536": dict(seed=4, seqlens=[65536], H_q=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
                        alpha_range=(0.95, 0.9999), state_std=0.02),
    # a serving prefill batch of many short requests (lengths uniform in [1, 256])
    "many_256req": dict(seed=6, seqlens=256, max_len=256, H_q=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
                        alpha_range=(0.85, 0.999), state_std=0.02),
}

DECODE_WORKLOAD = dict(seed=5, N=256, H_q=16, H_v=32, d_k=128, d_v=128, dtype="bf16", steps=16,
                       alpha_range=(0.85, 0.999), state_std=0.02)


def make_workload(name: str) -> PrefillInputs:
    return make_prefill(**WORKLOADS[name])


def decode_step_seed(step: int) -> int:
    return 5000 + step
