"""Pins for the oracle (CPU only).

Each test checks the fp64 oracle against something other than itself: the
independent chunk form, closed forms the pages' update rule implies, special
cases that reduce to the simpler rules on the same page (DeltaNet), torch
autograd, or a hand-derived worked example.  A plausible slip in the oracle
(a dropped decay, a wrong sign in the delta, k vs k^T, reading the state
before the update, a wrong GVA head, a cumulative gate that does not restart
per chunk) fails at least one of them.

Page cited throughout: "实验三：GDN Prefill 前向优化" (GDN prefill lab), sections
"GLA, DeltaNet 与 Gated DeltaNet", "Chunk-wise Parallel", "计算过程描述",
"输入输出定义".
"""
import json
import os

import numpy as np
import pytest

from oracle import chunk_form

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, T, H_q, H_v, dk, dv, unit=True, alpha=(0.85, 0.999)):
    q = rng.standard_normal((T, H_q, dk)).astype(np.float32)
    k = rng.standard_normal((T, H_q, dk)).astype(np.float32)
    if unit:
        q = (q / np.linalg.norm(q, axis=-1, keepdims=True)).astype(np.float32)
        k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((T, H_v, dv)).astype(np.float32)
    g = np.log(rng.uniform(alpha[0], alpha[1], (T, H_v))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((T, H_v))))).astype(np.float32)
    return q, k, v, g, beta


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------------------
# T1: recurrence == chunk form (independent algorithm), many C, ragged tails
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 100, 130])
@pytest.mark.parametrize("C", [1, 2, 3, 16, 64, 1000])
def test_recurrence_matches_chunk_form(oracle_mod, T, C):
    rng = np.random.default_rng(1000 * T + C)
    H_q, H_v, dk, dv = 2, 4, 8, 6
    q, k, v, g, beta = _rand_inputs(rng, T, H_q, H_v, dk, dv)
    s0 = rng.standard_normal((1, H_v, dk, dv)) * 0.3
    cu = np.array([0, T])
    scale = 1 / np.sqrt(dk)
    out, fin = oracle_mod.forward(q, k, v, g, beta, cu, H_q, H_v, scale, initial_state=s0)
    ref = chunk_form.chunk_forward(q, k, v, g, beta, cu, H_q, H_v, scale, initial_state=s0, C=C)
    assert _rel(out, ref["out"]) < 1e-12
    assert _rel(fin, ref["final_state"]) < 1e-12


def test_recurrence_matches_chunk_form_packed(oracle_mod):
    rng = np.random.default_rng(7)
    lens = [5, 64, 0, 129, 1, 70]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    H_q, H_v, dk, dv = 1, 2, 16, 16
    q, k, v, g, beta = _rand_inputs(rng, T, H_q, H_v, dk, dv)
    s0 = rng.standard_normal((len(lens), H_v, dk, dv)) * 0.1
    out, fin = oracle_mod.forward(q, k, v, g, beta, cu, H_q, H_v, 0.25, initial_state=s0)
    ref = chunk_form.chunk_forward(q, k, v, g, beta, cu, H_q, H_v, 0.25, initial_state=s0, C=64)
    assert _rel(out, ref["out"]) < 1e-12
    assert _rel(fin, ref["final_state"]) < 1e-12
    # a zero-length sequence hands its initial state straight through
    assert np.array_equal(fin[2], s0[2])


# ---------------------------------------------------------------------------
# T2: beta = 0 -> pure decay, closed form
# ---------------------------------------------------------------------------
def test_beta_zero_is_pure_decay(oracle_mod):
    rng = np.random.default_rng(2)
    T, H, dk, dv = 50, 2, 8, 8
    q, k, v, g, _ = _rand_inputs(rng, T, H, H, dk, dv)
    beta = np.zeros((T, H), np.float32)
    s0 = rng.standard_normal((1, H, dk, dv))
    scale = 0.5
    out, fin = oracle_mod.forward(q, k, v, g, beta, [0, T], H, H, scale, initial_state=s0)
    gam = np.exp(np.cumsum(g.astype(np.float64), axis=0))  # [T, H]
    for h in range(H):
        assert _rel(fin[0, h], gam[-1, h] * s0[0, h]) < 1e-14
        exp_o = scale * gam[:, h, None] * (q[:, h, :].astype(np.float64) @ s0[0, h])
        assert _rel(out[:, h, :], exp_o) < 1e-13


# ---------------------------------------------------------------------------
# T3: alpha = beta = 1, unit key -> k_t S_t = v_t exactly; q = k reads v back
# ---------------------------------------------------------------------------
def test_full_replacement_with_unit_keys(oracle_mod):
    rng = np.random.default_rng(3)
    T, dk, dv = 20, 64, 8
    k = np.zeros((T, 1, dk), np.float32)
    for t in range(T):
        # exactly unit norm in binary: 64 entries of +-1/8
        k[t, 0, :] = rng.choice([-0.125, 0.125], size=dk)
    q = k.copy()
    v = rng.standard_normal((T, 1, dv)).astype(np.float32)
    g = np.zeros((T, 1), np.float32)
    beta = np.ones((T, 1), np.float32)
    s0 = rng.standard_normal((1, 1, dk, dv))
    out, _, delta = oracle_mod.forward(q, k, v, g, beta, [0, T], 1, 1, 1.0, initial_state=s0, want_delta=True)
    # o_t = q_t S_t = k_t S_t = v_t
    assert np.max(np.abs(out[:, 0, :] - v[:, 0, :])) < 1e-13


def test_orthonormal_keys_write_exact_associations(oracle_mod):
    from scipy.linalg import hadamard

    rng = np.random.default_rng(4)
    dk, dv = 16, 5
    # Sylvester-Hadamard rows scaled by 1/4: exactly orthonormal in binary arithmetic
    Km = hadamard(dk).astype(np.float64) / 4.0
    Km = Km[rng.permutation(dk)]
    k = Km.astype(np.float32)[:, None, :]
    v = rng.standard_normal((dk, 1, dv)).astype(np.float32)
    g = np.zeros((dk, 1), np.float32)
    beta = np.ones((dk, 1), np.float32)
    s0 = rng.standard_normal((1, 1, dk, dv))
    _, fin = oracle_mod.forward(k, k, v, g, beta, [0, dk], 1, 1, 1.0, initial_state=s0)
    # each write replaces the association of its key; orthogonal keys do not
    # interfere, and a full orthonormal basis erases S0: S = sum_t k_t^T v_t
    expect = Km.T @ v[:, 0, :].astype(np.float64)
    assert _rel(fin[0, 0], expect) < 1e-13


# ---------------------------------------------------------------------------
# The delta write is one gradient step on 1/2 ||k S - v||^2 (torch autograd)
# ---------------------------------------------------------------------------
def test_delta_rule_is_gradient_step(oracle_mod):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    dk, dv = 7, 9
    q, k, v, g, beta = _rand_inputs(rng, 1, 1, 1, dk, dv)
    s0 = rng.standard_normal((1, 1, dk, dv))
    _, fin = oracle_mod.forward(q, k, v, g, beta, [0, 1], 1, 1, 1.0, initial_state=s0)
    alpha = float(np.exp(np.float64(g[0, 0])))
    Sbar = torch.tensor(alpha * s0[0, 0], dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k[0, 0].astype(np.float64))[None, :]
    vt = torch.tensor(v[0, 0].astype(np.float64))[None, :]
    loss = 0.5 * ((kt @ Sbar - vt) ** 2).sum()
    loss.backward()
    expect = (Sbar - float(beta[0, 0]) * Sbar.grad).detach().numpy()
    assert _rel(fin[0, 0], expect) < 1e-13


# ---------------------------------------------------------------------------
# T4 / T5: the product form alpha (I - beta k^T k) S + beta k^T v, and alpha = 1
# reduces to DeltaNet (v_hat = k S_{t-1}; S_t = S_{t-1} + beta k^T (v - v_hat))
# ---------------------------------------------------------------------------
def test_product_form_agrees(oracle_mod):
    rng = np.random.default_rng(6)
    T, dk, dv = 40, 6, 4
    q, k, v, g, beta = _rand_inputs(rng, T, 1, 1, dk, dv)
    s0 = rng.standard_normal((1, 1, dk, dv))
    out, fin = oracle_mod.forward(q, k, v, g, beta, [0, T], 1, 1, 0.7, initial_state=s0)
    S = s0[0, 0].copy()
    I = np.eye(dk)
    for t in range(T):
        kt = k[t, 0].astype(np.float64)[None, :]
        vt = v[t, 0].astype(np.float64)[None, :]
        a = np.exp(np.float64(g[t, 0]))
        b = np.float64(beta[t, 0])
        S = a * (I - b * kt.T @ kt) @ S + b * kt.T @ vt
        assert _rel(out[t, 0], 0.7 * (q[t, 0].astype(np.float64) @ S)) < 1e-12
    assert _rel(fin[0, 0], S) < 1e-12


def test_alpha_one_is_deltanet(oracle_mod):
    rng = np.random.default_rng(8)
    T, dk, dv = 33, 5, 3
    q, k, v, _, beta = _rand_inputs(rng, T, 1, 1, dk, dv)
    g = np.zeros((T, 1), np.float32)
    out, fin = oracle_mod.forward(q, k, v, g, beta, [0, T], 1, 1, 1.0)
    S = np.zeros((dk, dv))
    for t in range(T):
        kt = k[t, 0].astype(np.float64)
        vhat = kt @ S
        S = S + beta[t, 0] * np.outer(kt, v[t, 0] - vhat)
        assert _rel(out[t, 0], q[t, 0].astype(np.float64) @ S) < 1e-12
    assert _rel(fin[0, 0], S) < 1e-12


# ---------------------------------------------------------------------------
# Hand-derived worked example, d_k = d_v = 2, two tokens, scale 1.
#   S0 = I. Token 1: k=[1,0], v=[2,3], q=[0,1], alpha=1/2, beta=1/2
#     Sbar = I/2; k Sbar = [1/2, 0]; delta = (1/2)([2,3]-[1/2,0]) = [3/4, 3/2]
#     S1 = [[5/4, 3/2], [0, 1/2]];  o1 = q S1 = [0, 1/2]
#   Token 2: k=[0.6,0.8], v=[1,-1], q=[1,1], alpha=1, beta=1
#     k S1 = [0.75, 1.3]; delta = [0.25, -2.3]
#     S2 = S1 + k^T delta = [[1.4, 0.12], [0.2, -1.34]];  o2 = [1.6, -1.22]
# ---------------------------------------------------------------------------
def test_worked_example_d2(oracle_mod):
    q = np.array([[[0, 1]], [[1, 1]]], np.float32)
    k = np.array([[[1, 0]], [[0.6, 0.8]]], np.float32)
    v = np.array([[[2, 3]], [[1, -1]]], np.float32)
    g = np.log(np.array([[0.5], [1.0]])).astype(np.float32)
    beta = np.array([[0.5], [1.0]], np.float32)
    s0 = np.eye(2)[None, None]
    out, fin = oracle_mod.forward(q, k, v, g, beta, [0, 2], 1, 1, 1.0, initial_state=s0)
    # 0.6/0.8 are fp32-rounded, so allow their rounding (~3e-8 relative)
    np.testing.assert_allclose(out[:, 0, :], [[0, 0.5], [1.6, -1.22]], atol=1e-6)
    np.testing.assert_allclose(fin[0, 0], [[1.4, 0.12], [0.2, -1.34]], atol=1e-6)


# ---------------------------------------------------------------------------
# T8: GVA == explicit repetition of the query/key heads
# ---------------------------------------------------------------------------
def test_gva_equals_head_repetition(oracle_mod):
    rng = np.random.default_rng(9)
    T, H_q, G, dk, dv = 70, 2, 3, 8, 8
    H_v = H_q * G
    q, k, v, g, beta = _rand_inputs(rng, T, H_q, H_v, dk, dv)
    out, fin = oracle_mod.forward(q, k, v, g, beta, [0, T], H_q, H_v, 0.3)
    q_rep = np.repeat(q, G, axis=1)
    k_rep = np.repeat(k, G, axis=1)
    out2, fin2 = oracle_mod.forward(q_rep, k_rep, v, g, beta, [0, T], H_v, H_v, 0.3)
    assert np.array_equal(out, out2)
    assert np.array_equal(fin, fin2)


# ---------------------------------------------------------------------------
# T9: affine in S0; linear in V from a zero state
# ---------------------------------------------------------------------------
def test_affine_in_initial_state_and_linear_in_v(oracle_mod):
    rng = np.random.default_rng(10)
    T, H, dk, dv = 45, 1, 6, 6
    q, k, v, g, beta = _rand_inputs(rng, T, H, H, dk, dv)
    sa = rng.standard_normal((1, H, dk, dv))
    sb = rng.standard_normal((1, H, dk, dv))
    f = lambda s, vv=v: oracle_mod.forward(q, k, vv, g, beta, [0, T], H, H, 1.0, initial_state=s)
    oab, fab = f(sa + sb)
    ob, fb = f(sb)
    oa, fa = f(sa)
    o0, f0 = f(None)
    assert _rel(oab - ob, oa - o0) < 1e-10
    assert _rel(fab - fb, fa - f0) < 1e-10
    v2 = (2 * v).astype(np.float32)
    o2, f2 = f(None, v2)
    assert _rel(o2, 2 * o0) < 1e-13 and _rel(f2, 2 * f0) < 1e-13


# ---------------------------------------------------------------------------
# T6 / T7 / T11: split + state passing; packed == separate; decode continues prefill
# ---------------------------------------------------------------------------
def test_split_sequence_and_packing(oracle_mod):
    rng = np.random.default_rng(11)
    T, H_q, H_v, dk, dv = 150, 1, 2, 8, 4
    q, k, v, g, beta = _rand_inputs(rng, T, H_q, H_v, dk, dv)
    s0 = rng.standard_normal((1, H_v, dk, dv))
    out, fin = oracle_mod.forward(q, k, v, g, beta, [0, T], H_q, H_v, 0.5, initial_state=s0)
    s = 77
    o1, f1 = oracle_mod.forward(q[:s], k[:s], v[:s], g[:s], beta[:s], [0, s], H_q, H_v, 0.5, initial_state=s0)
    o2, f2 = oracle_mod.forward(q[s:], k[s:], v[s:], g[s:], beta[s:], [0, T - s], H_q, H_v, 0.5, initial_state=f1)
    assert np.array_equal(np.concatenate([o1, o2]), out)
    assert np.array_equal(f2, fin)
    # packed as two sequences (second starts from the first's final state) == separate runs
    op, fp = oracle_mod.forward(q, k, v, g, beta, [0, s, T], H_q, H_v, 0.5,
                                initial_state=np.concatenate([s0, f1]))
    assert np.array_equal(op, out) and np.array_equal(fp[1], fin[0])
    # decode step continues the prefill exactly
    st = f1.copy()
    o_dec = oracle_mod.decode_step(q[s:s + 1], k[s:s + 1], v[s:s + 1], g[s:s + 1], beta[s:s + 1], st, H_q, H_v, 0.5)
    assert np.array_equal(o_dec[0], out[s])
    o3, f3 = oracle_mod.forward(q[:s + 1], k[:s + 1], v[:s + 1], g[:s + 1], beta[:s + 1], [0, s + 1], H_q, H_v, 0.5,
                                initial_state=s0)
    assert np.array_equal(st, f3)


def test_decode_step_matches_single_token_sequences(oracle_mod):
    rng = np.random.default_rng(12)
    N, H_q, H_v, dk, dv = 5, 2, 4, 8, 8
    q, k, v, g, beta = _rand_inputs(rng, N, H_q, H_v, dk, dv)
    s0 = rng.standard_normal((N, H_v, dk, dv))
    st = s0.copy()
    o = oracle_mod.decode_step(q, k, v, g, beta, st, H_q, H_v, 0.3)
    out, fin = oracle_mod.forward(q, k, v, g, beta, np.arange(N + 1), H_q, H_v, 0.3, initial_state=s0)
    assert np.array_equal(o, out)
    assert np.array_equal(st, fin)
    # head subset computes only the listed heads, identically
    st2 = s0.copy()
    o2 = oracle_mod.decode_step(q, k, v, g, beta, st2, H_q, H_v, 0.3, heads=[3, 1])
    assert np.array_equal(o2[:, [1, 3]], o[:, [1, 3]])
    assert np.array_equal(st2[:, [0, 2]], s0[:, [0, 2]])


# ---------------------------------------------------------------------------
# T13: with unit keys and beta in (0,1), ||S_t||_2 <= alpha ||S_{t-1}||_2 + beta ||v_t||
# ---------------------------------------------------------------------------
def test_state_norm_bound(oracle_mod):
    rng = np.random.default_rng(13)
    T, dk, dv = 400, 8, 8
    q, k, v, g, beta = _rand_inputs(rng, T, 1, 1, dk, dv, alpha=(0.95, 0.9999))
    st = rng.standard_normal((1, 1, dk, dv))
    prev = np.linalg.norm(st[0, 0], 2)
    for t in range(T):
        oracle_mod.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], st, 1, 1, 1.0)
        cur = np.linalg.norm(st[0, 0], 2)
        a = np.exp(np.float64(g[t, 0]))
        kn = np.linalg.norm(k[t, 0].astype(np.float64))
        # with ||k|| = 1 up to fp32 rounding the bound holds to ~1e-7 relative
        assert cur <= a * prev * (1 + 1e-6) + beta[t, 0] * kn * np.linalg.norm(v[t, 0].astype(np.float64)) + 1e-12
        prev = cur


# ---------------------------------------------------------------------------
# Chunk-form intermediates obey their defining identities
# ---------------------------------------------------------------------------
def test_chunk_intermediates_identities():
    rng = np.random.default_rng(14)
    T, dk, dv = 100, 8, 8
    q, k, v, g, beta = _rand_inputs(rng, T, 1, 1, dk, dv)
    s0 = rng.standard_normal((1, 1, dk, dv))
    res = chunk_form.chunk_forward(q, k, v, g, beta, [0, T], 1, 1, 1.0, initial_state=s0, keep_intermediates=True)
    recs = res["chunks"][(0, 0)]
    assert len(recs) == 2 and recs[1]["A"].shape == (36, 36)
    for c, r in enumerate(recs):
        ell = r["A"].shape[0]
        # A is unit lower triangular
        assert np.allclose(np.diag(r["A"]), 1.0) and np.allclose(np.triu(r["A"], 1), 0.0)
        # cumulative gate restarts at the chunk start
        np.testing.assert_allclose(r["gc"], np.cumsum(g[c * 64:c * 64 + ell, 0].astype(np.float64)))
    np.testing.assert_allclose(recs[0]["h"], s0[0, 0])


def test_chunk_X_is_per_token_delta(oracle_mod):
    """U - W S equals the per-token write beta (v - k Sbar) of the recurrence."""
    rng = np.random.default_rng(15)
    T, dk, dv = 90, 8, 8
    q, k, v, g, beta = _rand_inputs(rng, T, 1, 2, dk, dv)
    s0 = rng.standard_normal((1, 2, dk, dv))
    _, _, delta = oracle_mod.forward(q, k, v, g, beta, [0, T], 1, 2, 1.0, initial_state=s0, want_delta=True)
    res = chunk_form.chunk_forward(q, k, v, g, beta, [0, T], 1, 2, 1.0, initial_state=s0, keep_intermediates=True)
    for h in range(2):
        X = np.concatenate([r["X"] for r in res["chunks"][(0, h)]])
        assert _rel(X, delta[:, h, :]) < 1e-12


# ---------------------------------------------------------------------------
# Stored fixture (written by tests/golden/make_golden.py from the oracle): guards
# the oracle against silent change
# ---------------------------------------------------------------------------
def test_golden_fixture(oracle_mod):
    with open(os.path.join(GOLDEN, "oracle_tiny_d8.json")) as f:
        fx = json.load(f)
    a = {kk: np.array(vv, dtype=np.float64) for kk, vv in fx["arrays"].items()}
    out, fin = oracle_mod.forward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"].astype(np.int64),
                                  fx["H_q"], fx["H_v"], fx["scale"], initial_state=a["initial_state"])
    assert _rel(out, a["out"]) < 1e-13
    assert _rel(fin, a["final_state"]) < 1e-13


def test_bad_arguments_rejected(oracle_mod):
    q = np.zeros((2, 3, 4), np.float32)
    with pytest.raises(ValueError):
        oracle_mod.forward(q, q, np.zeros((2, 4, 4), np.float32), np.zeros((2, 4), np.float32),
                           np.zeros((2, 4), np.float32), [0, 2], 3, 4, 1.0)


# ---------------------------------------------------------------------------
# Decode front end ("Qwen3.5-397B-A17B" trace page, Decode-GDN node 7, steps 1
# and 2; softplus branches of the "Kestrel_VLLM - 24" page, section 三)
# ---------------------------------------------------------------------------
def _fused_inputs(rng, N, H_q, H_v, d, a_scale=2.0):
    q = rng.standard_normal((N, H_q, d)).astype(np.float32)
    k = rng.standard_normal((N, H_q, d)).astype(np.float32)
    v = rng.standard_normal((N, H_v, d)).astype(np.float32)
    a = (a_scale * rng.standard_normal((N, H_v))).astype(np.float32)
    b = (2.0 * rng.standard_normal((N, H_v))).astype(np.float32)
    A_log = rng.uniform(-1.0, 1.0, H_v).astype(np.float32)
    dt_bias = rng.uniform(-0.5, 0.5, H_v).astype(np.float32)
    S = 0.1 * rng.standard_normal((N, H_v, d, d))
    return q, k, v, a, b, A_log, dt_bias, S


def _fused(oracle_mod, q, k, v, a, b, A_log, dt_bias, S, H_q, H_v, scale=0.125, rnd=False):
    S = np.ascontiguousarray(S, dtype=np.float64).copy()
    out, g, beta = oracle_mod.decode_step_fused(q, k, v, a, b, A_log, dt_bias, S, H_q, H_v, scale, rnd)
    return out, g, beta, S


def test_fused_gate_softplus_identities(oracle_mod):
    """With A_log = 0 the gate is -softplus(a + dt_bias): softplus(x) - softplus(-x) = x
    for |x| up to 60 (where e^x of a naive form overflows fp32's range of the
    kernels and would lose everything in fp64's tails), softplus(0) = ln 2, and the
    tails: softplus(x) - x = ln(1 + e^-x) ~ e^-x for large x, softplus(x) ~ e^x
    for very negative x."""
    x = np.concatenate([np.linspace(-59.5, 59.5, 239), [0.0]]).astype(np.float32)
    N, H = len(x), 1
    zeros = np.zeros(1, np.float32)
    q = np.ones((N, 1, 2), np.float32)
    k = np.ones((N, 1, 2), np.float32)
    v = np.ones((N, 1, 2), np.float32)
    S = np.zeros((N, 1, 2, 2))
    _, gp, _, _ = _fused(oracle_mod, q, k, v, x[:, None], np.zeros((N, H), np.float32), zeros, zeros, S, 1, 1)
    _, gm, _, _ = _fused(oracle_mod, q, k, v, -x[:, None], np.zeros((N, H), np.float32), zeros, zeros, S, 1, 1)
    np.testing.assert_allclose(-gp[:, 0] + gm[:, 0], x.astype(np.float64), rtol=0, atol=1e-12)
    assert abs(-gp[-1, 0] - np.log(2.0)) < 1e-15
    big = np.array([20.5, 30.0, 60.0, -20.5, -30.0, -60.0], np.float32)
    M = len(big)
    _, gb, _, _ = _fused(oracle_mod, q[:M], k[:M], v[:M], big[:, None], np.zeros((M, H), np.float32), zeros, zeros,
                         S[:M], 1, 1)
    xb = big.astype(np.float64)
    pos = xb > 0
    # tails: e^-|x| (1 - e^-|x| / 2) approximates ln(1 + e^-|x|) to within e^(-3|x|) / 3
    tail = np.exp(-np.abs(xb)) * (1.0 - 0.5 * np.exp(-np.abs(xb)))
    np.testing.assert_allclose(-gb[pos, 0], xb[pos] + tail[pos], rtol=4e-16, atol=0)  # fp64 rounding of x + tail
    np.testing.assert_allclose(-gb[~pos, 0], tail[~pos], rtol=1e-12, atol=0)
    # the learned scale multiplies: A_log = ln 3 triples the gate
    _, g3, _, _ = _fused(oracle_mod, q, k, v, x[:, None], np.zeros((N, H), np.float32),
                         np.array([np.log(3.0)], np.float32), zeros, S, 1, 1)
    np.testing.assert_allclose(g3[:, 0], 3.0 * gp[:, 0] * np.exp(np.float64(np.float32(np.log(3.0)))) / 3.0,
                               rtol=1e-12)
    assert np.all(gp <= 0)


def test_fused_beta_sigmoid_and_bf16_rounding(oracle_mod):
    """beta = sigmoid(b): logit(beta) = b without rounding; with the bf16 rounding
    beta is exactly representable in bf16 and within half a bf16 ulp of sigmoid(b)."""
    rng = np.random.default_rng(2)
    N = 64
    b = (3.0 * rng.standard_normal((N, 1))).astype(np.float32)
    b[0, 0] = 0.0
    q = np.ones((N, 1, 2), np.float32)
    zeros = np.zeros(1, np.float32)
    S = np.zeros((N, 1, 2, 2))
    _, _, beta, _ = _fused(oracle_mod, q, q, q, np.zeros((N, 1), np.float32), b, zeros, zeros, S, 1, 1)
    # beta is sigmoid rounded to fp32 (relative error <= 2^-24), which moves the
    # logit by at most 2^-24 / (1 - beta) + 2^-24 / beta ... use twice that
    bnd = 2.0 ** -23 * (1 / (1 - beta) + 1 / beta)
    assert np.all(np.abs(np.log(beta / (1 - beta)) - b.astype(np.float64)) <= bnd)
    assert beta[0, 0] == 0.5
    _, _, br, _ = _fused(oracle_mod, q, q, q, np.zeros((N, 1), np.float32), b, zeros, zeros, S, 1, 1, rnd=True)
    bits = br.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    assert np.all(np.abs(br - beta) <= beta * 2.0 ** -8 + 1e-12)   # half a bf16 ulp (8 significant bits)
    assert br[0, 0] == 0.5


def test_fused_l2_norm_scale_invariance_and_zero_keys(oracle_mod):
    """The q/k normalisation is an L2 norm: scaling q or k by c > 0 changes nothing
    (beyond the 1e-6 eps); zero keys leave only the decay (S' = alpha S) and the read."""
    rng = np.random.default_rng(3)
    N, H_q, H_v, d = 3, 2, 4, 16
    q, k, v, a, b, A_log, dt_bias, S = _fused_inputs(rng, N, H_q, H_v, d)
    o1, g1, _, S1 = _fused(oracle_mod, q, k, v, a, b, A_log, dt_bias, S, H_q, H_v)
    o2, _, _, S2 = _fused(oracle_mod, (7.0 * q).astype(np.float32), (0.25 * k).astype(np.float32), v, a, b, A_log,
                          dt_bias, S, H_q, H_v)
    assert _rel(o2, o1) < 1e-6 and _rel(S2, S1) < 1e-6
    kz = np.zeros_like(k)
    o0, g0, _, S0 = _fused(oracle_mod, q, kz, v, a, b, A_log, dt_bias, S, H_q, H_v)
    alpha = np.exp(g0)[:, :, None, None]
    assert _rel(S0, alpha * S) < 1e-14
    qn = q.astype(np.float64) / np.sqrt((q.astype(np.float64) ** 2).sum(-1, keepdims=True) + 1e-6)
    G = H_v // H_q
    ref = 0.125 * np.einsum("nhi,nhij->nhj", np.repeat(qn, G, axis=1), alpha * S)
    assert _rel(o0, ref) < 1e-12


def test_fused_matches_merged_update_formula(oracle_mod):
    """The page's merged form of the step, S' = alpha S (I - beta k k^T) + beta v k^T
    (column convention; here S' = alpha (I - beta k^T k) S + beta k^T v), with the
    norms from numpy and the gate from logaddexp, read as o = scale q_bar S'."""
    rng = np.random.default_rng(4)
    N, H_q, H_v, d = 2, 2, 4, 12
    q, k, v, a, b, A_log, dt_bias, S = _fused_inputs(rng, N, H_q, H_v, d)
    out, _, _, S1 = _fused(oracle_mod, q, k, v, a, b, A_log, dt_bias, S, H_q, H_v, scale=0.3)
    G = H_v // H_q
    for n in range(N):
        for h in range(H_v):
            kk = k[n, h // G].astype(np.float64)
            qq = q[n, h // G].astype(np.float64)
            kb = kk / np.linalg.norm(kk)
            qb = 0.3 * qq / np.linalg.norm(qq)
            alpha = np.exp(-np.exp(np.float64(A_log[h])) * np.logaddexp(0.0, np.float64(a[n, h]) + dt_bias[h]))
            beta = 1.0 / (1.0 + np.exp(-np.float64(b[n, h])))
            M = alpha * (np.eye(d) - beta * np.outer(kb, kb))
            Sn = M @ S[n, h] + beta * np.outer(kb, v[n, h].astype(np.float64))
            assert _rel(S1[n, h], Sn) < 1e-6   # eps 1e-6 inside the norm, fp32 sigmoid
            assert _rel(out[n, h], qb @ Sn) < 1e-6


def test_fused_front_end_then_plain_step(oracle_mod):
    """Feeding the normalised q, k and the returned gate and beta to the plain
    decode step reproduces the fused step (up to the fp32 rounding of q_bar, k_bar)."""
    rng = np.random.default_rng(5)
    N, H_q, H_v, d = 2, 1, 2, 32
    q, k, v, a, b, A_log, dt_bias, S = _fused_inputs(rng, N, H_q, H_v, d)
    out, g, beta, S1 = _fused(oracle_mod, q, k, v, a, b, A_log, dt_bias, S, H_q, H_v, scale=0.2)
    nrm = lambda x: x.astype(np.float64) / np.sqrt((x.astype(np.float64) ** 2).sum(-1, keepdims=True) + 1e-6)
    S2 = np.ascontiguousarray(S.copy())
    o2 = oracle_mod.decode_step(nrm(q), nrm(k), v, g, beta, S2, H_q, H_v, 0.2)
    assert _rel(o2, out) < 1e-6 and _rel(S2, S1) < 1e-6


# ---------------------------------------------------------------------------
# Prefill front end ("Qwen3.5-397B-A17B" trace page, section 1: nodes 8-10)
# ---------------------------------------------------------------------------
def _front_inputs(rng, T, H_q, H_v, d):
    q = rng.standard_normal((T, H_q, d)).astype(np.float32)
    k = rng.standard_normal((T, H_q, d)).astype(np.float32)
    v = rng.standard_normal((T, H_v, d)).astype(np.float32)
    a = rng.standard_normal((T, H_v)).astype(np.float32)
    b = rng.standard_normal((T, H_v)).astype(np.float32)
    A_log = np.log(rng.uniform(1.0, 16.0, H_v)).astype(np.float32)
    dt_bias = rng.uniform(-7.0, -2.3, H_v).astype(np.float32)
    return q, k, v, a, b, A_log, dt_bias


def test_front_end_gate_and_beta_match_c_decode_oracle(oracle_mod):
    """The numpy front end's gate and beta equal those the independent C decode
    oracle derives from the same a, b, A_log, dt_bias, over both softplus
    overflow branches and the middle, with and without the bf16 rounding of beta."""
    rng = np.random.default_rng(21)
    T, H = 40, 2
    a = np.concatenate([np.linspace(-45, 45, T // 2), 3 * rng.standard_normal(T - T // 2)]).astype(np.float32)
    a = np.stack([a, -a], axis=1)
    b = (4 * rng.standard_normal((T, H))).astype(np.float32)
    A_log = np.array([0.3, 1.7], np.float32)
    dt_bias = np.array([-4.0, 2.5], np.float32)
    q = np.ones((T, 1, 2), np.float32)
    for rnd in (False, True):
        _, g_c, beta_c, _ = _fused(oracle_mod, q, q, q, a, b, A_log, dt_bias, np.zeros((T, H, 2, 2)), 1, H, rnd=rnd)
        _, _, g, beta = oracle_mod.prefill_front_end(q, q, a, b, A_log, dt_bias, rnd)
        np.testing.assert_allclose(g, g_c, rtol=1e-15, atol=0)
        assert np.array_equal(beta, beta_c)


def test_front_end_rows_unit_norm_scale_invariant_and_rounded():
    """q_bar, k_bar rows have unit L2 norm (up to the 1e-6 inside the root), do
    not change when the raw row is scaled (norm per row and head, over d_k: a
    wrong axis breaks this), keep zero rows zero, and with the bf16 rounding are
    exactly representable and within half a bf16 ulp of the unrounded value."""
    from oracle.front_end import prefill_front_end
    rng = np.random.default_rng(22)
    T, H_q, H_v, d = 9, 2, 4, 64
    q, k, v, a, b, A_log, dt_bias = _front_inputs(rng, T, H_q, H_v, d)
    k[3, 1] = 0.0
    scale = rng.uniform(0.5, 20.0, (T, H_q, 1)).astype(np.float32)
    qn, kn, _, _ = prefill_front_end(q, k, a, b, A_log, dt_bias, False)
    qs, ks, _, _ = prefill_front_end(q * scale, k * scale, a, b, A_log, dt_bias, False)
    nr = np.linalg.norm(qn, axis=-1)
    assert np.all(np.abs(nr - 1.0) < 1e-6)
    assert _rel(qs, qn) < 1e-6 and _rel(ks, kn) < 1e-6
    assert not kn[3, 1].any()
    qr, kr, _, br = prefill_front_end(q, k, a, b, A_log, dt_bias, True)
    for x in (qr, kr, br):
        assert np.all(x.astype(np.float32).view(np.uint32) & 0xFFFF == 0)
    assert np.all(np.abs(qr - qn) <= np.abs(qn) * 2.0 ** -8 + 1e-30)


def test_forward_fused_equals_fused_decode_token_by_token(oracle_mod):
    """With fp32 inputs the prefill from raw inputs (front end, then the packed
    recurrence) equals the independent C fused decode step applied token by
    token from the same initial state (outputs and final state), for a packed
    batch of two sequences with grouped value heads."""
    rng = np.random.default_rng(23)
    H_q, H_v, d = 2, 4, 16
    lens = [7, 12]
    T = sum(lens)
    q, k, v, a, b, A_log, dt_bias = _front_inputs(rng, T, H_q, H_v, d)
    cu = np.array([0, lens[0], T], np.int64)
    s0 = (0.1 * rng.standard_normal((2, H_v, d, d))).astype(np.float64)
    out, fin = oracle_mod.forward_fused(q, k, v, a, b, A_log, dt_bias, cu, H_q, H_v, 0.25, False, initial_state=s0)
    for n in range(2):
        S = s0[n:n + 1].copy()
        for t in range(cu[n], cu[n + 1]):
            sl = slice(t, t + 1)
            o, _, _ = oracle_mod.decode_step_fused(q[sl], k[sl], v[sl], a[sl], b[sl], A_log, dt_bias, S, H_q, H_v,
                                                   0.25, False)
            assert _rel(out[t], o[0]) < 2e-6, (n, t)
        assert _rel(fin[n], S[0]) < 2e-6


# ---------------------------------------------------------------------------
# Gated RMSNorm epilogue ("Qwen3.5-397B-A17B" trace page, node 8)
# ---------------------------------------------------------------------------
def test_gated_rmsnorm_pins():
    from oracle import gated_rmsnorm

    rng = np.random.default_rng(6)
    o = rng.standard_normal((5, 3, 64))
    z = 2.0 * rng.standard_normal((5, 3, 64))
    w = rng.uniform(0.5, 1.5, 64)
    y = gated_rmsnorm(o, z, w, 0.0)
    # an RMS norm: scaling the read-out changes nothing (eps = 0)
    assert _rel(gated_rmsnorm(7.5 * o, z, w, 0.0), y) < 1e-14
    # a closed gate (z = 0) gives zero; silu(z) - silu(-z) = z
    assert np.all(gated_rmsnorm(o, np.zeros_like(z), w, 1e-6) == 0)
    diff = gated_rmsnorm(o, z, w, 0.0) - gated_rmsnorm(o, -z, w, 0.0)
    unit = gated_rmsnorm(o, np.ones_like(z), np.ones_like(w), 0.0) / (1 / (1 + np.exp(-1.0)))
    assert _rel(diff, unit * w * z) < 1e-13
    # saturated gate (silu(40) = 40 to double precision), unit weight: mean of squares
    # of y / 40 equals ms / (ms + eps) with ms the read-out's mean square
    eps = 1e-3
    y40 = gated_rmsnorm(o, np.full_like(z, 40.0), np.ones_like(w), eps) / 40.0
    ms = np.mean(o * o, axis=-1)
    assert _rel(np.mean(y40 * y40, axis=-1), ms / (ms + eps)) < 1e-12
    # linear in the weight
    assert _rel(gated_rmsnorm(o, z, 3.0 * w, 1e-6), 3.0 * gated_rmsnorm(o, z, w, 1e-6)) < 1e-14


# ---------------------------------------------------------------------------
# Causal conv1d + SiLU with its input history (trace page node 6; "Kestrel_VLLM
# - 24" page, section 三)
# ---------------------------------------------------------------------------
def _silu64(x):
    import torch

    return torch.nn.functional.silu(torch.from_numpy(np.asarray(x, dtype=np.float64))).numpy()


def test_conv_matches_numpy_convolve_and_torch_conv1d():
    import torch

    from oracle import conv_silu_varlen

    rng = np.random.default_rng(10)
    T, C, K = 37, 6, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, K))
    b = rng.standard_normal(C)
    y, fin = conv_silu_varlen(x, [0, T], w, b)
    for c in range(C):
        pre = np.convolve(x[:, c], w[c, ::-1])[:T] + b[c]   # causal: zeros before the start
        assert _rel(y[:, c], _silu64(pre)) < 1e-13
    tc = torch.nn.functional.conv1d(torch.from_numpy(x.T[None]), torch.from_numpy(w[:, None, :]),
                                    torch.from_numpy(b), padding=K - 1, groups=C)[0, :, :T].T
    assert _rel(y, _silu64(tc.numpy())) < 1e-13
    assert np.array_equal(fin[0], x[T - (K - 1):])


def test_conv_identity_kernel_is_silu_and_short_sequences():
    from oracle import conv_silu_varlen

    rng = np.random.default_rng(11)
    T, C, K = 9, 5, 4
    x = rng.standard_normal((T, C))
    w = np.zeros((C, K))
    w[:, K - 1] = 1.0
    y, _ = conv_silu_varlen(x, [0, T], w)
    assert _rel(y, _silu64(x)) < 1e-15
    # a 2-token sequence: its final history reaches into the initial one
    s0 = rng.standard_normal((1, K - 1, C))
    _, fin = conv_silu_varlen(x[:2], [0, 2], w, None, s0)
    assert np.array_equal(fin[0], np.concatenate([s0[0, 2:], x[:2]]))


def test_conv_split_and_decode_agree():
    from oracle import conv_silu_step, conv_silu_varlen

    rng = np.random.default_rng(12)
    T, C, K = 23, 7, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, K))
    b = rng.standard_normal(C)
    s0 = rng.standard_normal((1, K - 1, C))
    y, fin = conv_silu_varlen(x, [0, T], w, b, s0)
    # split at 10: pass the history
    y1, f1 = conv_silu_varlen(x[:10], [0, 10], w, b, s0)
    y2, f2 = conv_silu_varlen(x[10:], [0, T - 10], w, b, f1)
    assert _rel(np.concatenate([y1, y2]), y) < 1e-15 and np.array_equal(f2, fin)
    # packed: two sequences in one call equal two calls
    yp, fp = conv_silu_varlen(x, [0, 10, T], w, b, np.concatenate([s0, f1]))
    assert np.array_equal(yp[:10], y1) and np.array_equal(yp[10:], y2) and np.array_equal(fp[1], fin[0])
    # decode: token by token from the same history
    st = s0.copy()
    yd = np.stack([conv_silu_step(x[t:t + 1], w, b, st)[0] for t in range(T)])
    assert _rel(yd, y) < 1e-15 and np.array_equal(st, fin)
