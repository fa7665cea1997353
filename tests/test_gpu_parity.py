"""GPU parity: libgdn.so (through its C ABI) against the fp64 oracle.

Tolerances (max|err| / max|ref| per tensor): fp32 inputs 1e-4; bf16 q/k/v with
fp32 accumulation 1e-2 on the output and the final state.  Sizes span several
chunks and ragged tails; the full workloads are covered in
test_gpu_workloads.py.
"""
import math

import numpy as np
import pytest

import gdn_inputs
from tests.gpu_helpers import (a_frags_to_logical, chunk_fwd_device, f32_dev, frag_rows_to_logical, frag_u_to_logical, frag_w_to_logical,
                               rel_err, to_dev, to_host, unperm32)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_state_chunk_amd as gdn

    gdn.load_library()
    return torch


def _oracle_prefill(oracle_mod, inp, heads=None):
    s0 = None if inp.initial_state is None else inp.initial_state.astype(np.float64)
    return oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, inp.H_q, inp.H_v,
                              inp.scale, initial_state=s0, heads=heads)


# ---------------------------------------------------------------------------
# Decode step
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_recurrent_step_matches_oracle(torch_cuda, oracle_mod, dtype, d):
    import gated_deltanet_state_chunk_amd as gdn

    N, H_q, H_v = 5, 2, 4
    scale = 1 / math.sqrt(d)
    s0 = gdn_inputs.make_decode_state(77, N, H_v, d, d, std=0.1)
    st = f32_dev(s0)
    ref_state = s0.astype(np.float64)
    for step in range(3):
        tok = gdn_inputs.make_decode_token(900 + step, N, H_q, H_v, d, d, dtype=dtype)
        o = gdn.recurrent_step(to_dev(tok.q, dtype), to_dev(tok.k, dtype), to_dev(tok.v, dtype), f32_dev(tok.g),
                               f32_dev(tok.beta), st, scale=scale)
        ref_o = oracle_mod.decode_step(tok.q32(), tok.k32(), tok.v32(), tok.g, tok.beta, ref_state, H_q, H_v, scale)
        torch_cuda.cuda.synchronize()
        tol = TOL[dtype]
        assert rel_err(to_host(o), ref_o) < tol, f"step {step} out"
        assert rel_err(to_host(st), ref_state) < tol, f"step {step} state"


# ---------------------------------------------------------------------------
# Chunk prefill, small cases
# ---------------------------------------------------------------------------
def test_chunk_tiny_f32_workload(torch_cuda, oracle_mod):
    """The small fp32 workload: T=100 (64-chunk + 36-token tail), H=2, d=64, zero S0."""
    inp = gdn_inputs.make_workload("tiny_f32_T100")
    out, fin = chunk_fwd_device(inp)
    ref_o, ref_s = _oracle_prefill(oracle_mod, inp)
    assert rel_err(out, ref_o) < 1e-4
    assert rel_err(fin, ref_s) < 1e-4


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("lens", [[1], [63], [64], [65], [200], [130, 0, 5, 64, 71]])
def test_chunk_matches_oracle(torch_cuda, oracle_mod, dtype, d, lens):
    inp = gdn_inputs.make_prefill(seed=31 + len(lens) + sum(lens), seqlens=lens, H_q=2, H_v=4, d_k=d, d_v=d,
                                  dtype=dtype, state_std=0.05)
    out, fin = chunk_fwd_device(inp)
    ref_o, ref_s = _oracle_prefill(oracle_mod, inp)
    assert rel_err(out, ref_o) < TOL[dtype]
    assert rel_err(fin, ref_s) < TOL[dtype]


def test_chunk_zero_initial_state_and_no_final(torch_cuda, oracle_mod):
    import gated_deltanet_state_chunk_amd as gdn

    inp = gdn_inputs.make_prefill(seed=5, seqlens=[100], H_q=1, H_v=2, d_k=128, d_v=128, dtype="bf16",
                                  state_std=None)
    out, fin = chunk_fwd_device(inp)
    ref_o, ref_s = _oracle_prefill(oracle_mod, inp)
    assert rel_err(out, ref_o) < 1e-2 and rel_err(fin, ref_s) < 1e-2
    o2, f2 = gdn.chunk_fwd(to_dev(inp.q, "bf16"), to_dev(inp.k, "bf16"), to_dev(inp.v, "bf16"), f32_dev(inp.g),
                           f32_dev(inp.beta), inp.cu_seqlens, output_final_state=False)
    assert f2 is None
    assert np.array_equal(to_host(o2), out)


def test_chunk_in_place_state_and_determinism(torch_cuda, oracle_mod):
    """final_state may alias initial_state; two runs are bitwise identical."""
    import gated_deltanet_state_chunk_amd as gdn

    inp = gdn_inputs.make_prefill(seed=6, seqlens=[150, 70], H_q=2, H_v=4, d_k=128, d_v=128, dtype="bf16")
    out1, fin1 = chunk_fwd_device(inp)
    out2, fin2 = chunk_fwd_device(inp)
    assert np.array_equal(out1, out2) and np.array_equal(fin1, fin2)
    st = f32_dev(inp.initial_state)
    o3, f3 = gdn.chunk_fwd(to_dev(inp.q, "bf16"), to_dev(inp.k, "bf16"), to_dev(inp.v, "bf16"), f32_dev(inp.g),
                           f32_dev(inp.beta), inp.cu_seqlens, initial_state=st, final_state=st)
    torch_cuda.cuda.synchronize()
    assert f3.data_ptr() == st.data_ptr()
    assert np.array_equal(to_host(st), fin1) and np.array_equal(to_host(o3), out1)


def test_chunk_many_sequences_multiple_launch_groups(torch_cuda, oracle_mod):
    """More sequences than one launch's table holds (the host splits the batch)."""
    rng = np.random.default_rng(40)
    lens = [int(x) for x in rng.integers(0, 90, size=150)]
    inp = gdn_inputs.make_prefill(seed=41, seqlens=lens, H_q=1, H_v=2, d_k=64, d_v=64, dtype="bf16")
    out, fin = chunk_fwd_device(inp)
    ref_o, ref_s = _oracle_prefill(oracle_mod, inp)
    assert rel_err(out, ref_o) < 1e-2 and rel_err(fin, ref_s) < 1e-2


def test_prefill_then_decode_continues(torch_cuda, oracle_mod):
    """prefill(T) + decode(token T+1) == prefill(T+1) on the last output and the state."""
    import gated_deltanet_state_chunk_amd as gdn

    inp = gdn_inputs.make_prefill(seed=8, seqlens=[97], H_q=2, H_v=4, d_k=128, d_v=128, dtype="f32")
    T = inp.T
    q, k, v = to_dev(inp.q, "f32"), to_dev(inp.k, "f32"), to_dev(inp.v, "f32")
    g, beta = f32_dev(inp.g), f32_dev(inp.beta)
    s0 = f32_dev(inp.initial_state)
    out_all, fin_all = gdn.chunk_fwd(q, k, v, g, beta, [0, T], initial_state=s0)
    _, fin_pre = gdn.chunk_fwd(q[:T - 1].contiguous(), k[:T - 1].contiguous(), v[:T - 1].contiguous(),
                               g[:T - 1].contiguous(), beta[:T - 1].contiguous(), [0, T - 1], initial_state=s0)
    o_dec = gdn.recurrent_step(q[T - 1:], k[T - 1:], v[T - 1:], g[T - 1:], beta[T - 1:], fin_pre)
    torch_cuda.cuda.synchronize()
    assert rel_err(to_host(o_dec), to_host(out_all[T - 1:])) < 1e-5
    assert rel_err(to_host(fin_pre), to_host(fin_all)) < 1e-5


def test_inspection_regions_untouched_without_flags(torch_cuda):
    """The A region is written only under GDN_FWD_KEEP_A; W and U only where the
    scan reads them (the W form) or under GDN_FWD_KEEP_WU; A's fragments only in
    the A form.  The flags never change the outputs."""
    import torch

    import gated_deltanet_state_chunk_amd as gdn

    inp = gdn_inputs.make_prefill(seed=12, seqlens=[70, 64], H_q=1, H_v=2, d_k=64, d_v=64, dtype="bf16")
    lay = gdn.workspace_layout(inp.T, inp.cu_seqlens, 1, 2, 64, 64, "bf16")
    a0, a1 = lay["off_A"], lay["off_W"]
    f0, f1 = lay["off_Af"], lay["total_bytes"]
    w0, w1 = lay["off_W"], lay["off_Kc"]
    assert a1 > a0 and f1 > f0 and w1 > w0
    args = [to_dev(inp.q, "bf16"), to_dev(inp.k, "bf16"), to_dev(inp.v, "bf16"), f32_dev(inp.g), f32_dev(inp.beta),
            inp.cu_seqlens]

    def run(**kw):
        ws = torch.full((lay["total_bytes"],), 0xA5, dtype=torch.uint8, device="cuda")
        out, fin = gdn.chunk_fwd(*args, scale=inp.scale, workspace=ws, **kw)
        torch.cuda.synchronize()
        untouched = [bool((ws[lo:hi] == 0xA5).all()) for lo, hi in ((a0, a1), (f0, f1), (w0, w1))]
        return out, fin, untouched

    ow, fw, u = run(form="W")
    assert u == [True, True, False]        # W and U are the scan's operands
    ow2, fw2, u = run(form="W", keep_A=True)
    assert u == [False, True, False]
    oa, fa, u = run(form="A")
    assert u == [True, False, True]        # A's fragments are the scan's operands
    oa2, fa2, u = run(form="A", keep_A=True, keep_wu=True)
    assert u == [False, False, False]
    assert torch.equal(ow, ow2) and torch.equal(fw, fw2)
    assert torch.equal(oa, oa2) and torch.equal(fa, fa2)
    assert rel_err(to_host(oa), to_host(ow)) < 1e-2 and rel_err(to_host(fa), to_host(fw)) < 1e-2


def test_query_copy_in_operand_order(torch_cuda):
    """With one 16-column tile a state-scan workgroup, chunk_prep keeps each
    chunk's query rows (Qc) as the output waves' operand fragments: fragment
    (w, s) of a chunk and key head holds, in lane 16 a + r, slot 4 h + b,
    q[16 w + r][32 s + 16 h + 4 a + b], zero past the valid length.  With four
    tiles (and no front end) the scan reads q itself and Qc is left alone."""
    import torch

    import gated_deltanet_state_chunk_amd as gdn

    H_q, H_v, d = 2, 4, 128
    inp = gdn_inputs.make_prefill(seed=13, seqlens=[100, 37], H_q=H_q, H_v=H_v, d_k=d, d_v=d, dtype="bf16")
    lay = gdn.workspace_layout(inp.T, inp.cu_seqlens, H_q, H_v, d, d, "bf16")
    q0 = lay["off_Qc"]
    args = [to_dev(inp.q, "bf16"), to_dev(inp.k, "bf16"), to_dev(inp.v, "bf16"), f32_dev(inp.g), f32_dev(inp.beta),
            inp.cu_seqlens]
    # expected copy: [chunk][key head][w][s][lane][slot]
    starts = [(0, 64), (64, 36), (100, 37)]  # (first token, valid length) of each chunk
    exp = np.zeros((len(starts), H_q, 4, d // 32, 64, 8), dtype=np.float64)
    qf = inp.q32()
    for c, (t0, ell) in enumerate(starts):
        for hq in range(H_q):
            for w in range(4):
                for s in range(d // 32):
                    for lane in range(64):
                        a, r = lane // 16, lane % 16
                        if 16 * w + r < ell:
                            for hh in range(2):
                                exp[c, hq, w, s, lane, 4 * hh:4 * hh + 4] = \
                                    qf[t0 + 16 * w + r, hq, 32 * s + 16 * hh + 4 * a:32 * s + 16 * hh + 4 * a + 4]
    q1 = q0 + 2 * exp.size
    assert q1 <= lay["off_Af"]
    for form in ("W", "A"):
        ws = torch.full((lay["total_bytes"],), 0xA5, dtype=torch.uint8, device="cuda")
        gdn.chunk_fwd(*args, scale=inp.scale, workspace=ws, scan_ct=1, form=form)
        torch.cuda.synchronize()
        got = to_host(ws[q0:q1].view(torch.bfloat16)).reshape(exp.shape)
        assert np.array_equal(got, exp), form
        ws.fill_(0xA5)
        gdn.chunk_fwd(*args, scale=inp.scale, workspace=ws, scan_ct=4, form=form)
        torch.cuda.synchronize()
        assert bool((ws[q0:q1] == 0xA5).all()), form


# ---------------------------------------------------------------------------
# Per-stage intermediates against the chunk-form oracle
# ---------------------------------------------------------------------------
def _x_bound_w(r, inp, n, h, c, d, dtype, tol_h):
    """Worst-case error of the stored X = U - W S of one chunk, relative to max|X|,
    along the W form's path: the A and B V (B Gamma K) operands of U (W),
    U and W themselves, the S operand, X itself (unit u each: 2^-9 for bf16,
    2^-24 for fp32), fp32 accumulation over the 64 positions or d_k rows
    (2^-24 per term), and the chunk-start state's own error, taken at the
    tolerance h is held to (tol_h max|h|).  Each product term is bounded by the
    sums of |a| |b| (no cancellation assumed), so this is a bound, not an
    estimate; it depends on the inputs, not on the device result."""
    u = 2.0 ** -9 if dtype == "bf16" else 2.0 ** -24
    ua = 2.0 ** -24
    ell = r["U"].shape[0]
    t0 = int(inp.cu_seqlens[n]) + 64 * c
    hq = h // (inp.H_v // inp.H_q)
    V = inp.v32()[t0:t0 + ell, h].astype(np.float64)
    K = inp.k32()[t0:t0 + ell, hq].astype(np.float64)
    b = inp.beta[t0:t0 + ell, h].astype(np.float64)
    A, S, W, U, X = (np.abs(r[key]) for key in ("A", "h", "W", "U", "X"))
    BV, BGK = np.abs(b[:, None] * V), np.abs((b * np.exp(r["gc"]))[:, None] * K)
    dU = (2 * u + 64 * ua) * (A @ BV) + u * U
    dW = (2 * u + 64 * ua) * (A @ BGK) + u * W
    dX = dU + dW @ S + (u + d * ua) * (W @ S) + W.sum(1, keepdims=True) * tol_h * S.max() + u * X
    return float(dX.max() / X.max())


def _x_bound_a(r, inp, n, h, c, d, dtype, tol_h):
    """Worst-case error of the stored X = U - W S of one chunk, relative to max|X|,
    from the roundings along the A form's path, X = A (B (V - Gamma K S)):
    the chunk-start state S as an MFMA operand (unit u: 2^-9 for bf16, 2^-24
    for fp32) and its own error, taken at the tolerance h is held to (tol_h
    max|h|); fp32 accumulation over d_k rows and 64 positions (2^-24 per term);
    B Y and A rounded to the product type (binary16 for bf16 inputs: 2^-11;
    fp32 otherwise); X itself rounded to the input type.  K and V enter exactly
    (they are the inputs).  Each product term is bounded by the sums of |a| |b|
    (no cancellation assumed), so this is a bound, not an estimate; it depends
    on the inputs and the fp64 chunk form, not on the device result."""
    u = 2.0 ** -9 if dtype == "bf16" else 2.0 ** -24
    up = 2.0 ** -11 if dtype == "bf16" else 2.0 ** -24
    ua = 2.0 ** -24
    ell = r["X"].shape[0]
    t0 = int(inp.cu_seqlens[n]) + 64 * c
    hq = h // (inp.H_v // inp.H_q)
    V = inp.v32()[t0:t0 + ell, h].astype(np.float64)
    K = inp.k32()[t0:t0 + ell, hq].astype(np.float64)
    b = inp.beta[t0:t0 + ell, h].astype(np.float64)
    gam = np.exp(r["gc"])
    A, S, X = np.abs(r["A"]), r["h"], np.abs(r["X"])
    BY = np.abs(b[:, None] * (V - gam[:, None] * (K @ S)))
    dS = (u + d * ua) * np.abs(S) + tol_h * np.abs(S).max()
    dBY = b[:, None] * gam[:, None] * (np.abs(K) @ dS) + up * BY
    dX = A @ dBY + (up + 64 * ua) * (A @ BY) + u * X
    return float(dX.max() / X.max())


@pytest.mark.parametrize("dtype,d,tol,form", [("f32", 64, 1e-4, "W"), ("bf16", 128, 1e-2, "W"),
                                              ("bf16", 128, 1e-2, "A")])
def test_chunk_intermediates_match_chunk_form(torch_cuda, dtype, d, tol, form):
    """Every workspace intermediate against the fp64 chunk form, in both forms
    of the state scan's operands (W and U; A and the raw rows, with W and U
    written for inspection)."""
    import gated_deltanet_state_chunk_amd as gdn
    from oracle import chunk_form

    lens = [100, 64, 30]
    H_q, H_v = 1, 2
    inp = gdn_inputs.make_prefill(seed=9, seqlens=lens, H_q=H_q, H_v=H_v, d_k=d, d_v=d, dtype=dtype)
    _, _, ws = chunk_fwd_device(inp, return_ws=True, keep_A=True, keep_hx=True, keep_wu=True,
                                form=None if dtype == "f32" else form)
    lay = gdn.workspace_layout(inp.T, inp.cu_seqlens, H_q, H_v, d, d, dtype)
    nc = lay["n_chunks"]
    assert nc == 2 + 1 + 1

    def region(off, shape, is_f32=False, half=False):
        import torch

        nbytes = int(np.prod(shape)) * (4 if (is_f32 or dtype == "f32") else 2)
        raw = ws[off:off + nbytes]
        if is_f32 or dtype == "f32":
            t = raw.view(torch.float32)
        else:  # bf16 inputs: U is stored as fp16, the rest of the 2-byte regions as bf16
            t = raw.view(torch.float16) if half else raw.view(torch.bfloat16)
        return t.float().cpu().numpy().astype(np.float64).reshape(shape)

    gates = region(lay["off_gates"], (nc, H_v, 4, 64), is_f32=True)
    gc, kf, gb, gbg = gates[:, :, 0], gates[:, :, 1], gates[:, :, 2], gates[:, :, 3]
    A = region(lay["off_A"], (nc, H_v, 64, 64))
    W = frag_w_to_logical(region(lay["off_W"], (nc, H_v, 64 * d)), d)
    U = frag_u_to_logical(region(lay["off_U"], (nc, H_v, 64 * d), half=True), d)
    Af = a_frags_to_logical(region(lay["off_Af"], (nc, H_v, 6 * 64 * 8), half=True))
    # Kc: each row's 16-byte pieces stored permuted (piece i at i ^ p(r), as include/gdn.h states)
    es = 4 if dtype == "f32" else 2
    P = d * es // 16
    Kc_st = region(lay["off_Kc"], (nc, H_q, 64, P, 16 // es))
    Kc = np.empty_like(Kc_st)
    for r in range(64):
        pr = 2 * (r % (P // 2)) if es == 2 else 4 * ((r // 4) % (P // 4))
        Kc[:, :, r, np.arange(P) ^ pr] = Kc_st[:, :, r]
    Kc = Kc.reshape(nc, H_q, 64, d)
    k_in = inp.k32()
    Hs = np.swapaxes(frag_rows_to_logical(region(lay["off_Ht"], (nc, H_v, d * d)), d, d), -1, -2)
    X = np.swapaxes(unperm32(frag_rows_to_logical(region(lay["off_Xt"], (nc, H_v, d * 64)), d, 64)), -1, -2)

    ref = chunk_form.chunk_forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, H_q, H_v,
                                   inp.scale, initial_state=inp.initial_state, keep_intermediates=True)
    ci = 0
    for n, L in enumerate(lens):
        for c in range((L + 63) // 64):
            ell = min(64, L - 64 * c)
            t0 = int(inp.cu_seqlens[n]) + 64 * c
            for hq in range(H_q):  # the chunk's key rows, exactly, and zeros past the valid length
                assert np.array_equal(Kc[ci, hq, :ell], k_in[t0:t0 + ell, hq].astype(np.float64))
                assert np.all(Kc[ci, hq, ell:] == 0)
            for h in range(H_v):
                r = ref["chunks"][(n, h)][c]
                assert rel_err(gc[ci, h, :ell], r["gc"]) < 1e-5
                assert np.all(gc[ci, h, ell:] == 0)
                assert rel_err(A[ci, h, :ell, :ell], r["A"]) < tol
                assert np.all(A[ci, h, ell:, :] == 0) and np.all(A[ci, h, :, ell:] == 0)
                if form == "A":  # the state scan's fragments of A: the same lower triangle
                    # (in the product type), unit rows past the valid length, zeros above
                    assert rel_err(Af[ci, h, :ell, :ell], r["A"]) < tol
                    assert np.array_equal(Af[ci, h, ell:, :], np.eye(64)[ell:])
                    assert np.all(np.triu(Af[ci, h], 1) == 0)
                # gate block: beta as given (zero past the valid length), beta gamma
                b_in = inp.beta[t0:t0 + ell, h].astype(np.float64)
                assert np.array_equal(gb[ci, h, :ell], b_in) and np.all(gb[ci, h, ell:] == 0)
                assert rel_err(gbg[ci, h, :ell], b_in * np.exp(r["gc"])) < 1e-5
                assert np.all(gbg[ci, h, ell:] == 0)
                assert rel_err(W[ci, h, :ell], r["W"]) < tol
                assert rel_err(U[ci, h, :ell], r["U"]) < tol
                assert rel_err(Hs[ci, h], r["h"]) < tol
                xb = (_x_bound_w if form == "W" else _x_bound_a)(r, inp, n, h, c, d, dtype, tol)
                x_tol = max(tol, xb) if dtype == "f32" else xb
                assert rel_err(X[ci, h, :ell], r["X"]) < x_tol, (n, h, c, x_tol)
                assert np.all(W[ci, h, ell:] == 0) and np.all(X[ci, h, ell:] == 0)
                # keys of the state update carry the decay to the chunk end: gamma_l / gamma_r
                assert rel_err(kf[ci, h, :ell], np.exp(r["gc"][-1] - r["gc"])) < 1e-5
                assert np.all(kf[ci, h, ell:] == 0)
            ci += 1


# ---------------------------------------------------------------------------
# Pages' invariants on the device path
# ---------------------------------------------------------------------------
def test_beta_zero_pure_decay_on_gpu(torch_cuda):
    inp = gdn_inputs.make_prefill(seed=11, seqlens=[150], H_q=2, H_v=2, d_k=64, d_v=64, dtype="f32",
                                  beta_override=0.0, state_std=0.5)
    out, fin = chunk_fwd_device(inp)
    gam = np.exp(np.cumsum(inp.g.astype(np.float64), axis=0))
    for h in range(2):
        assert rel_err(fin[0, h], gam[-1, h] * inp.initial_state[0, h]) < 1e-5
        exp_o = inp.scale * gam[:, h, None] * (inp.q32()[:, h, :].astype(np.float64) @ inp.initial_state[0, h])
        assert rel_err(out[:, h, :], exp_o) < 1e-5


def test_strong_decay_stays_finite(torch_cuda, oracle_mod):
    """g down to -10 per token: Gamma^-1 alone would overflow fp32 within a chunk."""
    inp = gdn_inputs.make_prefill(seed=12, seqlens=[130], H_q=1, H_v=2, d_k=64, d_v=64, dtype="f32")
    inp.g[:] = np.float32(-10.0) * np.random.default_rng(3).uniform(0, 1, inp.g.shape).astype(np.float32)
    out, fin = chunk_fwd_device(inp)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(fin))
    ref_o, ref_s = _oracle_prefill(oracle_mod, inp)
    assert rel_err(out, ref_o) < 1e-4 and rel_err(fin, ref_s) < 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_value_columns_are_independent(torch_cuda, dtype):
    """Permuting the d_v columns of v and of the initial state permutes the
    columns of the output and of the final state, bit for bit: every d_v column
    is computed the same way whichever 16-column tile it falls in."""
    inp = gdn_inputs.make_prefill(seed=13, seqlens=[130, 70], H_q=2, H_v=4, d_k=128, d_v=128, dtype=dtype)
    out, fin = chunk_fwd_device(inp)
    perm = np.random.default_rng(14).permutation(128)
    inp.v = np.ascontiguousarray(inp.v[..., perm])
    inp.initial_state = np.ascontiguousarray(inp.initial_state[..., perm])
    out_p, fin_p = chunk_fwd_device(inp)
    assert np.array_equal(out_p, out[..., perm])
    assert np.array_equal(fin_p, fin[..., perm])
