"""GPU parity of the fused decode step (gdn_recurrent_step_fused) against the
fp64 oracle's decode_step_fused: q/k L2 norm, gate from a / A_log / dt_bias,
beta from b ("Qwen3.5-397B-A17B" trace page, Decode-GDN node 7), then the
state update.  Tolerance: max|err| / max|ref| <= 1e-4 (fp32), 1e-2 (bf16), on
the outputs of every step and on the state after the last one.
"""
import numpy as np
import pytest

import gdn_inputs
from tests.gpu_helpers import f32_dev, rel_err, to_dev, to_host

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


def _step(tok, st_dev, scale):
    import gated_deltanet_state_chunk_amd as gdn

    dt = tok.dtype
    return gdn.recurrent_step_fused(to_dev(tok.q, dt), to_dev(tok.k, dt), to_dev(tok.v, dt), to_dev(tok.a, dt),
                                    to_dev(tok.b, dt), f32_dev(tok.A_log), f32_dev(tok.dt_bias), st_dev, scale=scale)


def _ref(oracle_mod, tok, state, H_q, H_v, scale, heads=None):
    out, g, beta = oracle_mod.decode_step_fused(tok.f32("q"), tok.f32("k"), tok.f32("v"), tok.f32("a"), tok.f32("b"),
                                                tok.A_log, tok.dt_bias, state, H_q, H_v, scale,
                                                tok.dtype == "bf16", heads=heads)
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_fused_decode_matches_oracle(torch_cuda, oracle_mod, dtype, d):
    N, H_q, H_v = 3, 2, 4
    scale = 1.0 / np.sqrt(d)
    s0 = gdn_inputs.make_decode_state(71, N, H_v, d, d)
    st = f32_dev(s0)
    ref = s0.astype(np.float64)
    for step in range(2):
        tok = gdn_inputs.make_decode_raw_token(700 + step, N, H_q, H_v, d, d, dtype)
        o = _step(tok, st, scale)
        ref_o = _ref(oracle_mod, tok, ref, H_q, H_v, scale)
        assert rel_err(to_host(o), ref_o) < TOL[dtype], f"step {step}"
    assert rel_err(to_host(st), ref) < TOL[dtype]


def test_fused_decode_edge_inputs(torch_cuda, oracle_mod):
    """Both softplus overflow branches (|a + dt_bias| > 20), saturated beta
    (b = +-30), and all-zero q or k vectors (the 1e-6 inside the norm keeps them 0)."""
    N, H_q, H_v, d = 8, 1, 2, 64
    tok = gdn_inputs.make_decode_raw_token(81, N, H_q, H_v, d, d, "f32")
    tok.a[:, 0] = np.array([-40, -25, -20.5, -3, 0, 20.5, 25, 40], np.float32)
    tok.a[:, 1] = np.array([40, 25, 20.5, 3, 0, -20.5, -25, -40], np.float32)
    tok.dt_bias[:] = 0.0
    tok.A_log[:] = np.array([-3.0, 0.5], np.float32)   # keep alpha away from underflow at a = 40
    tok.b[:, 0] = np.array([-30, -10, 0, 10, 30, 1, -1, 2], np.float32)
    tok.q[1] = 0.0
    tok.k[2] = 0.0
    s0 = gdn_inputs.make_decode_state(82, N, H_v, d, d)
    st = f32_dev(s0)
    ref = s0.astype(np.float64)
    o = _step(tok, st, 0.125)
    ref_o = _ref(oracle_mod, tok, ref, H_q, H_v, 0.125)
    assert rel_err(to_host(o), ref_o) < 1e-4
    assert rel_err(to_host(st), ref) < 1e-4
    assert np.all(to_host(o)[1] == 0)        # zero query reads nothing


def test_fused_decode_full_size_sampled_heads(torch_cuda, oracle_mod):
    """256 sequences x 32 value heads, d = 128, bf16, three steps; heads 0, 13, 31 checked."""
    cfg = gdn_inputs.DECODE_WORKLOAD
    N, H_q, H_v, d = cfg["N"], cfg["H_q"], cfg["H_v"], cfg["d_k"]
    heads = [0, 13, 31]
    scale = 1.0 / np.sqrt(d)
    s0 = gdn_inputs.make_decode_state(cfg["seed"], N, H_v, d, d, cfg["state_std"])
    st = f32_dev(s0)
    ref = np.zeros((N, H_v, d, d))
    ref[:, heads] = s0[:, heads]
    del s0
    for step in range(3):
        tok = gdn_inputs.make_decode_raw_token(900 + step, N, H_q, H_v, d, d, "bf16")
        o = _step(tok, st, scale)
        ref_o = _ref(oracle_mod, tok, ref, H_q, H_v, scale, heads=heads)
        e = rel_err(to_host(o)[:, heads], ref_o[:, heads])
        assert e < 1e-2, f"step {step}: {e}"
    e_s = rel_err(to_host(st[:, heads]), ref[:, heads])
    print(f"fused decode: state rel err after 3 steps {e_s:.3e}", flush=True)
    assert e_s < 1e-2
