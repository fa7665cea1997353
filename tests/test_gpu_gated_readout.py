"""GPU parity of the gated RMSNorm read-out epilogue ("Qwen3.5-397B-A17B"
trace page, Decode-GDN node 8; node 18 of the prefill graph) fused into
chunk_output_o (gdn_chunk_fwd_ex) and into the fused decode step
(gdn_recurrent_step_fused): out = o / sqrt(mean o^2 + eps) * weight * silu(z),
against the fp64 oracle's read-out passed through oracle.gated_rmsnorm.
Tolerance max|err| / max|ref|: 1e-4 (fp32), 1e-2 (bf16).
"""
import numpy as np
import pytest

import gdn_inputs
from tests.gpu_helpers import f32_dev, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 1e-2}
EPS = 1e-6


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_state_chunk_amd as gdn

    gdn.load_library()
    return torch


def _prefill(inp, z, w, eps=EPS):
    import gated_deltanet_state_chunk_amd as gdn

    dt = inp.dtype
    s0 = None if inp.initial_state is None else f32_dev(inp.initial_state)
    out, fin = gdn.chunk_fwd(to_dev(inp.q, dt), to_dev(inp.k, dt), to_dev(inp.v, dt), f32_dev(inp.g),
                             f32_dev(inp.beta), inp.cu_seqlens, initial_state=s0, scale=inp.scale,
                             gate=(to_dev(z, dt), f32_dev(w), eps))
    return to_host(out), to_host(fin)


def _ref_prefill(oracle_mod, inp, z, w, heads=None, eps=EPS):
    s0 = None if inp.initial_state is None else inp.initial_state.astype(np.float64)
    o, fin = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, inp.H_q, inp.H_v,
                                inp.scale, initial_state=s0, heads=heads)
    z32 = gdn_inputs.storage_to_f32(z, inp.dtype)
    return oracle_mod.gated_rmsnorm(o, z32, w, eps), fin


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_gated_prefill_matches_oracle(torch_cuda, oracle_mod, dtype, d):
    lens = [1, 63, 65, 130]
    inp = gdn_inputs.make_prefill(seed=91, seqlens=lens, H_q=2, H_v=4, d_k=d, d_v=d, dtype=dtype,
                                  state_std=0.02)
    z, w = gdn_inputs.make_gate(92, inp.T, inp.H_v, d, dtype)
    out, fin = _prefill(inp, z, w)
    ref, ref_fin = _ref_prefill(oracle_mod, inp, z, w)
    assert rel_err(out, ref) < TOL[dtype]
    assert rel_err(fin, ref_fin) < TOL[dtype]   # the epilogue leaves the state path alone


def test_gated_prefill_full_size_sampled_heads(torch_cuda, oracle_mod):
    """The T = 4096, 32-head bf16 workload with the read-out epilogue; heads 0, 9, 31."""
    inp = gdn_inputs.make_workload("prefill_T4096")
    z, w = gdn_inputs.make_gate(93, inp.T, inp.H_v, inp.d_v, inp.dtype)
    out, _ = _prefill(inp, z, w)
    heads = [0, 9, 31]
    ref, _ = _ref_prefill(oracle_mod, inp, z, w, heads=heads)
    e = rel_err(out[:, heads], ref[:, heads])
    print(f"gated prefill T=4096: rel err {e:.3e}", flush=True)
    assert e < 1e-2


def test_gated_prefill_zero_readout_and_closed_gate(torch_cuda):
    """A zero read-out (q = 0) and a closed gate (z = 0) both give exact zeros (eps > 0)."""
    inp = gdn_inputs.make_prefill(seed=94, seqlens=[70], H_q=1, H_v=2, d_k=64, d_v=64, dtype="f32")
    z, w = gdn_inputs.make_gate(95, inp.T, inp.H_v, 64, "f32")
    inp.q[:5] = 0.0
    z[10:12] = 0.0
    out, _ = _prefill(inp, z, w)
    assert np.all(out[:5] == 0) and np.all(out[10:12] == 0)
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_gated_fused_decode_matches_oracle(torch_cuda, oracle_mod, dtype, d):
    import gated_deltanet_state_chunk_amd as gdn

    N, H_q, H_v = 3, 2, 4
    scale = 1.0 / np.sqrt(d)
    s0 = gdn_inputs.make_decode_state(96, N, H_v, d, d)
    st = f32_dev(s0)
    ref = s0.astype(np.float64)
    for step in range(2):
        tok = gdn_inputs.make_decode_raw_token(960 + step, N, H_q, H_v, d, d, dtype)
        z, w = gdn_inputs.make_gate(970 + step, N, H_v, d, dtype)
        o = gdn.recurrent_step_fused(to_dev(tok.q, dtype), to_dev(tok.k, dtype), to_dev(tok.v, dtype),
                                     to_dev(tok.a, dtype), to_dev(tok.b, dtype), f32_dev(tok.A_log),
                                     f32_dev(tok.dt_bias), st, scale=scale, gate=(to_dev(z, dtype), f32_dev(w), EPS))
        ref_o, _, _ = oracle_mod.decode_step_fused(tok.f32("q"), tok.f32("k"), tok.f32("v"), tok.f32("a"),
                                                   tok.f32("b"), tok.A_log, tok.dt_bias, ref, H_q, H_v, scale,
                                                   dtype == "bf16")
        ref_y = oracle_mod.gated_rmsnorm(ref_o, gdn_inputs.storage_to_f32(z, dtype), w, EPS)
        assert rel_err(to_host(o), ref_y) < TOL[dtype], f"step {step}"
    assert rel_err(to_host(st), ref) < TOL[dtype]
