"""GPU parity of the causal conv1d + SiLU with its input history
(gdn_conv1d_silu_fwd / gdn_conv1d_silu_step) against the fp64 oracle
(oracle/conv.py; "Qwen3.5-397B-A17B" trace page, Decode-GDN node 6).
Outputs: max|err| / max|ref| <= 1e-5 (fp32), 1e-2 (bf16).  Histories hold raw
inputs, so they must match bit for bit.
"""
import numpy as np
import pytest

import gdn_inputs
from tests.gpu_helpers import f32_dev, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_state_chunk_amd as gdn

    gdn.load_library()
    return torch


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("with_state", [True, False])
def test_conv_prefill_matches_oracle(torch_cuda, oracle_mod, dtype, K, with_state):
    import gated_deltanet_state_chunk_amd as gdn

    lens = [1, 2, 63, 64, 65, 0, 150]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, C, N = int(cu[-1]), 72, len(lens)
    x, s0, w, b = gdn_inputs.make_conv(40 + K, T, C, K, N, dtype, with_state)
    out, fin = gdn.conv1d_silu(to_dev(x, dtype), cu, f32_dev(w), f32_dev(b),
                               initial_state=None if s0 is None else to_dev(s0, dtype))
    x32 = gdn_inputs.storage_to_f32(x, dtype)
    s32 = None if s0 is None else gdn_inputs.storage_to_f32(s0, dtype)
    ref, ref_fin = oracle_mod.conv_silu_varlen(x32, cu, w, b, s32)
    assert rel_err(to_host(out), ref) < TOL[dtype]
    assert np.array_equal(to_host(fin), ref_fin)


def test_conv_in_place_history_and_no_bias(torch_cuda, oracle_mod):
    """final_state may be initial_state; bias NULL means zero."""
    import gated_deltanet_state_chunk_amd as gdn

    cu = np.array([0, 5, 200], np.int32)
    x, s0, w, _ = gdn_inputs.make_conv(50, 200, 128, 4, 2, "bf16")
    st = to_dev(s0, "bf16")
    out, fin = gdn.conv1d_silu(to_dev(x, "bf16"), cu, f32_dev(w), None, initial_state=st, final_state=st)
    ref, ref_fin = oracle_mod.conv_silu_varlen(gdn_inputs.storage_to_f32(x, "bf16"), cu, w, None,
                                               gdn_inputs.storage_to_f32(s0, "bf16"))
    assert rel_err(to_host(out), ref) < 1e-2
    assert np.array_equal(to_host(st), ref_fin)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_decode_steps_match_prefill(torch_cuda, oracle_mod, dtype):
    """Token-by-token decode steps from a history equal the oracle's packed prefill."""
    import gated_deltanet_state_chunk_amd as gdn

    N, C, K, steps = 5, 96, 4, 6
    x, s0, w, b = gdn_inputs.make_conv(60, N * steps, C, K, N, dtype)
    xs = x.reshape(steps, N, C)
    st = to_dev(s0, dtype)
    ref_state = gdn_inputs.storage_to_f32(s0, dtype).astype(np.float64)
    for t in range(steps):
        o = gdn.conv1d_silu_step(to_dev(np.ascontiguousarray(xs[t]), dtype), f32_dev(w), f32_dev(b), st)
        ref = oracle_mod.conv_silu_step(gdn_inputs.storage_to_f32(xs[t], dtype), w, b, ref_state)
        assert rel_err(to_host(o), ref) < TOL[dtype]
    assert np.array_equal(to_host(st), ref_state)


def test_conv_full_size(torch_cuda, oracle_mod):
    """T = 4096 tokens, C = 8192 channels (q, k, v of 16 + 16 + 32 heads at d = 128), K = 4, bf16."""
    import gated_deltanet_state_chunk_amd as gdn

    T, C, K = 4096, 8192, 4
    cu = np.array([0, T], np.int32)
    x, s0, w, b = gdn_inputs.make_conv(70, T, C, K, 1, "bf16")
    out, fin = gdn.conv1d_silu(to_dev(x, "bf16"), cu, f32_dev(w), f32_dev(b), initial_state=to_dev(s0, "bf16"))
    cols = np.arange(0, C, 37)
    ref, ref_fin = oracle_mod.conv_silu_varlen(gdn_inputs.storage_to_f32(x, "bf16")[:, cols], cu, w[cols], b[cols],
                                               gdn_inputs.storage_to_f32(s0, "bf16")[:, :, cols])
    assert rel_err(to_host(out)[:, cols], ref) < 1e-2
    assert np.array_equal(to_host(fin)[:, :, cols], ref_fin)
