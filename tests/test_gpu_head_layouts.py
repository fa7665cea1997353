"""GPU parity over head layouts beyond the 2:1 grouping of the other tests:
one value head per key head, four and three value heads per key head, an odd
head count (so the per-XCD grouping of the state scan is padded), through the
chunk prefill and the decode step, against the fp64 oracle.

Tolerances as the other parity tests (max|err| / max|ref|): fp32 1e-4, bf16
1e-2.
"""
import math

import numpy as np
import pytest

import gdn_inputs
from tests.gpu_helpers import chunk_fwd_device, f32_dev, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}
LAYOUTS = [(4, 4), (1, 4), (1, 3), (3, 9), (5, 5)]  # (H_q, H_v)


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_state_chunk_amd as gdn

    gdn.load_library()
    return torch


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("H_q,H_v", LAYOUTS)
def test_chunk_head_layouts(torch_cuda, oracle_mod, dtype, d, H_q, H_v):
    inp = gdn_inputs.make_prefill(seed=300 + 10 * H_q + H_v, seqlens=[70, 130], H_q=H_q, H_v=H_v, d_k=d, d_v=d,
                                  dtype=dtype, state_std=0.05)
    out, fin = chunk_fwd_device(inp)
    ref_o, ref_s = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, H_q, H_v,
                                      inp.scale, initial_state=inp.initial_state.astype(np.float64))
    assert rel_err(out, ref_o) < TOL[dtype]
    assert rel_err(fin, ref_s) < TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("H_q,H_v", LAYOUTS)
def test_decode_head_layouts(torch_cuda, oracle_mod, dtype, d, H_q, H_v):
    import gated_deltanet_state_chunk_amd as gdn

    N = 3
    scale = 1 / math.sqrt(d)
    s0 = gdn_inputs.make_decode_state(400 + H_v, N, H_v, d, d, std=0.1)
    st = f32_dev(s0)
    ref_state = s0.astype(np.float64)
    for step in range(2):
        tok = gdn_inputs.make_decode_token(500 + 10 * H_q + H_v + step, N, H_q, H_v, d, d, dtype=dtype)
        o = gdn.recurrent_step(to_dev(tok.q, dtype), to_dev(tok.k, dtype), to_dev(tok.v, dtype), f32_dev(tok.g),
                               f32_dev(tok.beta), st, scale=scale)
        ref_o = oracle_mod.decode_step(tok.q32(), tok.k32(), tok.v32(), tok.g, tok.beta, ref_state, H_q, H_v, scale)
        torch_cuda.cuda.synchronize()
        assert rel_err(to_host(o), ref_o) < TOL[dtype], f"step {step} out"
        assert rel_err(to_host(st), ref_state) < TOL[dtype], f"step {step} state"
