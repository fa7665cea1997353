"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (one gdn_chunk_fwd / gdn_recurrent_step call per batch).

Value heads (sequence, head) are independent, so the oracle computes every
token of a sample of heads exactly; the sampled heads of the GPU result are
compared element by element.  Tolerance: max|err| / max|ref| <= 1e-2 on the
output and on the final state for the bf16 workloads, 1e-4 for the fp32 one.
"""
import numpy as np
import pytest

import gdn_inputs
from tests.gpu_helpers import chunk_fwd_device, f32_dev, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_state_chunk_amd as gdn

    gdn.load_library()
    return torch


def _check(oracle_mod, inp, out, fin, heads, tol):
    s0 = None if inp.initial_state is None else inp.initial_state.astype(np.float64)
    ref_o, ref_s = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, inp.H_q,
                                      inp.H_v, inp.scale, initial_state=s0, heads=heads)
    hs = list(range(inp.H_v)) if heads is None else list(heads)
    e_o = rel_err(out[:, hs], ref_o[:, hs])
    e_s = rel_err(fin[:, hs], ref_s[:, hs])
    print(f"heads {hs if len(hs) < 8 else 'all'}: out rel err {e_o:.3e}, final state rel err {e_s:.3e}", flush=True)
    assert e_o < tol and e_s < tol
    # per-head check as well, so one bad head cannot hide behind a large one
    for h in hs:
        assert rel_err(out[:, h], ref_o[:, h]) < tol
        assert rel_err(fin[:, h], ref_s[:, h]) < tol


def test_tiny_f32_T100(torch_cuda, oracle_mod):
    inp = gdn_inputs.make_workload("tiny_f32_T100")
    out, fin = chunk_fwd_device(inp)
    _check(oracle_mod, inp, out, fin, None, 1e-4)


def test_prefill_T4096_all_heads(torch_cuda, oracle_mod):
    inp = gdn_inputs.make_workload("prefill_T4096")
    out, fin = chunk_fwd_device(inp)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(fin))
    _check(oracle_mod, inp, out, fin, None, 1e-2)


def test_varlen_8seq_sampled_heads(torch_cuda, oracle_mod):
    inp = gdn_inputs.make_workload("varlen_8seq")
    lens = np.diff(inp.cu_seqlens)
    assert len(lens) == 8 and np.any(lens % 64 != 0)
    out, fin = chunk_fwd_device(inp)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(fin))
    _check(oracle_mod, inp, out, fin, [0, 1, 13, 30, 31], 1e-2)


def test_many_256req_sampled_heads(torch_cuda, oracle_mod):
    """The serving prefill batch of 256 requests of 1..256 tokens: four launch
    groups of 64 sequences, each group's state scan walking its sequences in
    bins (several sequences one after another per workgroup)."""
    inp = gdn_inputs.make_workload("many_256req")
    assert len(inp.cu_seqlens) == 257
    out, fin = chunk_fwd_device(inp)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(fin))
    _check(oracle_mod, inp, out, fin, [0, 14, 31], 1e-2)


def test_long_T65536_sampled_heads(torch_cuda, oracle_mod):
    inp = gdn_inputs.make_workload("long_T65536")
    out, fin = chunk_fwd_device(inp)
    assert np.all(np.isfinite(fin))
    _check(oracle_mod, inp, out, fin, [0, 17, 31], 1e-2)


def test_long_T65536_bitwise_repeatable(torch_cuda):
    """Two forwards of the 65536-token workload give bit-identical outputs and
    final states: 1024 serial chunk steps per head make any ordering race
    between the state kernel's waves show up here (the method is deterministic,
    so is every kernel: no atomics, fixed reduction orders)."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    inp = gdn_inputs.make_workload("long_T65536")
    q, k, v = (to_dev(a, inp.dtype) for a in (inp.q, inp.k, inp.v))
    g, beta = f32_dev(inp.g), f32_dev(inp.beta)
    ws = torch.empty(gdn.workspace_size(inp.T, inp.cu_seqlens, inp.H_q, inp.H_v, inp.d_k, inp.d_v, inp.dtype),
                     dtype=torch.uint8, device="cuda")
    s0 = None if inp.initial_state is None else f32_dev(inp.initial_state)
    res = [gdn.chunk_fwd(q, k, v, g, beta, inp.cu_seqlens, initial_state=s0, scale=inp.scale, workspace=ws)
           for _ in range(3)]
    torch.cuda.synchronize()
    for out, fin in res[1:]:
        assert torch.equal(out, res[0][0])
        assert torch.equal(fin, res[0][1])


def test_decode_256x16_steps(torch_cuda, oracle_mod):
    import gated_deltanet_state_chunk_amd as gdn

    cfg = gdn_inputs.DECODE_WORKLOAD
    N, H_q, H_v, d, dt = cfg["N"], cfg["H_q"], cfg["H_v"], cfg["d_k"], cfg["dtype"]
    s0 = gdn_inputs.make_decode_state(cfg["seed"], N, H_v, d, d, cfg["state_std"])
    st = f32_dev(s0)
    ref = s0.astype(np.float64)
    del s0
    scale = 1 / np.sqrt(d)
    worst = 0.0
    for s in range(cfg["steps"]):
        tok = gdn_inputs.make_decode_token(gdn_inputs.decode_step_seed(s), N, H_q, H_v, d, d, dt)
        o = gdn.recurrent_step(to_dev(tok.q, dt), to_dev(tok.k, dt), to_dev(tok.v, dt), f32_dev(tok.g),
                               f32_dev(tok.beta), st, scale=scale)
        ref_o = oracle_mod.decode_step(tok.q32(), tok.k32(), tok.v32(), tok.g, tok.beta, ref, H_q, H_v, scale)
        e = rel_err(to_host(o), ref_o)
        worst = max(worst, e)
        assert e < 1e-2, f"step {s}"
    e_s = rel_err(to_host(st), ref)
    print(f"decode: worst out rel err {worst:.3e}, state after {cfg['steps']} steps {e_s:.3e}", flush=True)
    assert e_s < 1e-2
