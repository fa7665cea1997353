"""GPU parity of the prefill with its front end (gdn_chunk_fwd_fused): q/k L2
norm and the gate / beta transform of the raw projections done inside the
chunk kernels ("Qwen3.5-397B-A17B" trace page, section 1, Prefill-GDN nodes
8-10), against the fp64 oracle's forward_fused (oracle/front_end.py, then the
token recurrence).  Tolerances: max|err| / max|ref| <= 1e-4 (fp32), 1e-2 (bf16),
on the outputs and the final states.
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


def _dev(inp):
    dt = inp.dtype
    return [to_dev(getattr(inp, n), dt) for n in ("q", "k", "v", "a", "b")] + [f32_dev(inp.A_log),
                                                                            f32_dev(inp.dt_bias)]


def _oracle(oracle_mod, inp, initial_state):
    return oracle_mod.forward_fused(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.f32("a"), inp.f32("b"), inp.A_log,
                                    inp.dt_bias, inp.cu_seqlens, inp.H_q, inp.H_v, inp.scale, inp.dtype == "bf16",
                                    initial_state=initial_state)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_fused_prefill_matches_oracle(torch_cuda, oracle_mod, dtype, d):
    import gated_deltanet_state_chunk_amd as gdn

    inp = gdn_inputs.make_prefill_raw(31 + d, [65, 1, 130, 0, 64, 7], 2, 4, d, d, dtype)
    out, fin = gdn.chunk_fwd_fused(*_dev(inp), inp.cu_seqlens, initial_state=f32_dev(inp.initial_state))
    ref_o, ref_f = _oracle(oracle_mod, inp, inp.initial_state)
    assert rel_err(to_host(out), ref_o) < TOL[dtype]
    assert rel_err(to_host(fin), ref_f) < TOL[dtype]


def test_fused_prefill_many_sequences_wide_tiles(torch_cuda, oracle_mod):
    """48 ragged requests (some empty) at H_q = 16, H_v = 32, d = 128, bf16:
    the host packs them into bins of four 16-column tiles a workgroup, whose
    output waves read the normalised query rows through LDS (one tile a
    workgroup loads them straight into registers; both from chunk_prep's copy
    in operand order).  Sampled heads against the oracle."""
    import gated_deltanet_state_chunk_amd as gdn

    lens = [int(x) for x in np.random.default_rng(47).integers(1, 200, 48)]
    lens[5] = lens[30] = 0
    inp = gdn_inputs.make_prefill_raw(48, lens, 16, 32, 128, 128, "bf16")
    print(f"[front wide] {len(lens)} sequences, T={inp.T}", flush=True)
    out, fin = gdn.chunk_fwd_fused(*_dev(inp), inp.cu_seqlens, initial_state=f32_dev(inp.initial_state))
    heads = [0, 13, 31]
    ref_o, ref_f = oracle_mod.forward_fused(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.f32("a"), inp.f32("b"),
                                            inp.A_log, inp.dt_bias, inp.cu_seqlens, inp.H_q, inp.H_v, inp.scale, True,
                                            initial_state=inp.initial_state, heads=heads)
    oh, fh = to_host(out), to_host(fin)
    for h in heads:
        assert rel_err(oh[:, h], ref_o[:, h]) < 1e-2, h
        assert rel_err(fh[:, h], ref_f[:, h]) < 1e-2, h


def test_fused_prefill_edge_inputs(torch_cuda, oracle_mod):
    """Gate inputs across both softplus overflow branches, saturated beta, and
    all-zero q or k rows (the 1e-6 inside the norm keeps them zero)."""
    import gated_deltanet_state_chunk_amd as gdn

    inp = gdn_inputs.make_prefill_raw(41, [70, 33], 2, 4, 128, 128, "f32")
    T = inp.T
    inp.a[:, 0] = np.linspace(-45, 45, T).astype(np.float32)
    inp.a[:, 1] = np.linspace(45, -45, T).astype(np.float32)
    inp.dt_bias[:2] = 0.0
    inp.A_log[:2] = np.array([-4.0, -3.0], np.float32)   # keep alpha away from underflow at a = 45
    inp.b[::5, 2] = 30.0
    inp.b[1::5, 3] = -30.0
    inp.q[5] = 0.0
    inp.k[9] = 0.0
    inp.k[80, 1] = 0.0
    out, fin = gdn.chunk_fwd_fused(*_dev(inp), inp.cu_seqlens, initial_state=f32_dev(inp.initial_state))
    ref_o, ref_f = _oracle(oracle_mod, inp, inp.initial_state)
    assert rel_err(to_host(out), ref_o) < 1e-4
    assert rel_err(to_host(fin), ref_f) < 1e-4


def test_fused_prefill_with_gate_and_state_pool(torch_cuda, oracle_mod):
    """The serving form: raw inputs, gated read-out, states in a pool by slot
    (one fresh request, one resuming, one without a row).  Bit-identical to the
    unpooled call on the gathered states; within tolerance of the oracle."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    inp = gdn_inputs.make_prefill_raw(51, [100, 64, 9], 2, 4, 128, 128, "bf16", state_std=None)
    P = 5
    pool0 = gdn_inputs.make_decode_state(52, P, 4, 128, 128)
    slots, has = [3, 0, -1], [0, 1, 1]
    z, w = gdn_inputs.make_gate(53, inp.T, 4, 128, "bf16")
    gate = (to_dev(z, "bf16"), f32_dev(w), 1e-6)
    pool = f32_dev(pool0)
    out, none = gdn.chunk_fwd_fused(*_dev(inp), inp.cu_seqlens, initial_state=pool, slots=slots, has_initial=has,
                                    gate=gate)
    assert none is None
    init = np.zeros((3, 4, 128, 128), np.float32)
    init[1] = pool0[0]
    out2, fin2 = gdn.chunk_fwd_fused(*_dev(inp), inp.cu_seqlens, initial_state=f32_dev(init), gate=gate)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert torch.equal(pool[3], fin2[0]) and torch.equal(pool[0], fin2[1])
    for r in (1, 2, 4):
        assert torch.equal(pool[r].cpu(), torch.from_numpy(pool0[r]))
    ref_o, ref_f = _oracle(oracle_mod, inp, init)
    ref_y = oracle_mod.gated_rmsnorm(ref_o, gdn_inputs.storage_to_f32(z, "bf16"), w, 1e-6)
    assert rel_err(to_host(out), ref_y) < 1e-2
    assert rel_err(to_host(pool[3]), ref_f[0]) < 1e-2 and rel_err(to_host(pool[0]), ref_f[1]) < 1e-2


def test_fused_prefill_then_fused_decode_continues(torch_cuda, oracle_mod):
    """fp32: prefill 70 tokens from raw inputs, then three fused decode steps from
    its final state, against the oracle's prefill over all 73 tokens."""
    import gated_deltanet_state_chunk_amd as gdn

    full = gdn_inputs.make_prefill_raw(61, [73], 2, 4, 128, 128, "f32")
    pre = gdn_inputs.make_prefill_raw(61, [73], 2, 4, 128, 128, "f32")
    for n in ("q", "k", "v", "a", "b"):
        setattr(pre, n, getattr(full, n)[:70])
    pre.cu_seqlens = np.array([0, 70], np.int32)
    out, st = gdn.chunk_fwd_fused(*_dev(pre), pre.cu_seqlens, initial_state=f32_dev(full.initial_state))
    ref_o, ref_f = _oracle(oracle_mod, full, full.initial_state)
    assert rel_err(to_host(out), ref_o[:70]) < 1e-4
    for t in range(70, 73):
        sl = slice(t, t + 1)
        o = gdn.recurrent_step_fused(*[f32_dev(getattr(full, n)[sl]) for n in ("q", "k", "v", "a", "b")],
                                     f32_dev(full.A_log), f32_dev(full.dt_bias), st, scale=full.scale)
        assert rel_err(to_host(o)[0], ref_o[t]) < 1e-4, t
    assert rel_err(to_host(st), ref_f) < 1e-4
