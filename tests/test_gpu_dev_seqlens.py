"""GPU tests of the prefill with device-resident cu_seqlens (gdn_chunk_fwd_dev):
bit-identical to gdn_chunk_fwd with the same boundaries on the host (the same
kernels run on the same tables, built on the device), across ragged and empty
sequences and more than one launch group; a captured graph replayed with new
boundaries matches eager calls; and the oracle bounds the results.
"""
import numpy as np
import pytest

import gdn_inputs
from tests.gpu_helpers import f32_dev, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_state_chunk_amd as gdn

    gdn.load_library()
    return torch


def _dev_args(inp):
    return [to_dev(inp.q, inp.dtype), to_dev(inp.k, inp.dtype), to_dev(inp.v, inp.dtype), f32_dev(inp.g),
            f32_dev(inp.beta)]


@pytest.mark.parametrize("dtype,lens", [("f32", [65, 0, 130, 7, 64, 200]), ("bf16", [65, 0, 130, 7, 64, 200]),
                                        ("bf16", list(np.random.default_rng(5).integers(0, 90, 70)))])
def test_dev_seqlens_equals_host_seqlens(torch_cuda, oracle_mod, dtype, lens):
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    inp = gdn_inputs.make_prefill(81, lens, 2, 4, 128, 128, dtype)
    args = _dev_args(inp)
    s0 = f32_dev(inp.initial_state)
    cu_dev = torch.tensor(inp.cu_seqlens, dtype=torch.int32, device="cuda")
    out_h, fin_h = gdn.chunk_fwd(*args, inp.cu_seqlens, initial_state=s0)
    out_d, fin_d = gdn.chunk_fwd_dev(*args, cu_dev, initial_state=s0)
    torch.cuda.synchronize()
    assert torch.equal(out_h, out_d)
    assert torch.equal(fin_h, fin_d)
    if len(lens) <= 8:
        ref_o, ref_f = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, 2, 4,
                                          inp.scale, initial_state=inp.initial_state.astype(np.float64))
        tol = 1e-4 if dtype == "f32" else 1e-2
        assert rel_err(to_host(out_d), ref_o) < tol and rel_err(to_host(fin_d), ref_f) < tol


def test_dev_seqlens_many_items(torch_cuda, oracle_mod):
    """A batch with over eight (chunk, value head) items per chunk_prep slot of
    a 256-CU part (291 chunks x 32 value heads), where chunk_prep runs one
    workgroup an item instead of looping: device and host boundaries agree bit
    for bit, and sampled heads match the oracle (bf16 bar, 1e-2)."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    lens = [9000, 5000, 3000, 1500]
    inp = gdn_inputs.make_prefill(86, lens, 16, 32, 128, 128, "bf16")
    assert sum(-(-n // 64) for n in lens) * 32 > 8 * 4 * 256
    args = _dev_args(inp)
    s0 = f32_dev(inp.initial_state)
    cu_dev = torch.tensor(inp.cu_seqlens, dtype=torch.int32, device="cuda")
    out_h, fin_h = gdn.chunk_fwd(*args, inp.cu_seqlens, initial_state=s0)
    out_d, fin_d = gdn.chunk_fwd_dev(*args, cu_dev, initial_state=s0)
    torch.cuda.synchronize()
    assert torch.equal(out_h, out_d)
    assert torch.equal(fin_h, fin_d)
    heads = [0, 13, 31]
    ref_o, ref_f = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, 16, 32,
                                      inp.scale, initial_state=inp.initial_state.astype(np.float64), heads=heads)
    out, fin = to_host(out_d), to_host(fin_d)
    assert rel_err(out[:, heads], ref_o[:, heads]) < 1e-2
    assert rel_err(fin[:, heads], ref_f[:, heads]) < 1e-2


def test_dev_seqlens_graph_replay_with_new_boundaries(torch_cuda):
    """One captured call, replayed with three different splits of the same T
    tokens into four sequences (written into the captured cu_seqlens buffer);
    each replay equals the eager host-boundary call, bit for bit."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    T, N = 300, 4
    inp = gdn_inputs.make_prefill(82, [T], 2, 4, 128, 128, "bf16", state_std=None)
    args = _dev_args(inp)
    s0 = f32_dev(gdn_inputs.make_decode_state(83, N, 4, 128, 128))
    z, w = gdn_inputs.make_gate(84, T, 4, 128, "bf16")
    gate = (to_dev(z, "bf16"), f32_dev(w), 1e-6)
    cu_dev = torch.tensor([0, 100, 200, 250, T], dtype=torch.int32, device="cuda")
    ws = torch.empty(gdn.dev_workspace_size(T, N, 2, 4, 128, 128, torch.bfloat16), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, 4, 128), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((N, 4, 128, 128), dtype=torch.float32, device="cuda")

    def call():
        gdn.chunk_fwd_dev(*args, cu_dev, initial_state=s0, out=out, final_state=fin, workspace=ws, gate=gate)

    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for cu in ([0, 64, 65, 250, T], [0, 0, 190, 191, T], [0, 130, 260, 299, T]):
        cu_dev.copy_(torch.tensor(cu, dtype=torch.int32))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_o, ref_f = gdn.chunk_fwd(*args, np.array(cu, np.int32), initial_state=s0, gate=gate)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), cu
        assert torch.equal(fin, ref_f), cu


@pytest.mark.parametrize("with_initial", [True, False])
def test_dev_seqlens_all_sequences_empty(torch_cuda, with_initial):
    """T = 0 with three (empty) sequences: every final state is the initial
    state (zero without one), as on the host-boundary path."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    N, H_q, H_v, d = 3, 2, 4, 128
    q = torch.empty((0, H_q, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((0, H_v, d), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((0, H_v), dtype=torch.float32, device="cuda")
    s0 = f32_dev(gdn_inputs.make_decode_state(85, N, H_v, d, d)) if with_initial else None
    cu_dev = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    fin = torch.full((N, H_v, d, d), float("nan"), dtype=torch.float32, device="cuda")
    out_d, fin_d = gdn.chunk_fwd_dev(q, q, v, g, g, cu_dev, initial_state=s0, final_state=fin)
    out_h, fin_h = gdn.chunk_fwd(q, q, v, g, g, [0] * (N + 1), initial_state=s0)
    torch.cuda.synchronize()
    assert out_d.shape == (0, H_v, d)
    ref = s0 if with_initial else torch.zeros_like(fin)
    assert torch.equal(fin_d, ref)
    assert torch.equal(fin_h, ref)


def test_dev_seqlens_bins_of_short_sequences_four_tiles(torch_cuda, oracle_mod):
    """80 requests of 0..199 tokens at H_v = 32, d = 128: with device tables the
    host picks four tiles a workgroup from the mean length and the table kernel
    fills four bins of about 16 sequences per launch group in boustrophedon
    order (host tables pack them differently); the results agree bit for bit
    with the host-table call, and sampled heads match the oracle."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    lens = [int(x) for x in np.random.default_rng(707).integers(0, 200, 80)]
    inp = gdn_inputs.make_prefill(708, lens, 16, 32, 128, 128, "bf16", state_std=0.02)
    args = _dev_args(inp)
    s0 = f32_dev(inp.initial_state)
    cu_dev = torch.tensor(inp.cu_seqlens, dtype=torch.int32, device="cuda")
    print(f"[dev bins] {len(lens)} sequences, T={inp.T}", flush=True)
    out_h, fin_h = gdn.chunk_fwd(*args, inp.cu_seqlens, initial_state=s0)
    out_d, fin_d = gdn.chunk_fwd_dev(*args, cu_dev, initial_state=s0)
    torch.cuda.synchronize()
    assert torch.equal(out_h, out_d)
    assert torch.equal(fin_h, fin_d)
    heads = [0, 21, 31]
    ref_o, ref_f = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, 16, 32,
                                      inp.scale, initial_state=inp.initial_state.astype(np.float64), heads=heads)
    oh, fh = to_host(out_d), to_host(fin_d)
    for h in heads:
        assert rel_err(oh[:, h], ref_o[:, h]) < 1e-2 and rel_err(fh[:, h], ref_f[:, h]) < 1e-2, h
