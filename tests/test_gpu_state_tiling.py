"""GPU parity of the state scan's workgroup shapes: one, two or four 16-column
tiles of d_v per workgroup, which the launcher picks from the number of tiles
per CU (1 sequence x 32 heads x 8 tiles = one a CU on a 256-CU part; 2
sequences = two; 5 sequences = more), on bf16 d = 128 with ragged lengths,
against the fp64 oracle on every head.  The three shapes run the same MFMAs in
the same order, so the results must also agree bitwise across them (the same
head, same tokens, in batches of different sizes).
"""
import dataclasses

import numpy as np
import pytest

import gdn_inputs
from tests.gpu_helpers import chunk_fwd_device, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_state_chunk_amd as gdn

    gdn.load_library()
    return torch


@pytest.mark.parametrize("lens", [[197], [197, 130], [197, 130, 65, 1, 100]])
def test_state_scan_tiling_matches_oracle(torch_cuda, oracle_mod, lens):
    inp = gdn_inputs.make_prefill(seed=700, seqlens=lens, H_q=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
                                  state_std=0.02)
    out, fin = chunk_fwd_device(inp)
    ref_o, ref_s = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, 16, 32,
                                      inp.scale, initial_state=inp.initial_state.astype(np.float64))
    assert rel_err(out, ref_o) < 1e-2
    assert rel_err(fin, ref_s) < 1e-2


def test_state_scan_tiling_bitwise_consistent(torch_cuda):
    """The first sequence alone (one tile a CU), with one more (two), and with
    four more (four tiles a workgroup): its outputs and final state agree bit
    for bit."""
    full = gdn_inputs.make_prefill(seed=701, seqlens=[197, 130, 65, 1, 100], H_q=16, H_v=32, d_k=128, d_v=128,
                                   dtype="bf16", state_std=0.02)
    res = []
    for n in (1, 2, 5):
        t = int(full.cu_seqlens[n])
        sub = dataclasses.replace(full, q=full.q[:t], k=full.k[:t], v=full.v[:t], g=full.g[:t], beta=full.beta[:t],
                                  cu_seqlens=full.cu_seqlens[:n + 1], initial_state=full.initial_state[:n])
        out, fin = chunk_fwd_device(sub)
        res.append((out[:197], fin[0]))
    for o, f in res[1:]:
        assert np.array_equal(o, res[0][0]) and np.array_equal(f, res[0][1])


@pytest.mark.parametrize("n_seq,d", [(8, 128), (40, 128), (40, 64)])
def test_state_scan_tiling_odd_heads_many_sequences(torch_cuda, oracle_mod, n_seq, d):
    """Five value heads on five key heads (groups not a multiple of 8, so the
    per-XCD grid is padded) over many short ragged sequences: 8 sequences at
    d = 128 give 320 tiles (two a workgroup), 40 sequences four a workgroup."""
    lens = [int(x) for x in np.random.default_rng(702 + n_seq + d).integers(0, 140, n_seq)]
    inp = gdn_inputs.make_prefill(seed=703 + n_seq, seqlens=lens, H_q=5, H_v=5, d_k=d, d_v=d, dtype="bf16",
                                  state_std=0.02)
    out, fin = chunk_fwd_device(inp)
    ref_o, ref_s = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, 5, 5,
                                      inp.scale, initial_state=inp.initial_state.astype(np.float64))
    assert rel_err(out, ref_o) < 1e-2
    assert rel_err(fin, ref_s) < 1e-2
