"""GPU parity of the state scan's work split: one, two or four 16-column tiles
of d_v per workgroup, and bins of sequences that one workgroup scans one after
another.  The host picks both from the chunk counts (on a 256-CU part: one
sequence of 4 chunks x 32 heads -> one tile a workgroup; 4 + 3 chunks -> two
tiles, one sequence a bin; 4 + 3 + 2 + 1 + 2 chunks -> four tiles, four bins,
one of them two sequences), checked on bf16 d = 128 with ragged lengths
against the fp64 oracle on every head.  The scan reads either the chunk's W
and U (X = U - W S) or A and the raw rows (X = A B (V - Gamma K S)); within a
form every split runs the same MFMAs in the same order for a sequence, so the
results must also agree bitwise across them (the same head, same tokens, in
batches of different sizes), and across the two forms within the rounding of
their different products.
"""
import dataclasses

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


@pytest.mark.parametrize("lens", [[197], [197, 130], [197, 130, 65, 1, 100]])
def test_state_scan_tiling_matches_oracle(torch_cuda, oracle_mod, lens):
    inp = gdn_inputs.make_prefill(seed=700, seqlens=lens, H_q=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
                                  state_std=0.02)
    out, fin = chunk_fwd_device(inp)
    ref_o, ref_s = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, 16, 32,
                                      inp.scale, initial_state=inp.initial_state.astype(np.float64))
    assert rel_err(out, ref_o) < 1e-2
    assert rel_err(fin, ref_s) < 1e-2


@pytest.mark.parametrize("form", ["W", "A"])
def test_state_scan_tiling_bitwise_consistent(torch_cuda, form):
    """The first sequence alone (one tile a CU), with one more (two), and with
    four more (four tiles a workgroup), in one form of the scan's operands:
    its outputs and final state agree bit for bit."""
    full = gdn_inputs.make_prefill(seed=701, seqlens=[197, 130, 65, 1, 100], H_q=16, H_v=32, d_k=128, d_v=128,
                                   dtype="bf16", state_std=0.02)
    res = []
    for n in (1, 2, 5):
        t = int(full.cu_seqlens[n])
        sub = dataclasses.replace(full, q=full.q[:t], k=full.k[:t], v=full.v[:t], g=full.g[:t], beta=full.beta[:t],
                                  cu_seqlens=full.cu_seqlens[:n + 1], initial_state=full.initial_state[:n])
        out, fin = chunk_fwd_device(sub, form=form)
        res.append((out[:197], fin[0]))
    for o, f in res[1:]:
        assert np.array_equal(o, res[0][0]) and np.array_equal(f, res[0][1])


def test_state_scan_forms_agree(torch_cuda):
    """The two forms of the scan's operands on one batch: within the rounding of
    their different products (each is held to the oracle elsewhere)."""
    inp = gdn_inputs.make_prefill(seed=704, seqlens=[197, 130, 65, 1, 100], H_q=16, H_v=32, d_k=128, d_v=128,
                                  dtype="bf16", state_std=0.02)
    ow, fw = chunk_fwd_device(inp, form="W")
    oa, fa = chunk_fwd_device(inp, form="A")
    assert rel_err(oa, ow) < 1e-2 and rel_err(fa, fw) < 1e-2


@pytest.mark.parametrize("n_seq,d", [(8, 128), (40, 128), (40, 64)])
def test_state_scan_tiling_odd_heads_many_sequences(torch_cuda, oracle_mod, n_seq, d):
    """Five value heads on five key heads (groups not a multiple of 8, so the
    per-XCD grid is padded) over many short ragged sequences, with empty ones:
    bins of several sequences a workgroup at every tile width."""
    lens = [int(x) for x in np.random.default_rng(702 + n_seq + d).integers(0, 140, n_seq)]
    inp = gdn_inputs.make_prefill(seed=703 + n_seq, seqlens=lens, H_q=5, H_v=5, d_k=d, d_v=d, dtype="bf16",
                                  state_std=0.02)
    out, fin = chunk_fwd_device(inp)
    ref_o, ref_s = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, 5, 5,
                                      inp.scale, initial_state=inp.initial_state.astype(np.float64))
    assert rel_err(out, ref_o) < 1e-2
    assert rel_err(fin, ref_s) < 1e-2


@pytest.mark.parametrize("d", [128, 64])
def test_state_scan_every_width_bins_bitwise(torch_cuda, oracle_mod, d):
    """Each work split of the state scan forced on one batch: 1, 2 and 4
    column tiles a workgroup, each with as many bins as fit on a 256-CU part
    (H_v = 4, d = 128: 8 / 16 / 32 bins; d = 64: 16 / 32 / 40), so 40 ragged
    sequences, some empty, make bins of several sequences at every width,
    including the widths whose three-stage ring reads the next chunk's stage
    half a step early, across sequence changes.  In each form of the scan's
    operands the three results agree bit for bit and match the oracle on every
    head."""
    lens = [int(x) for x in np.random.default_rng(710 + d).integers(0, 300, 40)]
    for i in (3, 17, 39):
        lens[i] = 0
    inp = gdn_inputs.make_prefill(seed=711 + d, seqlens=lens, H_q=2, H_v=4, d_k=d, d_v=d, dtype="bf16",
                                  state_std=0.02)
    ref_o, ref_s = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, 2, 4,
                                      inp.scale, initial_state=inp.initial_state.astype(np.float64))
    for form in ("W", "A"):
        res = {}
        for ct in (1, 2, 4):
            print(f"[widths] d={d} form={form} scan_ct={ct} T={inp.T}", flush=True)
            res[ct] = chunk_fwd_device(inp, scan_ct=ct, form=form)
        for ct in (2, 4):
            assert np.array_equal(res[ct][0], res[1][0]), (form, ct)
            assert np.array_equal(res[ct][1], res[1][1]), (form, ct)
        assert rel_err(res[1][0], ref_o) < 1e-2, form
        assert rel_err(res[1][1], ref_s) < 1e-2, form


def test_state_scan_bins_short_sequences_pool_and_empties(torch_cuda, oracle_mod):
    """80 requests of 1..199 tokens, every tenth empty, at H_v = 32, d = 128,
    over a state pool: the first launch group's 64 sequences go four bins of
    about 16 sequences (four tiles a workgroup), the last 16 into bins of
    their own shape.  Sampled heads against the oracle; an empty sequence ends
    in the state it starts from (its cached row, or zeros without one); pool
    rows no sequence names are untouched."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    rng = np.random.default_rng(704)
    lens = [int(x) for x in rng.integers(1, 200, 80)]
    for i in range(0, 80, 10):
        lens[i] = 0
    n, H_q, H_v, d, P = len(lens), 16, 32, 128, 96
    inp = gdn_inputs.make_prefill(seed=705, seqlens=lens, H_q=H_q, H_v=H_v, d_k=d, d_v=d, dtype="bf16",
                                  state_std=None)
    pool0 = gdn_inputs.make_decode_state(706, P, H_v, d, d)
    slots = [int(x) for x in rng.permutation(P)[:n]]
    slots[3] = -1  # no row: starts from zeros, final state not kept
    has = [int(x) for x in rng.integers(0, 2, n)]
    has[0] = 1   # an empty sequence with a cached prefix keeps its row
    has[10] = 0  # an empty sequence without one ends in zeros
    pool = f32_dev(pool0)
    dev = [to_dev(inp.q, "bf16"), to_dev(inp.k, "bf16"), to_dev(inp.v, "bf16"), f32_dev(inp.g), f32_dev(inp.beta)]
    print(f"[bins] {n} sequences, T={inp.T}, H_v={H_v}, pool={P}", flush=True)
    out = gdn.chunk_fwd_pooled(*dev, inp.cu_seqlens, pool, slots, has)
    torch.cuda.synchronize()
    init = np.zeros((n, H_v, d, d))
    for i, (r, hv) in enumerate(zip(slots, has)):
        if r >= 0 and hv:
            init[i] = pool0[r]
    heads = [0, 17, 31]
    ref_o, ref_s = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, H_q, H_v,
                                      inp.scale, initial_state=init, heads=heads)
    oh, ph = to_host(out), to_host(pool)
    for h in heads:
        assert rel_err(oh[:, h], ref_o[:, h]) < 1e-2, h
        fin = np.stack([ph[r, h] if r >= 0 else ref_s[i, h] for i, r in enumerate(slots)])
        assert rel_err(fin, ref_s[:, h]) < 1e-2, h
    for i in range(0, n, 10):
        r = slots[i]
        if r >= 0:
            assert np.array_equal(ph[r], init[i]), f"empty sequence {i}"
    for r in sorted(set(range(P)) - {r for r in slots if r >= 0}):
        assert np.array_equal(ph[r], pool0[r].astype(np.float64)), f"row {r} touched"
