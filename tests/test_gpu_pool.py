"""GPU tests of the state-pool entry points (serving-state plumbing): prefill
and decode read and write per-request rows of a state pool by slot, padding
slots leave the pool alone and give zero outputs, has_initial picks which
sequences resume a cached state, and pool rows can be reset or cloned.

The "Qwen3.5-397B-A17B" trace page (section 3.6.6) asks that a GDN check cover
the output, the conv state and the SSM state over consecutive steps, with
padding and slot reuse; these tests do that against the fp64 oracle
(tolerances as the other parity tests: max|err| / max|ref| <= 1e-4 fp32,
1e-2 bf16; conv histories hold raw inputs, so they match bit for bit), and
check that each pooled call is bit-identical to the unpooled call on the
gathered states.
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


def _gather(pool0, slots, has, shape):
    init = np.zeros(shape, np.float32)
    for i, (r, h) in enumerate(zip(slots, has)):
        if r >= 0 and h:
            init[i] = pool0[r]
    return init


@pytest.mark.parametrize("dtype,gated", [("f32", False), ("bf16", False), ("bf16", True)])
def test_chunk_pooled(torch_cuda, oracle_mod, dtype, gated):
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    lens = [65, 0, 130, 7, 64, 0]
    slots = [7, 4, 2, -1, 0, 8]
    has = [1, 1, 0, 1, 1, 0]
    H_q, H_v, d, P = 2, 4, 128, 9
    inp = gdn_inputs.make_prefill(91, lens, H_q, H_v, d, d, dtype, state_std=None)
    pool0 = gdn_inputs.make_decode_state(92, P, H_v, d, d)
    pool = f32_dev(pool0)
    cu = inp.cu_seqlens
    dev = [to_dev(inp.q, dtype), to_dev(inp.k, dtype), to_dev(inp.v, dtype), f32_dev(inp.g), f32_dev(inp.beta)]
    gate = None
    if gated:
        z, w = gdn_inputs.make_gate(93, inp.T, H_v, d, dtype)
        gate = (to_dev(z, dtype), f32_dev(w), 1e-6)
    out = gdn.chunk_fwd_pooled(*dev, cu, pool, slots, has, gate=gate)
    init = _gather(pool0, slots, has, (len(lens), H_v, d, d))

    # bit-identical to the unpooled call on the gathered states
    out2, fin2 = gdn.chunk_fwd(*dev, cu, initial_state=f32_dev(init), gate=gate)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    for i, r in enumerate(slots):
        if r >= 0:
            assert torch.equal(pool[r], fin2[i]), f"slot {r}"
    pool_h = to_host(pool)
    for r in set(range(P)) - {r for r in slots if r >= 0}:
        assert np.array_equal(pool_h[r], pool0[r].astype(np.float64)), f"row {r} touched"

    # and within tolerance of the oracle
    ref_o, ref_fin = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, cu, H_q, H_v, inp.scale,
                                        init)
    for i, r in enumerate(slots):
        if r >= 0:
            assert rel_err(pool_h[r], ref_fin[i]) < TOL[dtype], f"state of sequence {i}"
    if gated:
        ref_o = oracle_mod.gated_rmsnorm(ref_o, gdn_inputs.storage_to_f32(z, dtype), w, 1e-6)
    assert rel_err(to_host(out), ref_o) < TOL[dtype]
    # the empty sequence without a cached prefix leaves a zero state in its row
    assert not pool_h[8].any()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_pooled(torch_cuda, oracle_mod, dtype):
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    lens = [1, 2, 70, 0, 5]
    slots = [3, -1, 0, 5, 1]
    has = [1, 1, 0, 1, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, C, K, P = int(cu[-1]), 64, 4, 6
    x, pool0, w, b = gdn_inputs.make_conv(94, T, C, K, P, dtype)
    pool = to_dev(pool0, dtype)
    xd, wd, bd = to_dev(x, dtype), f32_dev(w), f32_dev(b)
    out = gdn.conv1d_silu_pooled(xd, cu, wd, bd, pool, slots, has)
    pool32 = gdn_inputs.storage_to_f32(pool0, dtype)
    init = _gather(pool32, slots, has, (len(lens), K - 1, C))
    out2, fin2 = gdn.conv1d_silu(xd, cu, wd, bd, initial_state=to_dev(gdn_inputs.round_to(init, dtype), dtype))
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    ref, ref_fin = oracle_mod.conv_silu_varlen(gdn_inputs.storage_to_f32(x, dtype), cu, w, b, init)
    assert rel_err(to_host(out), ref) < {"f32": 1e-5, "bf16": 1e-2}[dtype]
    pool_h = to_host(pool)
    for i, r in enumerate(slots):
        if r >= 0:
            assert np.array_equal(pool_h[r], ref_fin[i]), f"history of sequence {i}"
    for r in set(range(P)) - {r for r in slots if r >= 0}:
        assert np.array_equal(pool_h[r], pool32[r].astype(np.float64)), f"row {r} touched"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_pooled_with_padding(torch_cuda, oracle_mod, dtype):
    """Two fused steps and two conv steps over pools, with a negative and an
    out-of-range slot as padding."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    N, H_q, H_v, d, P = 5, 2, 4, 128, 7
    slots = [4, -1, 0, 9, 2]
    valid = [i for i, r in enumerate(slots) if 0 <= r < P]
    pad = [i for i in range(N) if i not in valid]
    scale = 1.0 / np.sqrt(d)
    pool0 = gdn_inputs.make_decode_state(95, P, H_v, d, d)
    pool = f32_dev(pool0)
    slot_dev = torch.tensor(slots, dtype=torch.int32, device="cuda")
    ref = np.zeros((N, H_v, d, d))
    for i in valid:
        ref[i] = pool0[slots[i]]
    C, K = 64, 3
    _, cpool0, w, b = gdn_inputs.make_conv(96, 1, C, K, P, dtype)
    cpool = to_dev(cpool0, dtype)
    cref = np.zeros((N, K - 1, C))
    for i in valid:
        cref[i] = gdn_inputs.storage_to_f32(cpool0, dtype)[slots[i]]
    for step in range(2):
        tok = gdn_inputs.make_decode_raw_token(960 + step, N, H_q, H_v, d, d, dtype)
        args = [to_dev(getattr(tok, n), dtype) for n in ("q", "k", "v", "a", "b")]
        # the unpooled step on the gathered states must agree bit for bit
        gathered = pool[slot_dev[valid].long()].clone()
        o = gdn.recurrent_step_fused_pooled(*args, f32_dev(tok.A_log), f32_dev(tok.dt_bias), pool, slot_dev,
                                            scale=scale)
        o2 = gdn.recurrent_step_fused(*[t[valid].contiguous() for t in args], f32_dev(tok.A_log),
                                      f32_dev(tok.dt_bias), gathered, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o[valid], o2)
        assert not o[pad].any()
        ref_o = oracle_mod.decode_step_fused(tok.f32("q"), tok.f32("k"), tok.f32("v"), tok.f32("a"), tok.f32("b"),
                                             tok.A_log, tok.dt_bias, ref, H_q, H_v, scale, dtype == "bf16")[0]
        assert rel_err(to_host(o)[valid], ref_o[valid]) < TOL[dtype], f"step {step}"

        xs = gdn_inputs.make_conv(970 + step, N, C, K, 1, dtype, with_state=False)[0]
        y = gdn.conv1d_silu_step_pooled(to_dev(xs, dtype), f32_dev(w), f32_dev(b), cpool, slot_dev)
        ref_y = oracle_mod.conv_silu_step(gdn_inputs.storage_to_f32(xs, dtype), w, b, cref)
        assert not y[pad].any()
        assert rel_err(to_host(y)[valid], ref_y[valid]) < {"f32": 1e-5, "bf16": 1e-2}[dtype]
    pool_h, cpool_h = to_host(pool), to_host(cpool)
    for i in valid:
        assert rel_err(pool_h[slots[i]], ref[i]) < TOL[dtype]
        assert np.array_equal(cpool_h[slots[i]], cref[i])
    for r in set(range(P)) - {slots[i] for i in valid}:
        assert np.array_equal(pool_h[r], pool0[r].astype(np.float64)), f"row {r} touched"
        assert np.array_equal(cpool_h[r], gdn_inputs.storage_to_f32(cpool0, dtype)[r].astype(np.float64))


def test_state_rows_zero_and_copy(torch_cuda):
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    g = torch.Generator(device="cuda").manual_seed(97)
    # rows of 2.5 MiB: more 16-byte units than one launch column covers at once
    pool = torch.randn((6, 40, 128, 128), device="cuda", generator=g)
    before = pool.clone()
    rows = torch.tensor([0, -1, 7, 2], dtype=torch.int32, device="cuda")
    gdn.state_rows_zero(pool, rows)
    expect = before.clone()
    expect[0] = 0
    expect[2] = 0
    torch.cuda.synchronize()
    assert torch.equal(pool, expect)

    # one source feeding two rows; a negative source and a row past the pool are skipped
    cur = pool.clone()
    src = torch.tensor([1, 1, 4, -3, 4], dtype=torch.int32, device="cuda")
    dst = torch.tensor([3, 5, 0, 2, 9], dtype=torch.int32, device="cuda")
    gdn.state_rows_copy(pool, src, dst)
    expect = cur.clone()
    expect[3] = cur[1]
    expect[5] = cur[1]
    expect[0] = cur[4]
    torch.cuda.synchronize()
    assert torch.equal(pool, expect)

    hist = torch.randn((5, 3, 8192), device="cuda", generator=g).to(torch.bfloat16)
    h0 = hist.clone()
    gdn.state_rows_copy(hist, torch.tensor([2], dtype=torch.int32, device="cuda"),
                        torch.tensor([4], dtype=torch.int32, device="cuda"))
    h0[4] = h0[2]
    torch.cuda.synchronize()
    assert torch.equal(hist, h0)


def test_serving_sequence(torch_cuda, oracle_mod):
    """Prefill three prompts into a pool (GDN and conv), decode three tokens in
    another batch order with a padding slot, then clone one request's states
    into a free slot (a speculative branch) and step both copies alike."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    dtype, H_q, H_v, d, P, C, K = "bf16", 2, 4, 128, 6, 128, 4
    scale = 1.0 / np.sqrt(d)
    lens, pre_slots = [70, 9, 130], [5, 1, 3]
    inp = gdn_inputs.make_prefill(98, lens, H_q, H_v, d, d, dtype, state_std=None)
    cu = inp.cu_seqlens
    pool = torch.zeros((P, H_v, d, d), dtype=torch.float32, device="cuda")
    cpool = torch.zeros((P, K - 1, C), dtype=torch.bfloat16, device="cuda")
    x, _, w, b = gdn_inputs.make_conv(99, inp.T, C, K, 1, dtype, with_state=False)
    wd, bd = f32_dev(w), f32_dev(b)
    gdn.chunk_fwd_pooled(to_dev(inp.q, dtype), to_dev(inp.k, dtype), to_dev(inp.v, dtype), f32_dev(inp.g),
                         f32_dev(inp.beta), cu, pool, pre_slots, has_initial=[0, 0, 0])
    gdn.conv1d_silu_pooled(to_dev(x, dtype), cu, wd, bd, cpool, pre_slots, has_initial=[0, 0, 0])
    _, fin = oracle_mod.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, cu, H_q, H_v, inp.scale)
    _, cfin = oracle_mod.conv_silu_varlen(gdn_inputs.storage_to_f32(x, dtype), cu, w, b)

    order = [2, -1, 0, 1]                       # request index per batch row; -1 padding
    slot_dev = torch.tensor([pre_slots[r] if r >= 0 else -1 for r in order], dtype=torch.int32, device="cuda")
    valid = [i for i, r in enumerate(order) if r >= 0]
    ref = np.zeros((len(order), H_v, d, d))
    cref = np.zeros((len(order), K - 1, C))
    for i in valid:
        ref[i], cref[i] = fin[order[i]], cfin[order[i]]

    def step(seed, slots_dev, ref, cref, n):
        tok = gdn_inputs.make_decode_raw_token(seed, n, H_q, H_v, d, d, dtype)
        xs = gdn_inputs.make_conv(seed + 1, n, C, K, 1, dtype, with_state=False)[0]
        y = gdn.conv1d_silu_step_pooled(to_dev(xs, dtype), wd, bd, cpool, slots_dev)
        ref_y = oracle_mod.conv_silu_step(gdn_inputs.storage_to_f32(xs, dtype), w, b, cref)
        o = gdn.recurrent_step_fused_pooled(*[to_dev(getattr(tok, m), dtype) for m in ("q", "k", "v", "a", "b")],
                                            f32_dev(tok.A_log), f32_dev(tok.dt_bias), pool, slots_dev, scale=scale)
        ref_o = oracle_mod.decode_step_fused(tok.f32("q"), tok.f32("k"), tok.f32("v"), tok.f32("a"), tok.f32("b"),
                                             tok.A_log, tok.dt_bias, ref, H_q, H_v, scale, True)[0]
        return to_host(o), ref_o, to_host(y), ref_y

    for s in range(3):
        o, ref_o, y, ref_y = step(1000 + 10 * s, slot_dev, ref, cref, len(order))
        assert not o[1].any() and not y[1].any()
        assert rel_err(o[valid], ref_o[valid]) < 1e-2, f"decode step {s}"
        assert rel_err(y[valid], ref_y[valid]) < 1e-2, f"conv step {s}"
    pool_h, cpool_h = to_host(pool), to_host(cpool)
    for i in valid:
        assert rel_err(pool_h[pre_slots[order[i]]], ref[i]) < 1e-2
        assert np.array_equal(cpool_h[pre_slots[order[i]]], cref[i])
    for r in (0, 2, 4):
        assert not pool_h[r].any() and not cpool_h[r].any()

    # clone request 2 (slot 3) into free slot 0, then step both with the same inputs
    src = torch.tensor([3], dtype=torch.int32, device="cuda")
    dst = torch.tensor([0], dtype=torch.int32, device="cuda")
    gdn.state_rows_copy(pool, src, dst)
    gdn.state_rows_copy(cpool, src, dst)
    both = torch.tensor([3, 0], dtype=torch.int32, device="cuda")
    tok = gdn_inputs.make_decode_raw_token(1100, 1, H_q, H_v, d, d, dtype)
    dup = lambda a: np.concatenate([a, a])      # noqa: E731
    args = [to_dev(dup(getattr(tok, m)), dtype) for m in ("q", "k", "v", "a", "b")]
    o = gdn.recurrent_step_fused_pooled(*args, f32_dev(tok.A_log), f32_dev(tok.dt_bias), pool, both, scale=scale)
    xs = gdn_inputs.make_conv(1101, 1, C, K, 1, dtype, with_state=False)[0]
    y = gdn.conv1d_silu_step_pooled(to_dev(dup(xs), dtype), wd, bd, cpool, both)
    torch.cuda.synchronize()
    assert torch.equal(o[0], o[1]) and torch.equal(y[0], y[1])
    assert torch.equal(pool[3], pool[0]) and torch.equal(cpool[3], cpool[0])
    ref1 = ref[[0]].copy()                      # batch row 0 was request 2 (slot 3)
    ref_o = oracle_mod.decode_step_fused(tok.f32("q"), tok.f32("k"), tok.f32("v"), tok.f32("a"), tok.f32("b"),
                                         tok.A_log, tok.dt_bias, ref1, H_q, H_v, scale, True)[0]
    assert rel_err(to_host(o)[0], ref_o[0]) < 1e-2


def test_decode_graph_replay_with_new_slots(torch_cuda):
    """The pooled decode steps read their slots from device memory, so a
    captured graph replays with new slots and inputs; every replay must equal
    the same calls made eagerly on a second copy of the pools, bit for bit."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    dtype, N, H_q, H_v, d, P, C, K = "bf16", 4, 2, 4, 128, 6, 128, 4
    scale = 1.0 / np.sqrt(d)
    pool_g = f32_dev(gdn_inputs.make_decode_state(101, P, H_v, d, d))
    pool_e = pool_g.clone()
    _, cp0, w, b = gdn_inputs.make_conv(102, 1, C, K, P, dtype)
    cpool_g = to_dev(cp0, dtype)
    cpool_e = cpool_g.clone()
    wd, bd = f32_dev(w), f32_dev(b)
    tok0 = gdn_inputs.make_decode_raw_token(103, N, H_q, H_v, d, d, dtype)
    A_log, dt_bias = f32_dev(tok0.A_log), f32_dev(tok0.dt_bias)
    names = ("q", "k", "v", "a", "b")
    bufs = {m: to_dev(getattr(tok0, m), dtype) for m in names}
    x_b = to_dev(gdn_inputs.make_conv(104, N, C, K, 1, dtype, with_state=False)[0], dtype)
    slot_b = torch.zeros(N, dtype=torch.int32, device="cuda")
    o_b = torch.empty((N, H_v, d), dtype=torch.bfloat16, device="cuda")
    y_b = torch.empty((N, C), dtype=torch.bfloat16, device="cuda")

    def calls(pool, cpool, o, y):
        gdn.recurrent_step_fused_pooled(*[bufs[m] for m in names], A_log, dt_bias, pool, slot_b, scale=scale, out=o)
        gdn.conv1d_silu_step_pooled(x_b, wd, bd, cpool, slot_b, out=y)

    # warm-up outside capture on throwaway pools
    calls(pool_g.clone(), cpool_g.clone(), torch.empty_like(o_b), torch.empty_like(y_b))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(pool_g, cpool_g, o_b, y_b)
    torch.cuda.synchronize()

    for r, slots in enumerate([[5, 1, -1, 3], [1, 5, 3, 7], [0, -1, 2, 4]]):
        tok = gdn_inputs.make_decode_raw_token(110 + r, N, H_q, H_v, d, d, dtype)
        for m in names:
            bufs[m].copy_(to_dev(getattr(tok, m), dtype))
        x_b.copy_(to_dev(gdn_inputs.make_conv(120 + r, N, C, K, 1, dtype, with_state=False)[0], dtype))
        slot_b.copy_(torch.tensor(slots, dtype=torch.int32))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_e, y_e = torch.empty_like(o_b), torch.empty_like(y_b)
        calls(pool_e, cpool_e, o_e, y_e)
        torch.cuda.synchronize()
        assert torch.equal(o_b, o_e) and torch.equal(y_b, y_e), f"replay {r}"
        assert torch.equal(pool_g, pool_e) and torch.equal(cpool_g, cpool_e), f"replay {r}"
