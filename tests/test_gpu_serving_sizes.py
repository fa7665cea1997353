"""GPU parity of the serving forms at the sizes the benchmark times them, on
sampled heads against the fp64 oracle.

* The prefill from raw inputs with the gated read-out ("Qwen3.5-397B-A17B"
  trace page, section 1, Prefill-GDN nodes 8-10 and 18), one sequence of 4096
  tokens, H_q = 16, H_v = 32, d = 128, bf16: there chunk_prep holds two
  (chunk, value head) items per workgroup, so the prefetch of the next item's
  raw gate inputs runs, which the small front-end tests never reach.
* The fused decode step over a state pool (section 3, Decode-GDN node 7, with
  the cache slots of section 3.6.5): 256 sequences x 32 value heads whose rows
  are a seeded permutation of a 512-row pool.

Tolerance max|err| / max|ref| <= 1e-2 (bf16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest

import gdn_inputs
from tests.gpu_helpers import f32_dev, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_state_chunk_amd as gdn

    gdn.load_library()
    return torch


def test_prefill_serving_T4096_sampled_heads(torch_cuda, oracle_mod):
    """The benchmark's prefill_serving line: the same seeds, shapes and gate."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    base = gdn_inputs.make_workload("prefill_T4096")
    seqlens = [int(x) for x in (base.cu_seqlens[1:] - base.cu_seqlens[:-1])]
    inp = gdn_inputs.make_prefill_raw(71, seqlens, base.H_q, base.H_v, base.d_k, base.d_v, base.dtype)
    z, w = gdn_inputs.make_gate(72, inp.T, inp.H_v, inp.d_v, inp.dtype)
    args = [to_dev(getattr(inp, n), inp.dtype) for n in ("q", "k", "v", "a", "b")]
    gate = (to_dev(z, inp.dtype), f32_dev(w), 1e-6)
    print(f"[serving] prefill T={inp.T} H_q={inp.H_q} H_v={inp.H_v} d={inp.d_k}", flush=True)
    out, fin = gdn.chunk_fwd_fused(*args, f32_dev(inp.A_log), f32_dev(inp.dt_bias), inp.cu_seqlens,
                                   initial_state=f32_dev(inp.initial_state), gate=gate)
    torch.cuda.synchronize()
    heads = [0, 1, 14, 31]  # both value heads of key head 0, an interior head, the last
    ref_o, ref_f = oracle_mod.forward_fused(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.f32("a"), inp.f32("b"),
                                            inp.A_log, inp.dt_bias, inp.cu_seqlens, inp.H_q, inp.H_v, inp.scale,
                                            True, initial_state=inp.initial_state, heads=heads)
    zf = gdn_inputs.storage_to_f32(z, inp.dtype)
    ref_y = oracle_mod.gated_rmsnorm(ref_o[:, heads], zf[:, heads], w, 1e-6)
    oh, fh = to_host(out), to_host(fin)
    for i, h in enumerate(heads):
        e_o = rel_err(oh[:, h], ref_y[:, i])
        e_s = rel_err(fh[:, h], ref_f[:, h])
        print(f"[serving] head {h}: out {e_o:.3e} final state {e_s:.3e}", flush=True)
        assert e_o < TOL and e_s < TOL, h


def _expand_heads(tok, heads, G):
    """The decode token restricted to value heads `heads`, each with its own copy
    of its key head's q and k (GVA as explicit head repetition, H_q = H_v)."""
    kq = [h // G for h in heads]
    sub = {n: tok.f32(n)[:, kq] for n in ("q", "k")}
    sub.update({n: tok.f32(n)[:, heads] for n in ("v", "a", "b")})
    return sub, tok.A_log[heads], tok.dt_bias[heads]


def test_pooled_fused_decode_256x32_over_512_rows(torch_cuda, oracle_mod):
    """The benchmark's decode_fused_pooled line (two steps): bitwise equal to the
    unpooled step on the gathered states, within tolerance of the oracle on
    sampled heads, and the 256 pool rows no sequence names left untouched."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    cfg = gdn_inputs.DECODE_WORKLOAD
    N, H_q, H_v, d, dt = cfg["N"], cfg["H_q"], cfg["H_v"], cfg["d_k"], cfg["dtype"]
    G, P = H_v // H_q, 2 * N
    scale = 1.0 / np.sqrt(d)
    state0 = gdn_inputs.make_decode_state(cfg["seed"], N, H_v, d, d, cfg["state_std"])
    rows = np.random.default_rng(cfg["seed"] + 1).permutation(P)[:N].astype(np.int32)
    slot = torch.tensor(rows, device="cuda")
    pool = torch.zeros((P, H_v, d, d), dtype=torch.float32, device="cuda")
    pool[slot.long()] = f32_dev(state0)
    free = np.setdiff1d(np.arange(P), rows)
    heads = [0, 3, 16, 31]
    ref = np.ascontiguousarray(state0[:, heads], dtype=np.float64)
    print(f"[serving] pooled decode N={N} H_v={H_v} pool={P}", flush=True)
    for s in range(2):
        tok = gdn_inputs.make_decode_raw_token(gdn_inputs.decode_step_seed(s), N, H_q, H_v, d, d, dt)
        args = [to_dev(getattr(tok, n), dt) for n in ("q", "k", "v", "a", "b")]
        A_log, dt_bias = f32_dev(tok.A_log), f32_dev(tok.dt_bias)
        gathered = pool[slot.long()].clone()
        o = gdn.recurrent_step_fused_pooled(*args, A_log, dt_bias, pool, slot, scale=scale)
        o2 = gdn.recurrent_step_fused(*args, A_log, dt_bias, gathered, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o2), f"step {s}: pooled and unpooled outputs differ"
        assert torch.equal(pool[slot.long()], gathered), f"step {s}: pooled and unpooled states differ"
        sub, A_s, b_s = _expand_heads(tok, heads, G)
        ref_o = oracle_mod.decode_step_fused(sub["q"], sub["k"], sub["v"], sub["a"], sub["b"], A_s, b_s, ref,
                                             len(heads), len(heads), scale, True)[0]
        e_o = rel_err(to_host(o)[:, heads], ref_o)
        e_s = rel_err(to_host(pool[slot.long()][:, heads]), ref)
        print(f"[serving] step {s}: out {e_o:.3e} state {e_s:.3e}", flush=True)
        assert e_o < TOL and e_s < TOL, s
    assert not pool[torch.tensor(free, device="cuda").long()].any(), "a pool row no sequence names was written"


def test_binding_refuses_wrong_shaped_output_buffers(torch_cuda):
    """Caller-supplied outputs of the wrong shape are refused before any launch
    (the kernels would write past their end); the buffers keep their contents."""
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    inp = gdn_inputs.make_prefill(5, [70, 30], 2, 4, 64, 64, "bf16")
    q, k, v = (to_dev(getattr(inp, n), "bf16") for n in ("q", "k", "v"))
    g, beta = f32_dev(inp.g), f32_dev(inp.beta)
    T, N = inp.T, 2
    short = torch.full((T - 1, 4, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        gdn.chunk_fwd(q, k, v, g, beta, inp.cu_seqlens, out=short)
    fin_bad = torch.full((N, 4, 64, 32), float("nan"), device="cuda")
    with pytest.raises(ValueError):
        gdn.chunk_fwd(q, k, v, g, beta, inp.cu_seqlens, final_state=fin_bad)
    with pytest.raises(ValueError):
        gdn.chunk_fwd_dev(q, k, v, g, beta, torch.tensor(inp.cu_seqlens, dtype=torch.int32, device="cuda"),
                          out=short)
    tok = gdn_inputs.make_decode_token(6, 3, 2, 4, 64, 64, "bf16")
    st = f32_dev(gdn_inputs.make_decode_state(7, 3, 4, 64, 64))
    st0 = st.clone()
    o_bad = torch.full((2, 4, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        gdn.recurrent_step(*(to_dev(getattr(tok, n), "bf16") for n in ("q", "k", "v")), f32_dev(tok.g),
                           f32_dev(tok.beta), st, out=o_bad)
    x = torch.zeros((10, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    y_bad = torch.full((9, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        gdn.conv1d_silu(x, [0, 10], w, out=y_bad)
    with pytest.raises(ValueError):
        gdn.conv1d_silu_step(x, w, None, torch.zeros((10, 3, 64), dtype=torch.bfloat16, device="cuda"), out=y_bad)
    torch.cuda.synchronize()
    assert torch.isnan(short.float()).all() and torch.isnan(fin_bad).all() and torch.isnan(o_bad.float()).all()
    assert torch.isnan(y_bad.float()).all() and torch.equal(st, st0)
