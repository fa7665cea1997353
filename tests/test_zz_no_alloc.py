"""gdn_chunk_fwd_scratch (the prefill whose workspace is the library's static
device array, for callers that cannot allocate) against gdn_chunk_fwd with a
caller-provided workspace, both called through the C ABI: two calls in a row
on the shared array, the second on a smaller batch, each bit-identical to the
plain entry point on the same inputs (the same kernels run on the same data).
"""
import ctypes

import numpy as np
import pytest

import gdn_inputs
from tests.gpu_helpers import f32_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_state_chunk_amd as gdn

    gdn.load_library()
    return torch


def _run_both(torch, gdn, inp):
    lib = gdn.load_library()
    dt = gdn.DTYPE_BF16 if inp.dtype == "bf16" else gdn.DTYPE_F32
    q, k, v = (to_dev(getattr(inp, n), inp.dtype) for n in ("q", "k", "v"))
    g, beta, s0 = f32_dev(inp.g), f32_dev(inp.beta), f32_dev(inp.initial_state)
    N = len(inp.cu_seqlens) - 1
    cu = (ctypes.c_int32 * (N + 1))(*[int(x) for x in inp.cu_seqlens])
    shape_o, shape_s = (inp.T, inp.H_v, inp.d_v), (N, inp.H_v, inp.d_k, inp.d_v)
    outs = []
    for use_scratch in (True, False):
        out = torch.full(shape_o, float("nan"), dtype=q.dtype, device="cuda")
        fin = torch.full(shape_s, float("nan"), dtype=torch.float32, device="cuda")
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        common = (q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), cu, N, s0.data_ptr(),
                  out.data_ptr(), fin.data_ptr(), inp.T, inp.H_q, inp.H_v, inp.d_k, inp.d_v, inp.scale, dt)
        if use_scratch:
            rc = lib.gdn_chunk_fwd_scratch(*common, stream)
        else:
            nbytes = lib.gdn_chunk_fwd_workspace_size(cu, N, inp.H_q, inp.H_v, inp.d_k, inp.d_v, dt)
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            rc = lib.gdn_chunk_fwd(*common, ws.data_ptr(), nbytes, stream)
        assert rc == 0, lib.gdn_strerror(rc)
        torch.cuda.synchronize()
        outs.append((out, fin))
    return outs


def test_scratch_prefill_matches_workspace_prefill_twice(torch_cuda):
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    # first: the 4096-token, 32-value-head batch (193 MiB of the 256 MiB array);
    # second: a smaller packed batch with ragged tails, so stale contents of the
    # first call sit past every region the second one uses
    big = gdn_inputs.make_prefill(seed=301, seqlens=[4096], H_q=16, H_v=32, d_k=128, d_v=128, dtype="bf16")
    small = gdn_inputs.make_prefill(seed=302, seqlens=[200, 1, 77, 64], H_q=2, H_v=4, d_k=128, d_v=128,
                                    dtype="bf16")
    for name, inp in (("T=4096 H_v=32", big), ("4 sequences H_v=4", small)):
        print(f"[no-alloc] {name}", flush=True)
        (o_s, f_s), (o_w, f_w) = _run_both(torch, gdn, inp)
        assert not torch.isnan(o_s.float()).any() and not torch.isnan(f_s).any()
        assert torch.equal(o_s, o_w), name
        assert torch.equal(f_s, f_w), name
    # the smaller call again after the larger one: still equal (stream-ordered reuse)
    (o_s, f_s), (o_w, f_w) = _run_both(torch, gdn, small)
    assert torch.equal(o_s, o_w) and torch.equal(f_s, f_w)


def test_scratch_prefill_refuses_oversized_batch(torch_cuda):
    import gated_deltanet_state_chunk_amd as gdn

    torch = torch_cuda
    inp = gdn_inputs.make_prefill(seed=303, seqlens=[8192], H_q=16, H_v=32, d_k=128, d_v=128, dtype="bf16")
    out = torch.full((inp.T, 32, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.chunk_fwd_scratch(to_dev(inp.q, "bf16"), to_dev(inp.k, "bf16"), to_dev(inp.v, "bf16"), f32_dev(inp.g),
                              f32_dev(inp.beta), inp.cu_seqlens, out=out)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    assert np.isfinite(gdn.SCRATCH_BYTES)
