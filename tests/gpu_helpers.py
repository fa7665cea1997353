"""Helpers for the GPU parity tests: host->device transfer of seeded inputs,
the error metric, and un-permuting the documented workspace layout."""
import numpy as np


def rel_err(x, ref) -> float:
    """max|x - ref| / max|ref| over the whole tensor (the metric the tolerances use)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def to_dev(arr, dtype: str, device="cuda"):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def f32_dev(arr, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_host(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def perm32_index(n: int) -> np.ndarray:
    """perm32 storage offset of each logical index 0..n-1 (n a multiple of 32)."""
    i = np.arange(n)
    blk, r = i & ~31, i & 31
    h, a, b = r >> 4, (r >> 2) & 3, r & 3
    return blk + 8 * a + 4 * h + b


def unperm32(stored: np.ndarray) -> np.ndarray:
    """Logical array from a perm32-stored one (permutation along the last axis)."""
    return stored[..., perm32_index(stored.shape[-1])]


def _split32(i):
    s, r = i // 32, i % 32
    return s, r // 16, (r % 16) // 4, r % 4


def frag_w_to_logical(flat, d_k):
    """W [..., 64*d_k] in fragment order -> [..., 64, d_k]."""
    pos = np.arange(64)[:, None]
    k = np.arange(d_k)[None, :]
    s, h, a, b = _split32(k)
    off = ((pos // 16 * (d_k // 32) + s) * 64 + 16 * a + pos % 16) * 8 + 4 * h + b
    return flat[..., off]


# A's fragments as the state scan reads them: (row tile t, K-step s) in this order
A_FRAG_TILES = [(0, 0), (1, 0), (2, 0), (2, 1), (3, 0), (3, 1)]


def a_frags_to_logical(flat):
    """A [..., 6*64*8] as six fragments (t, s) of A_FRAG_TILES, lane 16 a + r, slot
    4 h + b holding A[16 t + r][32 s + 16 h + 4 a + b] -> [..., 64, 64] (zero
    where no fragment is stored: the blocks above the diagonal)."""
    out = np.zeros(flat.shape[:-1] + (64, 64), dtype=flat.dtype)
    for f, (t, s) in enumerate(A_FRAG_TILES):
        for lane in range(64):
            a, r = lane // 16, lane % 16
            for h in range(2):
                for b in range(4):
                    out[..., 16 * t + r, 32 * s + 16 * h + 4 * a + b] = flat[..., (f * 64 + lane) * 8 + 4 * h + b]
    return out


def frag_rows_to_logical(flat, rows, cols):
    """[..., rows*cols] in the row-operand fragment order of Ht / Xt (block (row/16,
    col/32), lane 16 ((col%32)/8) + row%16, slot col%8) -> [..., rows, cols]."""
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    off = ((r // 16 * (cols // 32) + c // 32) * 64 + 16 * ((c % 32) // 8) + r % 16) * 8 + c % 8
    return flat[..., off]


def frag_u_to_logical(flat, d_v):
    """U [..., 64*d_v] in accumulator order -> [..., 64, d_v]."""
    pos = np.arange(64)[:, None]
    j = np.arange(d_v)[None, :]
    off = ((j // 16 * 2 + pos // 32) * 64 + 16 * ((pos % 16) // 4) + j % 16) * 8 + 4 * ((pos // 16) % 2) + pos % 4
    return flat[..., off]


def chunk_fwd_device(inp, device="cuda", initial_state="from_inputs", return_ws=False, keep_A=False, keep_hx=False,
                     scan_ct=None, keep_wu=False, form=None):
    """Run gdn_chunk_fwd on seeded inputs; returns (out, final, workspace-or-None) as host arrays / tensor."""
    import torch

    import gated_deltanet_state_chunk_amd as gdn

    q = to_dev(inp.q, inp.dtype, device)
    k = to_dev(inp.k, inp.dtype, device)
    v = to_dev(inp.v, inp.dtype, device)
    g = f32_dev(inp.g, device)
    beta = f32_dev(inp.beta, device)
    s0 = None
    if initial_state == "from_inputs" and inp.initial_state is not None:
        s0 = f32_dev(inp.initial_state, device)
    ws = torch.empty(max(gdn.workspace_size(inp.T, inp.cu_seqlens, inp.H_q, inp.H_v, inp.d_k, inp.d_v,
                                            inp.dtype), 1), dtype=torch.uint8, device=device)
    out, fin = gdn.chunk_fwd(q, k, v, g, beta, inp.cu_seqlens, initial_state=s0, scale=inp.scale, workspace=ws,
                             keep_A=keep_A, keep_hx=keep_hx, scan_ct=scan_ct, keep_wu=keep_wu, form=form)
    torch.cuda.synchronize()
    res = (to_host(out), to_host(fin))
    if return_ws:
        return res + (ws,)
    return res
