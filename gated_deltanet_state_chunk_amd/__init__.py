"""Gated DeltaNet forward pass on MI355X (gfx950): Python binding of libgdn.so.

Argument marshalling only — every step of the computation runs in the HIP
kernels of libgdn.so (see include/gdn.h for the C ABI, layouts and errors).
PyTorch supplies device memory and the current stream.  There is no fallback:
if libgdn.so is missing, importing the library functions raises.

    import gated_deltanet_state_chunk_amd as gdn
    out, final_state = gdn.chunk_fwd(q, k, v, g, beta, cu_seqlens, initial_state)
    o = gdn.recurrent_step(q1, k1, v1, g1, beta1, state)   # state updated in place
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

__all__ = ["chunk_fwd", "chunk_form", "chunk_fwd_scratch", "SCRATCH_BYTES", "recurrent_step", "recurrent_step_fused", "conv1d_silu", "conv1d_silu_step",
           "chunk_fwd_fused", "chunk_fwd_dev", "chunk_fwd_pooled", "conv1d_silu_pooled", "recurrent_step_fused_pooled", "conv1d_silu_step_pooled",
           "state_rows_zero", "state_rows_copy", "stream_copy", "workspace_layout", "workspace_size", "lib_path", "load_library",
           "GdnError", "CHUNK", "DTYPE_F32", "DTYPE_BF16"]

CHUNK = 64
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdn.so")
_lib = None

DTYPE_F32 = 0
DTYPE_BF16 = 1
FWD_KEEP_A = 1  # gdn_chunk_fwd_ex flag: also write A to the workspace
FWD_KEEP_HX = 2  # gdn_chunk_fwd_ex flag: also write Ht and Xt (bf16 forms the output on chip)
FWD_SCAN_CT = {1: 4, 2: 8, 4: 16}  # gdn_chunk_fwd_ex flags: the state scan's column tiles a workgroup (bf16)
FWD_KEEP_WU = 32  # gdn_chunk_fwd_ex flag: also form W and U in the workspace
FWD_FORM = {"W": 64, "A": 128}  # gdn_chunk_fwd_ex flags: the state scan's operand form (bf16)
SCRATCH_BYTES = 256 << 20  # GDN_SCRATCH_BYTES: the static workspace of gdn_chunk_fwd_scratch

_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace", -4: "hip"}


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        lib = load_library()
        msg = lib.gdn_strerror(status).decode()  # names the HIP error too for a failed launch
        super().__init__(f"{what}: {msg} ({status})")
        self.status = status


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [("n_chunks", ctypes.c_int64), ("off_gates", ctypes.c_size_t), ("off_A", ctypes.c_size_t),
                ("off_Af", ctypes.c_size_t), ("off_W", ctypes.c_size_t), ("off_U", ctypes.c_size_t),
                ("off_Kc", ctypes.c_size_t), ("off_Ht", ctypes.c_size_t), ("off_Xt", ctypes.c_size_t),
                ("off_P", ctypes.c_size_t), ("off_Qc", ctypes.c_size_t),
                ("total_bytes", ctypes.c_size_t)]


class OutputGate(ctypes.Structure):
    """gdn_output_gate: read-out epilogue out = rmsnorm(o) * weight * silu(z)."""
    _fields_ = [("z", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("eps", ctypes.c_float)]


class FrontEnd(ctypes.Structure):
    """gdn_front_end: raw gate inputs a, b and the per-head A_log, dt_bias."""
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p)]


class StateSlots(ctypes.Structure):
    """gdn_state_slots: host pool rows of a prefill's sequences (-1: none) and which resume."""
    _fields_ = [("slot", ctypes.POINTER(ctypes.c_int32)), ("has_initial", ctypes.POINTER(ctypes.c_uint8)),
                ("pool_size", ctypes.c_int32)]


def _slots_arg(slots, has_initial, pool_size, N):
    """(host slots, host has_initial or None, pool rows) -> (StateSlots, keep-alive)."""
    torch = _torch()
    vals = [int(x) for x in (slots.tolist() if isinstance(slots, torch.Tensor) else slots)]
    if len(vals) != N:
        raise ValueError(f"slots must have one entry per sequence ({N}), got {len(vals)}")
    sl = (ctypes.c_int32 * max(N, 1))(*vals)
    hi = None
    if has_initial is not None:
        flags = [1 if bool(x) else 0 for x in (has_initial.tolist() if isinstance(has_initial, torch.Tensor)
                                               else has_initial)]
        if len(flags) != N:
            raise ValueError("has_initial must have one entry per sequence")
        hi = (ctypes.c_uint8 * max(N, 1))(*flags)
    st = StateSlots(ctypes.cast(sl, ctypes.POINTER(ctypes.c_int32)),
                    ctypes.cast(hi, ctypes.POINTER(ctypes.c_uint8)) if hi is not None else None, int(pool_size))
    return st, (sl, hi)


def _check_slot_dev(slot, N):
    torch = _torch()
    _check_dev("slot", slot, torch.int32)
    if tuple(slot.shape) != (N,):
        raise ValueError(f"slot must be int32 [{N}]")


def _gate_arg(gate, dtype, rows, H_v, d_v):
    """(z, weight, eps) -> (ctypes pointer or None, keep-alive)."""
    if gate is None:
        return None, None
    torch = _torch()
    z, weight, eps = gate
    _check_dev("z", z, dtype)
    _check_dev("gate weight", weight, torch.float32)
    if tuple(z.shape) != (rows, H_v, d_v) or tuple(weight.shape) != (d_v,):
        raise ValueError("gate: z must be [rows, H_v, d_v] and weight [d_v]")
    g = OutputGate(_ptr(z), _ptr(weight), float(eps))
    return ctypes.byref(g), g


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgdn.so (built in-tree by gated_deltanet_state_chunk_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m gated_deltanet_state_chunk_amd.build`")
    # torch first: its HIP runtime (soname libamdhip64.so.7) then satisfies
    # libgdn.so's dependency, so streams and memory come from one runtime.
    _torch()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.gdn_version.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_strerror.argtypes = [ctypes.c_int]
    lib.gdn_strerror.restype = ctypes.c_char_p
    lib.gdn_last_hip_error.restype = ctypes.c_char_p
    lib.gdn_chunk_fwd_workspace_layout.argtypes = [I32, I32, P, I32, I32, I32, I32, ctypes.c_int,
                                                   ctypes.POINTER(WorkspaceLayout)]
    lib.gdn_chunk_fwd_workspace_layout.restype = ctypes.c_int
    lib.gdn_chunk_fwd_workspace_size.argtypes = [P, I32, I32, I32, I32, I32, ctypes.c_int]
    lib.gdn_chunk_fwd_workspace_size.restype = ctypes.c_size_t
    lib.gdn_chunk_fwd_form.argtypes = [I32, I32, I32, I32, ctypes.c_int]
    lib.gdn_chunk_fwd_form.restype = ctypes.c_int
    lib.gdn_chunk_fwd.argtypes = [P, P, P, P, P, P, I32, P, P, P, I32, I32, I32, I32, I32, F, ctypes.c_int, P,
                                  ctypes.c_size_t, P]
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_fwd_ex.argtypes = lib.gdn_chunk_fwd.argtypes + [ctypes.c_uint32, P, P]
    lib.gdn_chunk_fwd_scratch.argtypes = [P, P, P, P, P, P, I32, P, P, P, I32, I32, I32, I32, I32, F, ctypes.c_int, P]
    lib.gdn_chunk_fwd_scratch.restype = ctypes.c_int
    lib.gdn_chunk_fwd_ex.restype = ctypes.c_int
    lib.gdn_recurrent_step.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, F, ctypes.c_int, P]
    lib.gdn_recurrent_step.restype = ctypes.c_int
    lib.gdn_recurrent_step_fused.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, F, ctypes.c_int, P,
                                             P]
    lib.gdn_recurrent_step_fused.restype = ctypes.c_int
    lib.gdn_conv1d_silu_fwd.argtypes = [P, P, I32, I32, I32, I32, P, P, P, P, P, ctypes.c_int, P]
    lib.gdn_conv1d_silu_fwd.restype = ctypes.c_int
    lib.gdn_conv1d_silu_step.argtypes = [P, I32, I32, I32, P, P, P, P, ctypes.c_int, P]
    lib.gdn_conv1d_silu_step.restype = ctypes.c_int
    SL = ctypes.POINTER(StateSlots)
    lib.gdn_chunk_fwd_pooled.argtypes = [P, P, P, P, P, P, I32, P, SL, P, I32, I32, I32, I32, I32, F, ctypes.c_int, P,
                                         ctypes.c_size_t, P, P]
    lib.gdn_conv1d_silu_fwd_pooled.argtypes = [P, P, I32, I32, I32, I32, P, P, P, SL, P, ctypes.c_int, P]
    lib.gdn_recurrent_step_fused_pooled.argtypes = [P, P, P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, F,
                                                    ctypes.c_int, P, P]
    lib.gdn_conv1d_silu_step_pooled.argtypes = [P, I32, I32, I32, P, P, P, P, I32, P, ctypes.c_int, P]
    lib.gdn_chunk_fwd_fused.argtypes = [P, P, P, ctypes.POINTER(FrontEnd), P, I32, P, P, P, SL, I32, I32, I32, I32,
                                        I32, F, ctypes.c_int, P, ctypes.c_size_t, P, P]
    lib.gdn_chunk_fwd_fused.restype = ctypes.c_int
    lib.gdn_chunk_fwd_dev_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, ctypes.c_int]
    lib.gdn_chunk_fwd_dev_workspace_size.restype = ctypes.c_size_t
    lib.gdn_chunk_fwd_dev.argtypes = [P, P, P, P, P, P, I32, P, P, P, I32, I32, I32, I32, I32, F, ctypes.c_int, P,
                                      ctypes.c_size_t, P, P]
    lib.gdn_chunk_fwd_dev.restype = ctypes.c_int
    lib.gdn_stream_copy.argtypes = [P, P, ctypes.c_size_t, P]
    lib.gdn_stream_copy.restype = ctypes.c_int
    lib.gdn_state_rows_zero.argtypes = [P, I32, ctypes.c_size_t, P, I32, P]
    lib.gdn_state_rows_copy.argtypes = [P, I32, ctypes.c_size_t, P, P, I32, P]
    for fn in ("gdn_chunk_fwd_pooled", "gdn_conv1d_silu_fwd_pooled", "gdn_recurrent_step_fused_pooled",
               "gdn_conv1d_silu_step_pooled", "gdn_state_rows_zero", "gdn_state_rows_copy"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_dev(name, t, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    # the library launches on the calling thread's current device
    if t.device.index != _torch().cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, not on the current device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _check_buf(name, t, dtype, shape):
    """A caller-supplied output buffer: on the current device, contiguous, of the
    given dtype and exactly the given shape (the kernels write every element of
    that shape, so a smaller buffer would be overrun)."""
    _check_dev(name, t, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _host_cu(cu_seqlens) -> "ctypes.Array":
    torch = _torch()
    if isinstance(cu_seqlens, torch.Tensor):
        if cu_seqlens.is_cuda:
            raise TypeError("cu_seqlens must be a host array (list, numpy or CPU tensor)")
        vals = [int(x) for x in cu_seqlens.tolist()]
    else:
        vals = [int(x) for x in cu_seqlens]
    return (ctypes.c_int32 * len(vals))(*vals)


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def workspace_layout(T: int, cu_seqlens, H_q: int, H_v: int, d_k: int, d_v: int, dtype) -> dict:
    """Byte offsets of the workspace regions (see gdn_workspace_layout in include/gdn.h)."""
    lib = load_library()
    cu = _host_cu(cu_seqlens)
    code = dtype if isinstance(dtype, int) else _dtype_code_from(dtype)
    lay = WorkspaceLayout()
    rc = lib.gdn_chunk_fwd_workspace_layout(T, len(cu) - 1, cu, H_q, H_v, d_k, d_v, code, ctypes.byref(lay))
    if rc != 0:
        raise GdnError(rc, "gdn_chunk_fwd_workspace_layout")
    return {f: getattr(lay, f) for f, _ in WorkspaceLayout._fields_}


def _dtype_code_from(dtype) -> int:
    torch = _torch()
    if dtype in (torch.bfloat16, "bf16"):
        return DTYPE_BF16
    if dtype in (torch.float32, "f32"):
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {dtype}")


def chunk_form(T: int, num_seqs: int, H_v: int, d: int, dtype) -> str:
    """Operand form the state scan of chunk_fwd takes for such a call: "W" (W and U)
    or "A" (A and the raw rows); gdn_chunk_fwd_form."""
    rc = load_library().gdn_chunk_fwd_form(T, num_seqs, H_v, d, _dtype_code_from(dtype))
    if rc < 0:
        raise GdnError(rc, "gdn_chunk_fwd_form")
    return "A" if rc else "W"


def workspace_size(T: int, cu_seqlens, H_q: int, H_v: int, d_k: int, d_v: int, dtype) -> int:
    """Workspace bytes of chunk_fwd (gdn_chunk_fwd_workspace_size); raises on invalid arguments."""
    workspace_layout(T, cu_seqlens, H_q, H_v, d_k, d_v, dtype)  # validates
    code = dtype if isinstance(dtype, int) else _dtype_code_from(dtype)
    return load_library().gdn_chunk_fwd_workspace_size(_host_cu(cu_seqlens), len(cu_seqlens) - 1, H_q, H_v, d_k,
                                                       d_v, code)


# ---------------------------------------------------------------------------
# operations
# ---------------------------------------------------------------------------

def chunk_fwd(q, k, v, g, beta, cu_seqlens: Sequence[int], initial_state=None, scale: Optional[float] = None,
              out=None, final_state=None, output_final_state: bool = True, workspace=None, stream=None,
              keep_A: bool = False, gate=None, keep_hx: bool = False, scan_ct: Optional[int] = None,
              keep_wu: bool = False, form: Optional[str] = None):
    """Chunk-wise GDN prefill over a packed batch (gdn_chunk_fwd; gdn_chunk_fwd_ex with options).

    q, k: [T, H_q, d_k]; v: [T, H_v, d_v] (bf16 or fp32, same dtype); g, beta:
    [T, H_v] fp32 (g = ln alpha per token); cu_seqlens: host int sequence [N+1];
    initial_state: fp32 [N, H_v, d_k, d_v] or None.  Returns (out, final_state)
    with final_state None when output_final_state is False.  ``workspace`` may
    be a preallocated uint8 device tensor of at least workspace_size() bytes;
    keep_A also writes the A intermediate into it (GDN_FWD_KEEP_A), keep_wu W
    and U (GDN_FWD_KEEP_WU), keep_hx the chunk-start states and U - W S
    (GDN_FWD_KEEP_HX).  ``gate`` =
    (z [T, H_v, d_v] in q's dtype, weight fp32 [d_v], eps) applies the gated
    RMSNorm read-out epilogue to out (gdn_chunk_fwd_ex).  ``scan_ct`` (1, 2 or
    4) fixes the state scan's column tiles a workgroup (GDN_FWD_SCAN_CT*)
    instead of the host cost model's choice; ``form`` ("W" or "A") the operands
    the state scan reads (GDN_FWD_FORM_*) instead of the library's choice.
    """
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(q)
    if scan_ct is not None and scan_ct not in FWD_SCAN_CT:
        raise ValueError("scan_ct must be 1, 2 or 4")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    _check_dev("g", g, torch.float32)
    _check_dev("beta", beta, torch.float32)
    T, H_q, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, H_v) or beta.shape != (T, H_v):
        raise ValueError("inconsistent q/k/v/g/beta shapes")
    cu = _host_cu(cu_seqlens)
    N = len(cu) - 1
    if initial_state is not None:
        _check_dev("initial_state", initial_state, torch.float32)
        if tuple(initial_state.shape) != (N, H_v, d_k, d_v):
            raise ValueError("initial_state must be [N, H_v, d_k, d_v]")
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if out is None:
        out = torch.empty((T, H_v, d_v), dtype=q.dtype, device=q.device)
    else:
        _check_buf("out", out, q.dtype, (T, H_v, d_v))
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H_v, d_k, d_v), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _check_buf("final_state", final_state, torch.float32, (N, H_v, d_k, d_v))
    ws_bytes = lib.gdn_chunk_fwd_workspace_size(cu, N, H_q, H_v, d_k, d_v, dt)
    if ws_bytes == 0 and N > 0 and T > 0:
        lay = WorkspaceLayout()
        rc = lib.gdn_chunk_fwd_workspace_layout(T, N, cu, H_q, H_v, d_k, d_v, dt, ctypes.byref(lay))
        raise GdnError(rc, "gdn_chunk_fwd_workspace_size")
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    else:
        _check_dev("workspace", workspace)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu, N, _ptr(initial_state), _ptr(out),
            _ptr(final_state), T, H_q, H_v, d_k, d_v, float(scale), dt, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    gptr, _keep = _gate_arg(gate, q.dtype, T, H_v, d_v)
    if form is not None and form not in FWD_FORM:
        raise ValueError('form must be "W" or "A"')
    flags = ((FWD_KEEP_A if keep_A else 0) | (FWD_KEEP_HX if keep_hx else 0) | (FWD_KEEP_WU if keep_wu else 0) |
             FWD_SCAN_CT.get(scan_ct, 0) | FWD_FORM.get(form, 0))
    if flags or gate is not None:
        rc, name = lib.gdn_chunk_fwd_ex(*args, flags, gptr, None), "gdn_chunk_fwd_ex"
    else:
        rc, name = lib.gdn_chunk_fwd(*args), "gdn_chunk_fwd"
    if rc != 0:
        raise GdnError(rc, name)
    return out, final_state


def chunk_fwd_scratch(q, k, v, g, beta, cu_seqlens: Sequence[int], initial_state=None,
                      scale: Optional[float] = None, out=None, final_state=None, stream=None):
    """chunk_fwd whose workspace is the library's static device array
    (gdn_chunk_fwd_scratch): the C call allocates nothing.  ``out`` and
    ``final_state`` must be preallocated by callers that cannot allocate (this
    wrapper allocates them only when they are None).  Batches needing more than
    SCRATCH_BYTES of workspace are refused (GdnError, workspace).  Calls that
    overlap in time on one GPU share the array and race."""
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    _check_dev("g", g, torch.float32)
    _check_dev("beta", beta, torch.float32)
    T, H_q, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, H_v) or beta.shape != (T, H_v):
        raise ValueError("inconsistent q/k/v/g/beta shapes")
    cu = _host_cu(cu_seqlens)
    N = len(cu) - 1
    if initial_state is not None:
        _check_buf("initial_state", initial_state, torch.float32, (N, H_v, d_k, d_v))
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if out is None:
        out = torch.empty((T, H_v, d_v), dtype=q.dtype, device=q.device)
    else:
        _check_buf("out", out, q.dtype, (T, H_v, d_v))
    if final_state is None:
        final_state = torch.empty((N, H_v, d_k, d_v), dtype=torch.float32, device=q.device)
    else:
        _check_buf("final_state", final_state, torch.float32, (N, H_v, d_k, d_v))
    rc = lib.gdn_chunk_fwd_scratch(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu, N, _ptr(initial_state),
                                   _ptr(out), _ptr(final_state), T, H_q, H_v, d_k, d_v, float(scale), dt,
                                   _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_chunk_fwd_scratch")
    return out, final_state


def recurrent_step(q, k, v, g, beta, state, scale: Optional[float] = None, out=None, stream=None):
    """One recurrent decode step (gdn_recurrent_step); ``state`` is updated in place.

    q, k: [N, H_q, d_k]; v: [N, H_v, d_v] (bf16 or fp32); g, beta: [N, H_v] fp32;
    state: fp32 [N, H_v, d_k, d_v].  Returns out [N, H_v, d_v] in q's dtype.
    """
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    _check_dev("g", g, torch.float32)
    _check_dev("beta", beta, torch.float32)
    _check_dev("state", state, torch.float32)
    N, H_q, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != N or g.shape != (N, H_v) or beta.shape != (N, H_v) or \
            tuple(state.shape) != (N, H_v, d_k, d_v):
        raise ValueError("inconsistent decode shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if out is None:
        out = torch.empty((N, H_v, d_v), dtype=q.dtype, device=q.device)
    else:
        _check_buf("out", out, q.dtype, (N, H_v, d_v))
    rc = lib.gdn_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(out), N, H_q, H_v,
                                d_k, d_v, float(scale), dt, _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_recurrent_step")
    return out


def recurrent_step_fused(q, k, v, a, b, A_log, dt_bias, state, scale: Optional[float] = None, out=None,
                         stream=None, gate=None):
    """One decode step from the raw inputs (gdn_recurrent_step_fused): q/k L2 norm,
    gate from a, A_log, dt_bias, beta from b, then the state update; ``state`` is
    updated in place.

    q, k: [N, H_q, d_k] (not normalised); v: [N, H_v, d_v]; a, b: [N, H_v] (q's
    dtype); A_log, dt_bias: fp32 [H_v]; state: fp32 [N, H_v, d_k, d_v].  Returns
    out [N, H_v, d_v] in q's dtype.  scale defaults to 1/sqrt(d_k).  ``gate`` =
    (z [N, H_v, d_v], weight fp32 [d_v], eps) adds the gated RMSNorm read-out.
    """
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("a", a), ("b", b)):
        _check_dev(name, t, q.dtype)
    _check_dev("A_log", A_log, torch.float32)
    _check_dev("dt_bias", dt_bias, torch.float32)
    _check_dev("state", state, torch.float32)
    N, H_q, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != N or a.shape != (N, H_v) or b.shape != (N, H_v) or \
            A_log.shape != (H_v,) or dt_bias.shape != (H_v,) or tuple(state.shape) != (N, H_v, d_k, d_v):
        raise ValueError("inconsistent decode shapes")
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if out is None:
        out = torch.empty((N, H_v, d_v), dtype=q.dtype, device=q.device)
    else:
        _check_buf("out", out, q.dtype, (N, H_v, d_v))
    gptr, _keep = _gate_arg(gate, q.dtype, N, H_v, d_v)
    rc = lib.gdn_recurrent_step_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                                      _ptr(state), _ptr(out), N, H_q, H_v, d_k, d_v, float(scale), dt, gptr,
                                      _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_recurrent_step_fused")
    return out


def conv1d_silu(x, cu_seqlens: Sequence[int], weight, bias=None, initial_state=None, final_state=None,
                output_final_state: bool = True, out=None, stream=None):
    """Causal depthwise conv1d + SiLU over a packed batch (gdn_conv1d_silu_fwd).

    x: [T, C] (bf16 or fp32); weight: fp32 [C, K] (oldest tap first); bias: fp32
    [C] or None; initial_state: [N, K-1, C] in x's dtype or None.  Returns
    (out [T, C], final_state [N, K-1, C] or None).
    """
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(x)
    _check_dev("x", x, x.dtype)
    _check_dev("weight", weight, torch.float32)
    T, C = x.shape
    K = weight.shape[1]
    if tuple(weight.shape) != (C, K):
        raise ValueError("weight must be [C, K]")
    if bias is not None:
        _check_dev("bias", bias, torch.float32)
    cu = _host_cu(cu_seqlens)
    N = len(cu) - 1
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None:
            _check_dev(name, t, x.dtype)
            if tuple(t.shape) != (N, K - 1, C):
                raise ValueError(f"{name} must be [N, K-1, C]")
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_buf("out", out, x.dtype, tuple(x.shape))
    if final_state is None and output_final_state:
        final_state = torch.empty((N, K - 1, C), dtype=x.dtype, device=x.device)
    rc = lib.gdn_conv1d_silu_fwd(_ptr(x), cu, N, T, C, K, _ptr(weight), _ptr(bias), _ptr(initial_state), _ptr(out),
                                 _ptr(final_state), dt, _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_conv1d_silu_fwd")
    return out, final_state


def conv1d_silu_step(x, weight, bias, state, out=None, stream=None):
    """One decode token of the convolution (gdn_conv1d_silu_step): x [N, C];
    state [N, K-1, C] updated in place.  Returns out [N, C]."""
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(x)
    _check_dev("x", x, x.dtype)
    _check_dev("weight", weight, torch.float32)
    _check_dev("state", state, x.dtype)
    N, C = x.shape
    K = weight.shape[1]
    if tuple(state.shape) != (N, K - 1, C) or tuple(weight.shape) != (C, K):
        raise ValueError("inconsistent conv step shapes")
    if bias is not None:
        _check_dev("bias", bias, torch.float32)
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_buf("out", out, x.dtype, tuple(x.shape))
    rc = lib.gdn_conv1d_silu_step(_ptr(x), N, C, K, _ptr(weight), _ptr(bias), _ptr(state), _ptr(out), dt,
                                  _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_conv1d_silu_step")
    return out


# ---------------------------------------------------------------------------
# state pools (serving): rows addressed by slot
# ---------------------------------------------------------------------------

def chunk_fwd_pooled(q, k, v, g, beta, cu_seqlens: Sequence[int], state_pool, slots, has_initial=None,
                     scale: Optional[float] = None, out=None, workspace=None, stream=None, gate=None):
    """Chunk-wise prefill reading and writing states in a pool (gdn_chunk_fwd_pooled).

    state_pool: fp32 [P, H_v, d_k, d_v]; slots: host ints [N], the pool row of
    each sequence (-1: starts from zeros, final state not kept); has_initial:
    host bools [N] or None (all True) — False starts that sequence from zeros
    although it has a row (a request without a cached prefix).  Returns out.
    """
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    _check_dev("g", g, torch.float32)
    _check_dev("beta", beta, torch.float32)
    _check_dev("state_pool", state_pool, torch.float32)
    T, H_q, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, H_v) or beta.shape != (T, H_v):
        raise ValueError("inconsistent q/k/v/g/beta shapes")
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H_v, d_k, d_v):
        raise ValueError("state_pool must be [P, H_v, d_k, d_v]")
    cu = _host_cu(cu_seqlens)
    N = len(cu) - 1
    st, _keep_slots = _slots_arg(slots, has_initial, state_pool.shape[0], N)
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if out is None:
        out = torch.empty((T, H_v, d_v), dtype=q.dtype, device=q.device)
    else:
        _check_buf("out", out, q.dtype, (T, H_v, d_v))
    ws_bytes = lib.gdn_chunk_fwd_workspace_size(cu, N, H_q, H_v, d_k, d_v, dt)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    else:
        _check_dev("workspace", workspace)
    gptr, _keep = _gate_arg(gate, q.dtype, T, H_v, d_v)
    rc = lib.gdn_chunk_fwd_pooled(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu, N, _ptr(state_pool),
                                  ctypes.byref(st), _ptr(out), T, H_q, H_v, d_k, d_v, float(scale), dt,
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), gptr,
                                  _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_chunk_fwd_pooled")
    return out


def chunk_fwd_fused(q, k, v, a, b, A_log, dt_bias, cu_seqlens: Sequence[int], initial_state=None,
                    scale: Optional[float] = None, out=None, final_state=None, output_final_state: bool = True,
                    workspace=None, stream=None, gate=None, slots=None, has_initial=None):
    """Chunk-wise prefill from the raw inputs (gdn_chunk_fwd_fused): q, k are
    L2-normalised and g, beta formed from a, b, A_log, dt_bias inside the kernels.

    q, k: [T, H_q, d_k] (not normalised); v: [T, H_v, d_v]; a, b: [T, H_v] in q's
    dtype; A_log, dt_bias: fp32 [H_v].  Without ``slots``: initial_state fp32
    [N, H_v, d_k, d_v] or None, returns (out, final_state) as chunk_fwd.  With
    ``slots`` (host ints [N]) and ``has_initial``: ``initial_state`` is a state
    pool [P, H_v, d_k, d_v] read and written by slot; returns (out, None).
    ``gate`` as for chunk_fwd.
    """
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("a", a), ("b", b)):
        _check_dev(name, t, q.dtype)
    _check_dev("A_log", A_log, torch.float32)
    _check_dev("dt_bias", dt_bias, torch.float32)
    T, H_q, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != T or a.shape != (T, H_v) or b.shape != (T, H_v) or \
            A_log.shape != (H_v,) or dt_bias.shape != (H_v,):
        raise ValueError("inconsistent q/k/v/a/b/A_log/dt_bias shapes")
    cu = _host_cu(cu_seqlens)
    N = len(cu) - 1
    st, keep_slots = None, None
    if slots is not None:
        if initial_state is None:
            raise ValueError("with slots, initial_state is the state pool")
        _check_dev("state pool", initial_state, torch.float32)
        if initial_state.dim() != 4 or tuple(initial_state.shape[1:]) != (H_v, d_k, d_v):
            raise ValueError("state pool must be [P, H_v, d_k, d_v]")
        st, keep_slots = _slots_arg(slots, has_initial, initial_state.shape[0], N)
        final_state = None
    else:
        if initial_state is not None:
            _check_dev("initial_state", initial_state, torch.float32)
            if tuple(initial_state.shape) != (N, H_v, d_k, d_v):
                raise ValueError("initial_state must be [N, H_v, d_k, d_v]")
        if final_state is None and output_final_state:
            final_state = torch.empty((N, H_v, d_k, d_v), dtype=torch.float32, device=q.device)
        elif final_state is not None:
            _check_buf("final_state", final_state, torch.float32, (N, H_v, d_k, d_v))
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if out is None:
        out = torch.empty((T, H_v, d_v), dtype=q.dtype, device=q.device)
    else:
        _check_buf("out", out, q.dtype, (T, H_v, d_v))
    ws_bytes = lib.gdn_chunk_fwd_workspace_size(cu, N, H_q, H_v, d_k, d_v, dt)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    else:
        _check_dev("workspace", workspace)
    fe = FrontEnd(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias))
    gptr, _keep = _gate_arg(gate, q.dtype, T, H_v, d_v)
    rc = lib.gdn_chunk_fwd_fused(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(fe), cu, N, _ptr(initial_state), _ptr(out),
                                 _ptr(final_state), ctypes.byref(st) if st is not None else None, T, H_q, H_v, d_k,
                                 d_v, float(scale), dt, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 gptr, _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_chunk_fwd_fused")
    return out, final_state


def chunk_fwd_dev(q, k, v, g, beta, cu_seqlens_dev, initial_state=None, scale: Optional[float] = None, out=None,
                  final_state=None, output_final_state: bool = True, workspace=None, stream=None, gate=None):
    """gdn_chunk_fwd with cu_seqlens in device memory (gdn_chunk_fwd_dev): the
    call depends on T and the number of sequences only, so it can be captured
    in a graph and replayed with new boundaries.  cu_seqlens_dev: device int32
    [N+1].  Other arguments and results as chunk_fwd (workspace sized by
    dev_workspace_size)."""
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_dev(name, t, q.dtype)
    _check_dev("g", g, torch.float32)
    _check_dev("beta", beta, torch.float32)
    _check_dev("cu_seqlens_dev", cu_seqlens_dev, torch.int32)
    T, H_q, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, H_v) or beta.shape != (T, H_v) or \
            cu_seqlens_dev.dim() != 1:
        raise ValueError("inconsistent q/k/v/g/beta/cu_seqlens shapes")
    N = cu_seqlens_dev.numel() - 1
    if initial_state is not None:
        _check_dev("initial_state", initial_state, torch.float32)
        if tuple(initial_state.shape) != (N, H_v, d_k, d_v):
            raise ValueError("initial_state must be [N, H_v, d_k, d_v]")
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if out is None:
        out = torch.empty((T, H_v, d_v), dtype=q.dtype, device=q.device)
    else:
        _check_buf("out", out, q.dtype, (T, H_v, d_v))
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H_v, d_k, d_v), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _check_buf("final_state", final_state, torch.float32, (N, H_v, d_k, d_v))
    if workspace is None:
        workspace = torch.empty(max(dev_workspace_size(T, N, H_q, H_v, d_k, d_v, q.dtype), 1), dtype=torch.uint8,
                                device=q.device)
    else:
        _check_dev("workspace", workspace)
    gptr, _keep = _gate_arg(gate, q.dtype, T, H_v, d_v)
    rc = lib.gdn_chunk_fwd_dev(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens_dev), N,
                               _ptr(initial_state), _ptr(out), _ptr(final_state), T, H_q, H_v, d_k, d_v, float(scale),
                               dt, _ptr(workspace), workspace.numel() * workspace.element_size(), gptr,
                               _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_chunk_fwd_dev")
    return out, final_state


def dev_workspace_size(T: int, num_seqs: int, H_q: int, H_v: int, d_k: int, d_v: int, dtype) -> int:
    """Workspace bytes of chunk_fwd_dev (gdn_chunk_fwd_dev_workspace_size)."""
    lib = load_library()
    code = dtype if isinstance(dtype, int) else _dtype_code_from(dtype)
    return lib.gdn_chunk_fwd_dev_workspace_size(T, num_seqs, H_q, H_v, d_k, d_v, code)


def conv1d_silu_pooled(x, cu_seqlens: Sequence[int], weight, bias, state_pool, slots, has_initial=None, out=None,
                       stream=None):
    """Packed conv1d + SiLU reading and writing histories in a pool
    (gdn_conv1d_silu_fwd_pooled): state_pool [P, K-1, C] in x's dtype; slots and
    has_initial as for chunk_fwd_pooled.  Returns out [T, C]."""
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(x)
    _check_dev("x", x, x.dtype)
    _check_dev("weight", weight, torch.float32)
    _check_dev("state_pool", state_pool, x.dtype)
    T, C = x.shape
    K = weight.shape[1]
    if tuple(weight.shape) != (C, K) or state_pool.dim() != 3 or tuple(state_pool.shape[1:]) != (K - 1, C):
        raise ValueError("weight must be [C, K] and state_pool [P, K-1, C]")
    if bias is not None:
        _check_dev("bias", bias, torch.float32)
    cu = _host_cu(cu_seqlens)
    N = len(cu) - 1
    st, _keep_slots = _slots_arg(slots, has_initial, state_pool.shape[0], N)
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_buf("out", out, x.dtype, tuple(x.shape))
    rc = lib.gdn_conv1d_silu_fwd_pooled(_ptr(x), cu, N, T, C, K, _ptr(weight), _ptr(bias), _ptr(state_pool),
                                        ctypes.byref(st), _ptr(out), dt, _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_conv1d_silu_fwd_pooled")
    return out


def recurrent_step_fused_pooled(q, k, v, a, b, A_log, dt_bias, state_pool, slot, scale: Optional[float] = None,
                                out=None, stream=None, gate=None):
    """Fused decode step over a state pool (gdn_recurrent_step_fused_pooled).

    state_pool: fp32 [P, H_v, d_k, d_v], updated in place; slot: device int32
    [N], the pool row of each sequence; a slot outside [0, P) is padding (zero
    output row, no pool access).  Other arguments as recurrent_step_fused.
    """
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("a", a), ("b", b)):
        _check_dev(name, t, q.dtype)
    _check_dev("A_log", A_log, torch.float32)
    _check_dev("dt_bias", dt_bias, torch.float32)
    _check_dev("state_pool", state_pool, torch.float32)
    N, H_q, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != N or a.shape != (N, H_v) or b.shape != (N, H_v) or \
            A_log.shape != (H_v,) or dt_bias.shape != (H_v,) or state_pool.dim() != 4 or \
            tuple(state_pool.shape[1:]) != (H_v, d_k, d_v):
        raise ValueError("inconsistent decode shapes")
    _check_slot_dev(slot, N)
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if out is None:
        out = torch.empty((N, H_v, d_v), dtype=q.dtype, device=q.device)
    else:
        _check_buf("out", out, q.dtype, (N, H_v, d_v))
    gptr, _keep = _gate_arg(gate, q.dtype, N, H_v, d_v)
    rc = lib.gdn_recurrent_step_fused_pooled(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
                                             _ptr(dt_bias), _ptr(state_pool), _ptr(slot), state_pool.shape[0],
                                             _ptr(out), N, H_q, H_v, d_k, d_v, float(scale), dt, gptr,
                                             _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_recurrent_step_fused_pooled")
    return out


def conv1d_silu_step_pooled(x, weight, bias, state_pool, slot, out=None, stream=None):
    """One decode token of the convolution over a history pool
    (gdn_conv1d_silu_step_pooled): x [N, C]; state_pool [P, K-1, C] updated in
    place; slot device int32 [N] (outside [0, P): padding).  Returns out [N, C]."""
    torch = _torch()
    lib = load_library()
    dt = _dtype_code(x)
    _check_dev("x", x, x.dtype)
    _check_dev("weight", weight, torch.float32)
    _check_dev("state_pool", state_pool, x.dtype)
    N, C = x.shape
    K = weight.shape[1]
    if tuple(weight.shape) != (C, K) or state_pool.dim() != 3 or tuple(state_pool.shape[1:]) != (K - 1, C):
        raise ValueError("inconsistent conv step shapes")
    if bias is not None:
        _check_dev("bias", bias, torch.float32)
    _check_slot_dev(slot, N)
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_buf("out", out, x.dtype, tuple(x.shape))
    rc = lib.gdn_conv1d_silu_step_pooled(_ptr(x), N, C, K, _ptr(weight), _ptr(bias), _ptr(state_pool), _ptr(slot),
                                         state_pool.shape[0], _ptr(out), dt, _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_conv1d_silu_step_pooled")
    return out


def _pool_rows(pool, src, dst, what, stream):
    torch = _torch()
    lib = load_library()
    _check_dev("pool", pool)
    _check_dev("rows", dst, torch.int32)
    if src is not None:
        _check_dev("src rows", src, torch.int32)
        if src.shape != dst.shape:
            raise ValueError("src and dst rows must have the same length")
    if dst.dim() != 1:
        raise ValueError("rows must be 1-D")
    P = pool.shape[0]
    row_bytes = pool[0].numel() * pool.element_size() if P > 0 else 0
    if P == 0:
        return
    if src is None:
        rc = lib.gdn_state_rows_zero(_ptr(pool), P, row_bytes, _ptr(dst), dst.numel(), _stream_ptr(stream))
    else:
        rc = lib.gdn_state_rows_copy(_ptr(pool), P, row_bytes, _ptr(src), _ptr(dst), dst.numel(),
                                     _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, what)


def stream_copy(src, dst, stream=None):
    """Measurement aid (gdn_stream_copy): dst := src as a plain streaming copy,
    for the achievable-HBM figure.  Contiguous device tensors of equal byte size
    (a multiple of 16)."""
    lib = load_library()
    _check_dev("src", src)
    _check_dev("dst", dst)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    rc = lib.gdn_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream_ptr(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_stream_copy")


def state_rows_zero(pool, rows, stream=None):
    """Reset pool rows to zero (gdn_state_rows_zero): pool [P, ...] (state or
    conv history), rows device int32 [n]; rows outside [0, P) are skipped."""
    _pool_rows(pool, None, rows, "gdn_state_rows_zero", stream)


def state_rows_copy(pool, src_rows, dst_rows, stream=None):
    """Copy pool rows (gdn_state_rows_copy): row dst_rows[i] := row src_rows[i]
    (e.g. cloning a state for a speculative branch); pairs with a row outside
    [0, P) are skipped."""
    _pool_rows(pool, src_rows, dst_rows, "gdn_state_rows_copy", stream)
