"""C-ABI tests that need no GPU: the library loads, exports every function
include/gdn.h declares, computes workspace layouts on the host, and rejects bad
arguments before touching the device (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_state_chunk_amd as gdn

    if not os.path.exists(gdn.lib_path()):
        from gated_deltanet_state_chunk_amd import build

        build.build()
    gdn.load_library()
    return gdn


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(gdn):
    names = _declared()
    assert {"gdn_chunk_fwd", "gdn_recurrent_step", "gdn_chunk_fwd_workspace_size", "gdn_strerror"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.lib_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (gdn_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(gdn.lib_path())
    for n in names:
        getattr(lib, n)


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "gdn.h"\nint main(void){ return GDN_OK; }\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(tmp_path / "t")], check=True)


def test_status_strings(gdn):
    lib = gdn.load_library()
    assert lib.gdn_status_string(0) == b"ok"
    assert lib.gdn_status_string(-3).startswith(b"workspace")
    assert lib.gdn_version().startswith(b"0.")
    assert lib.gdn_last_hip_error() == b""
    # gdn_strerror: the same texts while no HIP error has been recorded
    for status in (0, -1, -2, -3, -4, -99, 5):
        assert lib.gdn_strerror(status) == lib.gdn_status_string(status)


def test_contract_names_compile(tmp_path):
    # The names and signatures a caller coded to the documented boundary uses
    # (status and dtype enums, hipStream_t, the workspace query on cu_seqlens).
    src = tmp_path / "c.c"
    src.write_text(r'''
#include "gdn.h"
int main(void) {
    const int32_t cu[3] = {0, 100, 164};
    size_t ws = gdn_chunk_fwd_workspace_size(cu, 2, 16, 32, 128, 128, GDN_BF16);
    hipStream_t s = 0;
    int (*fwd)(const void *, const void *, const void *, const float *, const float *, const int32_t *, int32_t,
               const float *, void *, float *, int32_t, int32_t, int32_t, int32_t, int32_t, float, gdn_dtype,
               void *, size_t, hipStream_t) = gdn_chunk_fwd;
    int (*step)(const void *, const void *, const void *, const float *, const float *, float *, void *, int32_t,
                int32_t, int32_t, int32_t, int32_t, float, gdn_dtype, hipStream_t) = gdn_recurrent_step;
    const char *(*err)(int) = gdn_strerror;
    int codes[] = {GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EWORKSPACE, GDN_ELAUNCH, GDN_F32};
    return (ws == 0) + (s != 0) + (fwd == 0) + (step == 0) + (err == 0) + codes[0];
}
''')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-c", str(src), "-o",
                    str(tmp_path / "c.o")], check=True)


def test_workspace_size_contract(gdn):
    lib = gdn.load_library()
    assert lib.gdn_chunk_fwd_workspace_size(_cu([0, 100, 164]), 2, 16, 32, 128, 128, 1) == \
        gdn.workspace_layout(164, [0, 100, 164], 16, 32, 128, 128, "bf16")["total_bytes"]
    assert lib.gdn_chunk_fwd_workspace_size(None, 0, 16, 32, 128, 128, 1) == 0  # empty batch: nothing needed
    assert lib.gdn_chunk_fwd_workspace_size(None, 2, 16, 32, 128, 128, 1) == 0  # missing cu_seqlens
    assert lib.gdn_chunk_fwd_workspace_size(_cu([0, 5, 3]), 2, 16, 32, 128, 128, 1) == 0


def _cu(vals):
    return (ctypes.c_int32 * len(vals))(*vals)


def test_workspace_layout(gdn):
    lay = gdn.workspace_layout(4096, [0, 4096], 16, 32, 128, 128, "bf16")
    assert lay["n_chunks"] == 64
    offs = [lay[k] for k in ("off_gates", "off_A", "off_W", "off_U", "off_Kc", "off_Ht", "off_Xt", "off_P",
                             "off_Qc", "off_Af", "total_bytes")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    chv = 64 * 32
    assert lay["off_A"] - lay["off_gates"] == chv * 4 * 64 * 4      # gc, kf, beta, beta gamma (fp32)
    assert lay["off_W"] - lay["off_A"] == chv * 64 * 64 * 2
    assert lay["off_Kc"] - lay["off_U"] == chv * 128 * 64 * 2
    assert lay["total_bytes"] - lay["off_Af"] == chv * 6 * 64 * 8 * 2  # A's six fragments (binary16)
    assert lay["off_Ht"] - lay["off_Kc"] == 64 * 16 * 64 * 128 * 2  # chunks x key heads x rows x d_k
    assert lay["off_Xt"] - lay["off_Ht"] == chv * 128 * 128 * 2
    assert lay["off_Qc"] - lay["off_P"] == chv * 6 * 1024            # P: six 1 KiB fragments (bf16)
    assert lay["off_Af"] - lay["off_Qc"] == 64 * 16 * 64 * 128 * 2  # Qc: as Kc
    # chunks are counted per sequence: ceil(100/64) + 0 + ceil(1/64) + ceil(128/64)
    lay2 = gdn.workspace_layout(229, [0, 100, 100, 101, 229], 2, 4, 64, 64, "f32")
    assert lay2["n_chunks"] == 2 + 0 + 1 + 2
    assert lay2["off_Af"] == lay2["off_P"] == lay2["off_Qc"]          # no P or Qc region for fp32
    assert gdn.workspace_size(0, [0], 2, 4, 64, 64, "f32") >= 0


@pytest.mark.parametrize("args,status", [
    # (T, cu, H_q, H_v, d_k, d_v, dtype) -> status
    ((10, [0, 5, 10], 2, 4, 128, 128, 1), 0),
    ((10, [0, 5, 9], 2, 4, 128, 128, 1), -1),   # cu[N] != T
    ((10, [1, 5, 10], 2, 4, 128, 128, 1), -1),  # cu[0] != 0
    ((10, [0, 6, 5, 10], 2, 4, 128, 128, 1), -1),  # decreasing
    ((10, [0, 10], 3, 4, 128, 128, 1), -2),     # H_v % H_q
    ((10, [0, 10], 2, 4, 128, 64, 1), -2),      # d_k != d_v
    ((10, [0, 10], 2, 4, 96, 96, 1), -2),       # unsupported d
    ((10, [0, 10], 2, 4, 128, 128, 7), -2),     # dtype
    ((10, [0, 10], 0, 4, 128, 128, 1), -1),     # H_q = 0
])
def test_layout_validation(gdn, args, status):
    lib = gdn.load_library()
    T, cu, H_q, H_v, dk, dv, dt = args
    lay = gdn.WorkspaceLayout()
    rc = lib.gdn_chunk_fwd_workspace_layout(T, len(cu) - 1, _cu(cu), H_q, H_v, dk, dv, dt, ctypes.byref(lay))
    assert rc == status
    # the size query takes T from cu_seqlens itself, so a cu[N] != T batch is a
    # valid batch of cu[N] tokens there
    size = lib.gdn_chunk_fwd_workspace_size(_cu(cu), len(cu) - 1, H_q, H_v, dk, dv, dt)
    assert (size > 0) == (status == 0 or cu[-1] != T)
    if status == 0:
        assert size == lay.total_bytes


def _fake(n=1):
    # 256-byte aligned host addresses that are never dereferenced: every call
    # below fails validation before the library touches memory or the device.
    buf = np.zeros(64 * n + 64, dtype=np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    return buf, base


def test_chunk_fwd_rejects_before_any_device_work(gdn):
    lib = gdn.load_library()
    keep, p = _fake()
    cu = _cu([0, 10])
    good = dict(q=p, k=p, v=p, g=p, beta=p, cu=cu, N=1, s0=None, out=p, fin=p, T=10, H_q=2, H_v=4, dk=128, dv=128,
                scale=0.1, dt=1, ws=p, wsb=1 << 40, stream=None)

    def call(**kw):
        a = dict(good, **kw)
        return lib.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"], a["s0"], a["out"],
                                 a["fin"], a["T"], a["H_q"], a["H_v"], a["dk"], a["dv"], a["scale"], a["dt"],
                                 a["ws"], a["wsb"], a["stream"])

    assert call(q=None) == -1
    assert call(out=None) == -1
    assert call(q=p + 8) == -2                 # misaligned
    assert call(H_q=3) == -2
    assert call(dk=64) == -2
    assert call(scale=float("nan")) == -1
    assert call(ws=None) == -3
    assert call(wsb=16) == -3
    assert call(cu=_cu([0, 11])) == -1
    # empty batch is a no-op that succeeds without launching anything
    assert call(N=0, T=0, cu=_cu([0])) == 0

    def call_ex(flags, **kw):
        a = dict(good, **kw)
        return lib.gdn_chunk_fwd_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"], a["s0"], a["out"],
                                    a["fin"], a["T"], a["H_q"], a["H_v"], a["dk"], a["dv"], a["scale"], a["dt"],
                                    a["ws"], a["wsb"], a["stream"], flags, None, None)

    assert call_ex(256) == -1                  # unknown flag bit
    assert call_ex(gdn.FWD_FORM["W"] | gdn.FWD_FORM["A"]) == -1  # both forms
    assert call_ex(gdn.FWD_FORM["A"], N=0, T=0, cu=_cu([0])) == 0
    assert call_ex(gdn.FWD_KEEP_WU, q=None) == -1
    assert call_ex(gdn.FWD_KEEP_WU, N=0, T=0, cu=_cu([0])) == 0
    assert call_ex(gdn.FWD_SCAN_CT[1] | gdn.FWD_SCAN_CT[2]) == -1  # two tile widths
    assert call_ex(gdn.FWD_SCAN_CT[4], q=None) == -1
    assert call_ex(gdn.FWD_SCAN_CT[2], N=0, T=0, cu=_cu([0])) == 0

    def call_gate(z, w, eps):
        g = gdn.OutputGate(z, w, eps)
        a = good
        return lib.gdn_chunk_fwd_ex(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"], a["s0"], a["out"],
                                    a["fin"], a["T"], a["H_q"], a["H_v"], a["dk"], a["dv"], a["scale"], a["dt"],
                                    a["ws"], a["wsb"], a["stream"], 0, ctypes.byref(g), None)

    assert call_gate(p, p, 0.0) == -1          # eps must be > 0
    assert call_gate(p, p, float("nan")) == -1
    assert call_gate(None, p, 1e-6) == -1      # z missing
    assert call_gate(p + 8, p, 1e-6) == -2     # z misaligned
    assert call_ex(gdn.FWD_KEEP_A, q=None) == -1
    assert call_ex(gdn.FWD_KEEP_A, N=0, T=0, cu=_cu([0])) == 0


def test_recurrent_step_rejects_before_any_device_work(gdn):
    lib = gdn.load_library()
    keep, p = _fake()

    def call(**kw):
        a = dict(q=p, k=p, v=p, g=p, beta=p, st=p, out=p, N=4, H_q=2, H_v=4, dk=128, dv=128, scale=0.1, dt=1)
        a.update(kw)
        return lib.gdn_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["st"], a["out"], a["N"],
                                      a["H_q"], a["H_v"], a["dk"], a["dv"], a["scale"], a["dt"], None)

    assert call(st=None) == -1
    assert call(N=-1) == -1
    assert call(H_q=3) == -2
    assert call(dk=32, dv=32) == -2
    assert call(out=p + 4) == -2
    assert call(N=0) == 0


def test_recurrent_step_fused_rejects_before_any_device_work(gdn):
    lib = gdn.load_library()
    keep, p = _fake()
    good = dict(q=p, k=p, v=p, a=p, b=p, A=p, dtb=p, st=p, out=p, N=4, H_q=2, H_v=4, dk=128, dv=128, scale=0.1,
                dt=1, stream=None)

    def call(**kw):
        x = dict(good, **kw)
        return lib.gdn_recurrent_step_fused(x["q"], x["k"], x["v"], x["a"], x["b"], x["A"], x["dtb"], x["st"],
                                            x["out"], x["N"], x["H_q"], x["H_v"], x["dk"], x["dv"], x["scale"],
                                            x["dt"], None, x["stream"])

    assert call(a=None) == -1
    assert call(dtb=None) == -1
    assert call(q=p + 8) == -2                 # misaligned tensor
    assert call(a=p + 1) == -2                 # bf16 scalar off its 2-byte alignment
    assert call(A=p + 2) == -2                 # fp32 parameter off its 4-byte alignment
    assert call(H_q=3) == -2
    assert call(N=-1) == -1
    assert call(scale=float("nan")) == -1
    assert call(N=0) == 0


def test_conv_entry_points_reject_before_any_device_work(gdn):
    lib = gdn.load_library()
    keep, p = _fake()
    cu = _cu([0, 10])

    def fwd(**kw):
        a = dict(x=p, cu=cu, N=1, T=10, C=64, K=4, w=p, b=None, s0=None, out=p, fin=None, dt=1)
        a.update(kw)
        return lib.gdn_conv1d_silu_fwd(a["x"], a["cu"], a["N"], a["T"], a["C"], a["K"], a["w"], a["b"], a["s0"],
                                       a["out"], a["fin"], a["dt"], None)

    assert fwd(K=5) == -2 and fwd(K=1) == -2   # taps outside 2..4
    assert fwd(C=60) == -2                     # not whole 16-byte channel groups (bf16)
    assert fwd(w=None) == -1
    assert fwd(x=p + 8) == -2
    assert fwd(cu=_cu([0, 11])) == -1
    assert fwd(N=0, T=0, cu=_cu([0])) == 0

    def step(**kw):
        a = dict(x=p, N=3, C=64, K=4, w=p, b=None, st=p, out=p, dt=0)
        a.update(kw)
        return lib.gdn_conv1d_silu_step(a["x"], a["N"], a["C"], a["K"], a["w"], a["b"], a["st"], a["out"],
                                        a["dt"], None)

    assert step(st=None) == -1
    assert step(C=62) == -2
    assert step(w=p + 4) == -2                 # weights are read as 16-byte vectors
    assert step(N=0) == 0


def test_pooled_entry_points_reject_before_any_device_work(gdn):
    lib = gdn.load_library()
    keep, p = _fake()
    cu2 = _cu([0, 10, 30])

    def slots(vals, pool, has=None):
        st, ka = gdn._slots_arg(vals, has, pool, len(vals))
        return st, ka

    def chunk(sl, **kw):
        a = dict(q=p, k=p, v=p, g=p, beta=p, cu=cu2, N=2, pool=p, out=p, T=30, H_q=2, H_v=4, dk=128, dv=128,
                 scale=0.1, dt=1, ws=p, wsb=1 << 40)
        a.update(kw)
        return lib.gdn_chunk_fwd_pooled(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"], a["pool"],
                                        ctypes.byref(sl[0]) if sl is not None else None, a["out"], a["T"], a["H_q"],
                                        a["H_v"], a["dk"], a["dv"], a["scale"], a["dt"], a["ws"], a["wsb"], None,
                                        None)

    assert chunk(None) == -1                          # slots are required
    assert chunk(slots([3, 3], 8)) == -1              # one row kept by two sequences
    assert chunk(slots([0, 8], 8)) == -1              # row past the pool
    assert chunk(slots([0, 1], -1)) == -1             # negative pool size
    assert chunk(slots([0, 1], 8), pool=None) == -1   # rows named but no pool
    assert chunk(slots([0, 1], 8), pool=p + 8) == -2  # misaligned pool
    assert chunk(slots([1, 2], 8), dk=64) == -2       # shape checks still apply
    assert chunk(slots([], 8), N=0, T=0, cu=_cu([0])) == 0

    def conv(sl, **kw):
        a = dict(x=p, cu=cu2, N=2, T=30, C=64, K=4, w=p, pool=p, out=p, dt=1)
        a.update(kw)
        return lib.gdn_conv1d_silu_fwd_pooled(a["x"], a["cu"], a["N"], a["T"], a["C"], a["K"], a["w"], None,
                                              a["pool"], ctypes.byref(sl[0]) if sl is not None else None,
                                              a["out"], a["dt"], None)

    assert conv(None) == -1
    assert conv(slots([5, 5], 8)) == -1
    assert conv(slots([-1, 9], 8)) == -1
    assert conv(slots([0, 1], 8), K=5) == -2

    def step(**kw):
        x = dict(q=p, k=p, v=p, a=p, b=p, A=p, dtb=p, pool=p, slot=p, P=8, out=p, N=4, H_q=2, H_v=4, dk=128,
                 dv=128, scale=0.1, dt=1)
        x.update(kw)
        return lib.gdn_recurrent_step_fused_pooled(x["q"], x["k"], x["v"], x["a"], x["b"], x["A"], x["dtb"],
                                                   x["pool"], x["slot"], x["P"], x["out"], x["N"], x["H_q"],
                                                   x["H_v"], x["dk"], x["dv"], x["scale"], x["dt"], None, None)

    assert step(slot=None) == -1
    assert step(P=-1) == -1
    assert step(pool=None) == -1
    assert step(slot=p + 2) == -2                     # int32 slots off their alignment
    assert step(N=0, slot=None) == 0

    def cstep(**kw):
        a = dict(x=p, N=3, C=64, K=4, w=p, pool=p, slot=p, P=8, out=p, dt=0)
        a.update(kw)
        return lib.gdn_conv1d_silu_step_pooled(a["x"], a["N"], a["C"], a["K"], a["w"], None, a["pool"], a["slot"],
                                               a["P"], a["out"], a["dt"], None)

    assert cstep(slot=None) == -1
    assert cstep(P=-1) == -1
    assert cstep(pool=None) == -1
    assert cstep(C=62) == -2

    assert lib.gdn_state_rows_zero(p, 8, 1024, p, 0, None) == 0    # nothing listed
    assert lib.gdn_state_rows_zero(p, 0, 1024, p, 4, None) == 0    # empty pool
    assert lib.gdn_state_rows_zero(p, 8, 1000, p, 4, None) == -2   # rows not whole 16-byte units
    assert lib.gdn_state_rows_zero(p, 8, 0, p, 4, None) == -1
    assert lib.gdn_state_rows_zero(p, 8, 1024, None, 4, None) == -1
    assert lib.gdn_state_rows_zero(p + 8, 8, 1024, p, 4, None) == -2
    assert lib.gdn_state_rows_copy(p, 8, 1024, p, p, -1, None) == -1
    assert lib.gdn_state_rows_copy(p, 8, 1024, p + 2, p, 4, None) == -2


def test_fused_prefill_rejects_before_any_device_work(gdn):
    lib = gdn.load_library()
    keep, p = _fake()
    cu = _cu([0, 10])

    def call(front, slots=None, **kw):
        a = dict(q=p, k=p, v=p, cu=cu, N=1, s0=p, out=p, fin=p, T=10, H_q=2, H_v=4, dk=128, dv=128, scale=0.1, dt=1,
                 ws=p, wsb=1 << 40)
        a.update(kw)
        return lib.gdn_chunk_fwd_fused(a["q"], a["k"], a["v"], ctypes.byref(front) if front is not None else None,
                                       a["cu"], a["N"], a["s0"], a["out"], a["fin"],
                                       ctypes.byref(slots[0]) if slots is not None else None, a["T"], a["H_q"],
                                       a["H_v"], a["dk"], a["dv"], a["scale"], a["dt"], a["ws"], a["wsb"], None, None)

    fe = gdn.FrontEnd(p, p, p, p)
    assert call(None) == -1                                   # the front end is required
    assert call(gdn.FrontEnd(None, p, p, p)) == -1            # a missing
    assert call(gdn.FrontEnd(p, p, None, p)) == -1            # A_log missing
    assert call(gdn.FrontEnd(p + 1, p, p, p)) == -2           # bf16 a off its 2-byte alignment
    assert call(gdn.FrontEnd(p, p, p, p + 2)) == -2           # fp32 dt_bias off its 4-byte alignment
    assert call(fe, dk=64) == -2
    assert call(fe, ws=None) == -3
    sl = gdn._slots_arg([0], None, 4, 1)
    assert call(fe, slots=sl, fin=p + 256) == -1              # with slots, final_state is the pool or NULL
    assert call(fe, slots=gdn._slots_arg([4], None, 4, 1)) == -1   # slot past the pool
    assert call(fe, N=0, T=0, cu=_cu([0])) == 0


def test_dev_seqlens_prefill_rejects_before_any_device_work(gdn):
    lib = gdn.load_library()
    keep, p = _fake()
    assert lib.gdn_chunk_fwd_dev_workspace_size(4096, 1, 16, 32, 128, 128, 1) > \
        lib.gdn_chunk_fwd_workspace_size(_cu([0, 4096]), 1, 16, 32, 128, 128, 1)
    assert lib.gdn_chunk_fwd_dev_workspace_size(100, 1, 3, 4, 64, 64, 1) == 0     # H_v % H_q != 0

    def call(**kw):
        a = dict(q=p, k=p, v=p, g=p, beta=p, cu=p, N=2, s0=None, out=p, fin=None, T=100, H_q=2, H_v=4, dk=64, dv=64,
                 scale=0.1, dt=1, ws=p, wsb=1 << 40)
        a.update(kw)
        return lib.gdn_chunk_fwd_dev(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["N"], a["s0"], a["out"],
                                     a["fin"], a["T"], a["H_q"], a["H_v"], a["dk"], a["dv"], a["scale"], a["dt"],
                                     a["ws"], a["wsb"], None, None)

    assert call(cu=None) == -1
    assert call(cu=p + 2) == -2               # int32 boundaries off their alignment
    assert call(g=None) == -1
    assert call(dk=32, dv=32) == -2
    assert call(wsb=1024) == -3
    assert call(N=-1) == -1
    assert call(N=0) == 0
    # T == 0 with sequences is not a no-op (their final states are written), and
    # its absent token tensors pass the checks up to the workspace test
    assert call(T=0, q=None, k=None, v=None, g=None, beta=None, out=None, wsb=0) == -3


def test_binding_refuses_host_tensors(gdn):
    torch = pytest.importorskip("torch")
    q = torch.zeros(4, 2, 64)
    with pytest.raises(ValueError):
        gdn.chunk_fwd(q, q, torch.zeros(4, 4, 64), torch.zeros(4, 4), torch.zeros(4, 4), [0, 4])
    with pytest.raises(TypeError):
        gdn.chunk_fwd(q.to(torch.float16), q, q, q, q, [0, 4])


def test_scratch_prefill_refuses_before_any_device_work(gdn):
    """gdn_chunk_fwd_scratch: an invalid batch, or one whose workspace exceeds
    the static array, is refused on the host (no GPU here: any HIP call would
    fail with GDN_ELAUNCH instead)."""
    lib = gdn.load_library()
    keep, p = _fake()
    assert gdn.SCRATCH_BYTES == 256 << 20

    def call(cu, T, H_q=16, H_v=32, d=128, dt=1, **kw):
        a = dict(q=p, k=p, v=p, g=p, beta=p, s0=None, out=p, fin=p, scale=0.1)
        a.update(kw)
        return lib.gdn_chunk_fwd_scratch(a["q"], a["k"], a["v"], a["g"], a["beta"], _cu(cu), len(cu) - 1, a["s0"],
                                         a["out"], a["fin"], T, H_q, H_v, d, d, a["scale"], dt, None)

    need = lambda T: lib.gdn_chunk_fwd_workspace_size(_cu([0, T]), 1, 16, 32, 128, 128, 1)  # noqa: E731
    assert need(4096) <= gdn.SCRATCH_BYTES < need(8192)
    assert call([0, 8192], 8192) == -3          # 8192 tokens at 32 heads: beyond the array
    assert call([0, 4096], 4000) == -1          # cu[N] != T
    assert call([0, 100], 100, H_q=3) == -2
    assert call([0], 0) == 0                    # empty batch: no-op


def test_stream_copy_validation(gdn):
    """gdn_stream_copy (measurement aid) refuses bad arguments on the host."""
    lib = gdn.load_library()
    keep, p = _fake(8)
    assert lib.gdn_stream_copy(p, p + 4096, 0, None) == 0         # nothing to copy
    assert lib.gdn_stream_copy(None, p, 256, None) == -1
    assert lib.gdn_stream_copy(p, p + 8, 256, None) == -2         # misaligned destination
    assert lib.gdn_stream_copy(p, p + 256, 24, None) == -2        # not a multiple of 16 bytes
    assert lib.gdn_stream_copy(p, p + 128, 256, None) == -1       # overlapping


def test_chunk_form_rule(gdn):
    """Which operands the state scan reads: W and U for a short single sequence
    (the operand stream fits the Infinity Cache, few tile chains), A and the raw
    rows for long sequences or batches with more tile chains than the chip holds
    twice over; fp32 always W and U.  Host logic only (on a part without a
    device the rule takes 256 compute units)."""
    assert gdn.chunk_form(4096, 1, 32, 128, "bf16") == "W"
    assert gdn.chunk_form(8192, 1, 32, 128, "bf16") == "A"
    assert gdn.chunk_form(65536, 1, 32, 128, "bf16") == "A"
    assert gdn.chunk_form(30702, 8, 32, 128, "bf16") == "A"
    assert gdn.chunk_form(34422, 256, 32, 128, "bf16") == "A"
    assert gdn.chunk_form(65536, 1, 32, 128, "f32") == "W"
    assert gdn.chunk_form(466, 6, 4, 128, "bf16") == "W"
    lib = gdn.load_library()
    assert lib.gdn_chunk_fwd_form(-1, 1, 32, 128, 1) == -1
    assert lib.gdn_chunk_fwd_form(64, 1, 32, 96, 1) == -1
    assert lib.gdn_chunk_fwd_form(64, 1, 32, 128, 7) == -2
