#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet forward hot path on one MI355X.

One step = one gdn_chunk_fwd over the headline prefill workload (one sequence
of T = 4096 tokens, H_q = 16 query/key heads, H_v = 32 value heads,
d_k = d_v = 128, bf16 q/k/v, fp32 gates and states, nonzero initial state),
all three kernels, inputs resident in HBM.  The batched decode step (256
sequences x 1 token, 537 MB of fp32 state updated in place, fresh seeded tokens
each step) is measured in the same run and reported under "decode", and the
same step taken from the raw inputs (q/k L2 norm, gate and beta computed inside
the step) under "decode_fused".

Prints ONE JSON line.  Timing: W untimed warm-up steps (default 300: a prefill
step on MI355X takes about 300 back-to-back steps, ~30 ms, to settle from
~100 to ~86 us at T = 4096; a streaming copy beforehand does not replace
them), then K timed steps of
the product entry point between two device synchronisations (value,
ms_per_step), then the same K steps again through gdn_chunk_fwd_ex, whose
start/stop HIP events are stamped by each kernel's own dispatch (per-kernel
durations for the roofline; the events themselves cost ~15 us a step, so they
are kept out of the first pass).  "roofline" reports the slowest kernel of the step against the
HBM roofline on its algorithmic bytes; "cpu_baseline" times the fp64 oracle on
the host cores over a bounded prefix of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s (Hv=32,d=128,T=4096) + MFMA util; decode state GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
FP32_MFMA_PEAK_TFLOPS = 157.3
# Kernels of one prefill launch, in stream order.  bf16: the output is formed
# inside the state scan and the third slot is the gated read-out pass (empty
# without the read-out); fp32: the separate output kernel.
STAGES_BF16 = ["chunk_prep", "chunk_state_o", "gated_readout"]
STAGES_F32 = ["chunk_prep", "chunk_state_h", "chunk_output_o"]


def stages_for(dtype):
    return STAGES_BF16 if dtype == "bf16" else STAGES_F32
CHUNK = 64


# ---------------------------------------------------------------------------
# algorithmic work of each kernel (bytes: every distinct input read once, every
# output written once; flops: 2 x multiply-adds of the chunk form, triangles
# exploited)
# ---------------------------------------------------------------------------

def prefill_work(T, N, n_chunks, H_q, H_v, d, es, has_s0=True, gated=False, form="W", qcopy=False):
    """Algorithmic bytes and flops of each kernel of one gdn_chunk_fwd.

    Bytes: every distinct input read once, every output and intermediate written
    once and read once per consuming kernel (K and Q are read once per key
    head).  chunk_prep writes, per (chunk, value head), the gate block (gc, kf,
    beta, beta gamma) and, once per key head, the key rows Kc; then either
    (form "W") W = A B Gamma K and U = A B V, which the state scan reads to
    form X = U - W S, or (form "A") A as six MFMA fragments, from which with
    the raw value rows the state scan forms X = A B (V - Gamma K S).  bf16 (es
    = 2): chunk_prep also forms P (the masked, decayed Q K^T, six 1 KiB
    fragments per chunk and value head), the state scan forms the output from
    P, q and its own on-chip h and X, and the gated read-out (when asked for)
    is a pass over the output.  qcopy (bf16, where the state scan takes one
    column tile a workgroup): chunk_prep also writes the query rows in the
    output waves' operand order (Qc, once per key head), which the scan then
    reads instead of q.  fp32 (always form "W"): the chunk-start states h and
    X go through HBM to a separate output kernel.  Flops: 2 x multiply-adds of
    the chunk form at full chunks, triangles exploited.
    """
    C = CHUNK
    chv, chq = n_chunks * H_v, n_chunks * H_q
    q_b = k_b = T * H_q * d * es
    v_b = o_b = T * H_v * d * es
    gate_b = T * H_v * 4     # g or beta
    G_b = chv * 4 * C * 4    # gate block per (chunk, value head)
    gc_b = chv * C * 4       # its gc row (what the fp32 output kernel reads)
    Af_b = chv * 6 * 64 * 8 * es  # A's six fragments
    W_b = U_b = X_b = chv * C * d * es
    Kc_b = chq * C * d * es  # the state scan's copy of the keys, one per key head
    H_b = chv * d * d * es
    S_b = N * H_v * d * d * 4
    P_b = chv * 6 * 1024
    tri = C * (C - 1) // 2   # strictly lower entries
    tri1 = C * (C + 1) // 2  # lower incl. diagonal
    s0 = S_b if has_s0 else 0
    if form == "A":
        prep = tri * d + C ** 3 // 6                       # K K^T, solve
        scan = 2 * C * d * d + tri1 * d                     # K S, A (B Y), Kc^T (kf X)
        prep_b = k_b + 2 * gate_b + G_b + Af_b + Kc_b
        scan_b = Kc_b + Af_b + G_b + v_b
    else:
        prep = tri * d + C ** 3 // 6 + 2 * tri1 * d        # K K^T, solve, W, U
        scan = 2 * C * d * d                                # W S, Kc^T (kf X)
        prep_b = k_b + v_b + 2 * gate_b + G_b + W_b + U_b + Kc_b
        scan_b = W_b + U_b + Kc_b + G_b
    if es == 2:
        qs_b = Kc_b if qcopy else q_b  # the scan's query rows: Qc (chunk-padded, like Kc) or q
        per = {"chunk_prep": prep + tri1 * d,                              # + Q K^T
               "chunk_state_o": scan + C * d * d + tri1 * d,               # + Q S, P X
               "gated_readout": 0}
        bytes_ = {"chunk_prep": prep_b + q_b + P_b + (Kc_b if qcopy else 0),
                  "chunk_state_o": scan_b + P_b + qs_b + s0 + S_b + o_b,
                  "gated_readout": (3 * o_b + d * 4) if gated else 0}      # o read, z read, out written
    else:
        per = {"chunk_prep": prep,
               "chunk_state_h": scan,
               "chunk_output_o": C * d * d + 2 * tri1 * d}                 # Q S, Q K^T, P X
        bytes_ = {"chunk_prep": prep_b,
                  "chunk_state_h": scan_b + s0 + H_b + X_b + S_b,
                  "chunk_output_o": q_b + k_b + gc_b + H_b + X_b + o_b + ((o_b + d * 4) if gated else 0)}
    flops = {k: 2 * v * chv for k, v in per.items()}
    return bytes_, flops


def decode_work(N, H_q, H_v, d, es, fused=False):
    """Bytes and flops of one decode step: the fp32 state read and written once,
    q, k, v, o, and g, beta (plain) or a, b and the per-head A_log, dt_bias (fused)."""
    state = N * H_v * d * d * 4
    gates = 2 * N * H_v * es + 2 * H_v * 4 if fused else 2 * N * H_v * 4
    io = 2 * N * H_q * d * es + 2 * N * H_v * d * es + gates
    return 2 * state + io, N * H_v * d * d * 8


# ---------------------------------------------------------------------------
# HIP events through the runtime torch loaded (same soname as libgdn's dependency)
# ---------------------------------------------------------------------------

class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        P = ctypes.c_void_p
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [P, P]
        self.lib.hipEventSynchronize.argtypes = [P]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        self.lib.hipEventDestroy.argtypes = [P]

    # Timing-only events: no system-scope fence (cache writeback + invalidate) when
    # they are recorded, so they do not perturb the kernels they bracket.
    DISABLE_SYSTEM_FENCE = 0x20000000

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return e

    def record(self, e, stream_ptr):
        rc = self.lib.hipEventRecord(e, ctypes.c_void_p(stream_ptr))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        self.lib.hipEventSynchronize(b)
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)


def per_step_ms(hip, stream_ptr, step, K, flush=None):
    """Milliseconds of each of K steps, each bracketed by its own pair of timing
    events on the stream: back to back, or with flush() queued before every step
    outside its events (so the step starts with cold caches)."""
    evs = [(hip.event(), hip.event()) for _ in range(K)]
    for i in range(K):
        if flush is not None:
            flush()
        hip.record(evs[i][0], stream_ptr)
        step()
        hip.record(evs[i][1], stream_ptr)
    return sorted(hip.elapsed_ms(a, b) for a, b in evs)


def stats(ms):
    """median / min / mean of a list of per-step milliseconds."""
    n = len(ms)
    med = ms[n // 2] if n % 2 else 0.5 * (ms[n // 2 - 1] + ms[n // 2])
    return {"median_ms": med, "min_ms": min(ms), "mean_ms": sum(ms) / n, "n": n}


class CacheFlush:
    """Evicts the 256 MB Infinity Cache (and L2) between timed steps: a 1 GiB
    streaming copy (two 512 MiB buffers) through gdn_stream_copy, queued on the
    stream outside the steps' timing events."""

    def __init__(self, torch, gdn, device, nbytes=512 << 20):
        self.gdn = gdn
        self.src = torch.ones(nbytes, dtype=torch.uint8, device=device)
        self.dst = torch.empty_like(self.src)

    def __call__(self):
        self.gdn.stream_copy(self.src, self.dst)


def hbm_probe(torch, gdn, hip, device, nbytes=1 << 30, reps=20):
    """Achievable HBM bandwidth: a 1 GiB device-to-device copy through the
    library's own streaming copy kernel (read once, write once: 2 GiB of traffic,
    8x the Infinity Cache), median of `reps` event-timed copies."""
    src = torch.ones(nbytes, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    sptr = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        gdn.stream_copy(src, dst)
    torch.cuda.synchronize()
    st = stats(per_step_ms(hip, sptr, lambda: gdn.stream_copy(src, dst), reps))
    ok = bool(torch.equal(src[:4096], dst[:4096])) and bool(torch.equal(src[-4096:], dst[-4096:]))
    del src, dst
    torch.cuda.empty_cache()
    return {"kernel": "gdn_stream_copy", "bytes_per_copy": 2 * nbytes, "median_us": st["median_ms"] * 1e3,
            "gb_per_s": 2 * nbytes / (st["median_ms"] * 1e-3) / 1e9,
            "gb_per_s_best": 2 * nbytes / (st["min_ms"] * 1e-3) / 1e9, "copy_checked": ok}


def _dev(arr, dtype, torch, device):
    import numpy as np

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def _source_sha() -> str:
    """Hash of the kernel sources with comments and blank space removed, so that
    counter summaries stay tied to the code they were taken on, not its prose."""
    h = hashlib.sha256()
    for f in ("gdn_chunk.hip", "gdn_decode.hip", "gdn_device.h", "gdn_params.h"):
        with open(os.path.join(ROOT, "gated_deltanet_state_chunk_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments (no string in these sources holds //)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip()
        if line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=", 1)
        vals[k.strip()] = v.strip()
    if vals.get("source_sha") != _source_sha():
        return None
    key = f"{kernel}.hbm_bytes_per_launch"
    return float(vals[key]) if key in vals else None


# ---------------------------------------------------------------------------
# measurements
# ---------------------------------------------------------------------------

def bench_prefill(args, torch, gdn, hip, device, gated=False):
    """The prefill step; with gated, out also passes through the gated RMSNorm
    read-out epilogue (z and weight seeded, eps 1e-6)."""
    import gdn_inputs

    inp = gdn_inputs.make_workload(args.workload)
    dt = inp.dtype
    q, k, v = (_dev(x, dt, torch, device) for x in (inp.q, inp.k, inp.v))
    g, beta = _dev(inp.g, "f32", torch, device), _dev(inp.beta, "f32", torch, device)
    s0 = _dev(inp.initial_state, "f32", torch, device) if inp.initial_state is not None else None
    lay = gdn.workspace_layout(inp.T, inp.cu_seqlens, inp.H_q, inp.H_v, inp.d_k, inp.d_v, dt)
    ws_bytes = gdn.workspace_size(inp.T, inp.cu_seqlens, inp.H_q, inp.H_v, inp.d_k, inp.d_v, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    out = torch.empty((inp.T, inp.H_v, inp.d_v), dtype=q.dtype, device=device)
    fin = torch.empty((inp.N, inp.H_v, inp.d_k, inp.d_v), dtype=torch.float32, device=device)
    lib = gdn.load_library()
    cu = (ctypes.c_int32 * (inp.N + 1))(*[int(x) for x in inp.cu_seqlens])
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    code = gdn.DTYPE_BF16 if dt == "bf16" else gdn.DTYPE_F32
    gate_ref = None
    if gated:
        z, w = gdn_inputs.make_gate(93, inp.T, inp.H_v, inp.d_v, dt)
        zt, wt = _dev(z, dt, torch, device), _dev(w, "f32", torch, device)
        gate_obj = gdn.OutputGate(zt.data_ptr(), wt.data_ptr(), 1e-6)
        gate_ref = ctypes.byref(gate_obj)
    K = args.steps
    STAGES = stages_for(dt)
    NEV = 2 * len(STAGES)
    ev = [[hip.event() for _ in range(NEV)] for _ in range(max(K, 1))]

    def step(events=None):
        arr = None
        if events is not None:
            arr = (ctypes.c_void_p * NEV)(*[e.value for e in events])
        if events is None and gate_ref is None:
            rc = lib.gdn_chunk_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), cu,
                                   inp.N, None if s0 is None else s0.data_ptr(), out.data_ptr(), fin.data_ptr(),
                                   inp.T, inp.H_q, inp.H_v, inp.d_k, inp.d_v, inp.scale, code, ws.data_ptr(),
                                   ws_bytes, ctypes.c_void_p(sptr))
            if rc != 0:
                raise gdn.GdnError(rc, "gdn_chunk_fwd")
            return
        rc = lib.gdn_chunk_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), cu,
                                  inp.N, None if s0 is None else s0.data_ptr(), out.data_ptr(), fin.data_ptr(),
                                  inp.T, inp.H_q, inp.H_v, inp.d_k, inp.d_v, inp.scale, code, ws.data_ptr(),
                                  ws_bytes, ctypes.c_void_p(sptr), 0, gate_ref, arr)
        if rc != 0:
            raise gdn.GdnError(rc, "gdn_chunk_fwd_ex")

    # Whether chunk_prep writes the query copy (Qc) for this batch (the state
    # scan's choice of tile width): one step on a poisoned workspace.
    qc0 = lay["off_Qc"]
    qc1 = qc0 + lay["n_chunks"] * inp.H_q * 64 * inp.d_k * 2
    qcopy = False
    if dt == "bf16" and qc1 > qc0:
        ws[qc0:qc1].fill_(0xA5)
        step()
        torch.cuda.synchronize()
        qcopy = not bool((ws[qc0:qc1] == 0xA5).all())
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Pass 1: the product entry point, no per-kernel events (they cost ~15 us a step).
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(K):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    # Pass 2: the same steps with start/stop events stamped by each kernel's dispatch.
    t0.record(stream)
    for i in range(K):
        step(ev[i])
    t1.record(stream)
    torch.cuda.synchronize()
    timed_ms = t0.elapsed_time(t1) / K
    stage_ms = {s: sum(hip.elapsed_ms(ev[i][2 * j], ev[i][2 * j + 1]) for i in range(K)) / K
                for j, s in enumerate(STAGES)}
    ms_step = total_ms / K
    # Pass 3: per-step distribution, back to back; pass 4: each step after a
    # cache-evicting copy (outside its events), i.e. from HBM-resident data.
    nstep = max(K, 20)
    warm = stats(per_step_ms(hip, sptr, step, nstep))
    cold = stats(per_step_ms(hip, sptr, step, nstep, flush=CacheFlush(torch, gdn, device)))
    es = 2 if dt == "bf16" else 4
    form = gdn.chunk_form(inp.T, inp.N, inp.H_v, inp.d_k, dt)
    bytes_, flops = prefill_work(inp.T, inp.N, lay["n_chunks"], inp.H_q, inp.H_v, inp.d_k, es,
                                 has_s0=s0 is not None, gated=gated, form=form, qcopy=qcopy)
    return dict(inp=inp, lay=lay, ms_step=ms_step, wall_s=wall, stage_ms=stage_ms, bytes=bytes_, flops=flops,
                stages=STAGES, ms_step_with_events=timed_ms, warm=warm, cold=cold, form=form, qcopy=qcopy)


def bench_prefill_serving(args, torch, gdn, device):
    """The prefill as a serving layer calls it: raw q, k, a, b (L2 norm, gate and
    beta inside the kernels, gdn_chunk_fwd_fused) and the gated read-out, at the
    shapes of the prefill workload."""
    import gdn_inputs

    base = gdn_inputs.make_workload(args.workload)
    seqlens = [int(x) for x in (base.cu_seqlens[1:] - base.cu_seqlens[:-1])]
    inp = gdn_inputs.make_prefill_raw(71, seqlens, base.H_q, base.H_v, base.d_k, base.d_v, base.dtype)
    dt = inp.dtype
    q, k, v, a, b = (_dev(getattr(inp, n), dt, torch, device) for n in ("q", "k", "v", "a", "b"))
    A_log, dt_bias = _dev(inp.A_log, "f32", torch, device), _dev(inp.dt_bias, "f32", torch, device)
    s0 = _dev(inp.initial_state, "f32", torch, device)
    z, w = gdn_inputs.make_gate(72, inp.T, inp.H_v, inp.d_v, dt)
    gate = (_dev(z, dt, torch, device), _dev(w, "f32", torch, device), 1e-6)
    ws = torch.empty(gdn.workspace_size(inp.T, inp.cu_seqlens, inp.H_q, inp.H_v, inp.d_k, inp.d_v, dt),
                     dtype=torch.uint8, device=device)
    out = torch.empty((inp.T, inp.H_v, inp.d_v), dtype=q.dtype, device=device)
    fin = torch.empty((inp.N, inp.H_v, inp.d_k, inp.d_v), dtype=torch.float32, device=device)

    # Arguments marshalled once (as a serving loop would), so the timed loop is
    # the library call alone.
    lib = gdn.load_library()
    cu = (ctypes.c_int32 * (inp.N + 1))(*[int(x) for x in inp.cu_seqlens])
    fe = gdn.FrontEnd(a.data_ptr(), b.data_ptr(), A_log.data_ptr(), dt_bias.data_ptr())
    gate_obj = gdn.OutputGate(gate[0].data_ptr(), gate[1].data_ptr(), gate[2])
    code = gdn.DTYPE_BF16 if dt == "bf16" else gdn.DTYPE_F32
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args_c = (q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(fe), cu, inp.N, s0.data_ptr(), out.data_ptr(),
              fin.data_ptr(), None, inp.T, inp.H_q, inp.H_v, inp.d_k, inp.d_v, inp.scale, code, ws.data_ptr(),
              ws.numel(), ctypes.byref(gate_obj), sptr)

    def step():
        rc = lib.gdn_chunk_fwd_fused(*args_c)
        if rc != 0:
            raise gdn.GdnError(rc, "gdn_chunk_fwd_fused")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    return {"workload": args.workload + " from raw q, k, a, b (front end in the kernels) with the gated read-out",
            "ms_per_step": ms, "tokens_per_s": inp.T / (ms * 1e-3)}


def bench_prefill_many(args, torch, gdn, hip, device):
    """A serving prefill batch of 256 short requests (many_256req: lengths uniform
    in [1, 256], 34422 tokens, 32 value heads): gdn_chunk_fwd with host
    cu_seqlens and gdn_chunk_fwd_dev with device cu_seqlens, per-step medians."""
    import gdn_inputs

    inp = gdn_inputs.make_workload("many_256req")
    q, k, v = (_dev(x, inp.dtype, torch, device) for x in (inp.q, inp.k, inp.v))
    g, beta = _dev(inp.g, "f32", torch, device), _dev(inp.beta, "f32", torch, device)
    s0 = _dev(inp.initial_state, "f32", torch, device)
    out = torch.empty((inp.T, inp.H_v, inp.d_v), dtype=q.dtype, device=device)
    fin = torch.empty((inp.N, inp.H_v, inp.d_k, inp.d_v), dtype=torch.float32, device=device)
    ws = torch.empty(gdn.workspace_size(inp.T, inp.cu_seqlens, inp.H_q, inp.H_v, inp.d_k, inp.d_v, inp.dtype),
                     dtype=torch.uint8, device=device)
    wsd = torch.empty(gdn.dev_workspace_size(inp.T, inp.N, inp.H_q, inp.H_v, inp.d_k, inp.d_v, inp.dtype),
                      dtype=torch.uint8, device=device)
    cud = torch.tensor(inp.cu_seqlens, dtype=torch.int32, device=device)
    sptr = torch.cuda.current_stream().cuda_stream
    host = lambda: gdn.chunk_fwd(q, k, v, g, beta, inp.cu_seqlens, initial_state=s0, scale=inp.scale,  # noqa: E731
                                 out=out, final_state=fin, workspace=ws)
    devp = lambda: gdn.chunk_fwd_dev(q, k, v, g, beta, cud, initial_state=s0, scale=inp.scale,  # noqa: E731
                                     out=out, final_state=fin, workspace=wsd)
    res = {"workload": f"many_256req: {inp.N} sequences, lengths uniform in [1, 256], T={inp.T}, H_q={inp.H_q}, "
                       f"H_v={inp.H_v}, d={inp.d_k}, bf16"}
    for name, fn in (("gdn_chunk_fwd", host), ("gdn_chunk_fwd_dev", devp)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        st = stats(per_step_ms(hip, sptr, fn, max(args.steps, 20)))
        res[name] = {"median_us": st["median_ms"] * 1e3, "min_us": st["min_ms"] * 1e3,
                     "tokens_per_s": inp.T / (st["median_ms"] * 1e-3)}
    return res


def bench_decode(args, torch, gdn, hip, device, fused=False, gated=False, pooled=False):
    """Decode steps on the 256 x 32-head batch: the plain step (normalised q, k and
    final g, beta) or, with fused, the step from raw q, k, a, b (front end inside);
    with pooled (fused only), the states live in a pool of twice as many rows and
    each sequence's row comes from a seeded permutation (the serving form)."""
    import numpy as np

    import gdn_inputs

    cfg = gdn_inputs.DECODE_WORKLOAD
    N, H_q, H_v, d, dt = cfg["N"], cfg["H_q"], cfg["H_v"], cfg["d_k"], cfg["dtype"]
    state = _dev(gdn_inputs.make_decode_state(cfg["seed"], N, H_v, d, d, cfg["state_std"]), "f32", torch, device)
    toks = []
    for s in range(cfg["steps"]):
        if fused:
            t = gdn_inputs.make_decode_raw_token(gdn_inputs.decode_step_seed(s), N, H_q, H_v, d, d, dt)
            toks.append(tuple(_dev(x, dt, torch, device) for x in (t.q, t.k, t.v, t.a, t.b)) +
                        (_dev(t.A_log, "f32", torch, device), _dev(t.dt_bias, "f32", torch, device)))
        else:
            t = gdn_inputs.make_decode_token(gdn_inputs.decode_step_seed(s), N, H_q, H_v, d, d, dt)
            toks.append(tuple(_dev(x, dt, torch, device) for x in (t.q, t.k, t.v)) +
                        (_dev(t.g, "f32", torch, device), _dev(t.beta, "f32", torch, device)))
    step_fn = gdn.recurrent_step_fused if fused else gdn.recurrent_step
    if gated:
        z, w = gdn_inputs.make_gate(97, N, H_v, d, dt)
        gate = (_dev(z, dt, torch, device), _dev(w, "f32", torch, device), 1e-6)
        plain_fn = step_fn
        step_fn = lambda *a, **kw: plain_fn(*a, gate=gate, **kw)  # noqa: E731
    if pooled:
        assert fused
        P = 2 * N
        slot = torch.tensor(np.random.default_rng(cfg["seed"] + 1).permutation(P)[:N].astype(np.int32),
                            device=device)
        pool = torch.zeros((P, H_v, d, d), dtype=torch.float32, device=device)
        pool[slot.long()] = state
        state = pool
        unpooled_fn = step_fn
        step_fn = lambda *a, **kw: gdn.recurrent_step_fused_pooled(*a, slot, **kw)  # noqa: E731
        assert unpooled_fn is gdn.recurrent_step_fused
    out = torch.empty((N, H_v, d), dtype=toks[0][0].dtype, device=device)
    scale = 1.0 / math.sqrt(d)
    K = max(args.steps, cfg["steps"])
    for i in range(args.warmup):
        step_fn(*toks[i % len(toks)], state, scale=scale, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # Pass 1: back-to-back steps, no per-kernel events.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(K):
        step_fn(*toks[i % len(toks)], state, scale=scale, out=out)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    # Pass 2: the kernel bracketed by timing events.
    evs = [(hip.event(), hip.event()) for _ in range(K)]
    for i in range(K):
        hip.record(evs[i][0], stream.cuda_stream)
        step_fn(*toks[i % len(toks)], state, scale=scale, out=out)
        hip.record(evs[i][1], stream.cuda_stream)
    torch.cuda.synchronize()
    kst = stats(sorted(hip.elapsed_ms(a, b) for a, b in evs))
    kms = kst["mean_ms"]
    nbytes, nflops = decode_work(N, H_q, H_v, d, 2 if dt == "bf16" else 4, fused=fused)
    if gated:
        nbytes += N * H_v * d * (2 if dt == "bf16" else 4) + d * 4  # z, weight
    return dict(N=N, ms_step=ms, kernel_ms=kms, kernel_stats=kst, bytes=nbytes, flops=nflops, steps=K)


def bench_conv(args, torch, gdn, hip, device):
    """Causal conv1d + SiLU at the model's shapes: the prefill over T = 4096
    tokens of C = 8192 channels (q, k, v of 16 + 16 + 32 heads at d = 128), K = 4,
    bf16, with a history in and out; and the decode step for 256 sequences.
    "us": calls back to back (for the small step this is the host's call rate);
    "kernel_us": the median of the calls bracketed one by one by timing events."""
    import gdn_inputs

    T, C, K, N = 4096, 8192, 4, 256
    x, s0, w, b = gdn_inputs.make_conv(80, T, C, K, 1, "bf16")
    xd, s0d, wd, bd = (_dev(x, "bf16", torch, device), _dev(s0, "bf16", torch, device),
                       _dev(w, "f32", torch, device), _dev(b, "f32", torch, device))
    out = torch.empty_like(xd)
    fin = torch.empty_like(s0d)
    cu = [0, T]
    xs, ss, _, _ = gdn_inputs.make_conv(81, N, C, K, N, "bf16")
    xsd, ssd = _dev(xs, "bf16", torch, device), _dev(ss, "bf16", torch, device)
    outs = torch.empty_like(xsd)

    def timed(fn, K_):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(K_):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / K_

    def kernel_timed(fn, K_):
        sp = torch.cuda.current_stream().cuda_stream
        return stats(per_step_ms(hip, sp, fn, K_))["median_ms"]

    steps = max(args.steps, 20)
    fp = lambda: gdn.conv1d_silu(xd, cu, wd, bd, initial_state=s0d, final_state=fin, out=out)  # noqa: E731
    fs = lambda: gdn.conv1d_silu_step(xsd, wd, bd, ssd, out=outs)  # noqa: E731
    ms_p, ms_s = timed(fp, steps), timed(fs, steps)
    kms_p, kms_s = kernel_timed(fp, steps), kernel_timed(fs, steps)
    bytes_p = 2 * T * C * 2 + C * K * 4 + C * 4 + 2 * (K - 1) * C * 2
    bytes_s = 2 * N * C * 2 + 2 * N * (K - 1) * C * 2 + C * K * 4 + C * 4
    return {"prefill": {"workload": f"T={T}, C={C}, K={K}, bf16", "us": ms_p * 1e3, "kernel_us": kms_p * 1e3,
                        "gb_per_s": bytes_p / (kms_p * 1e-3) / 1e9,
                        "hbm_frac": bytes_p / (kms_p * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "decode_step": {"workload": f"N={N}, C={C}, K={K}, bf16", "us": ms_s * 1e3, "kernel_us": kms_s * 1e3,
                            "gb_per_s": bytes_s / (kms_s * 1e-3) / 1e9,
                            "hbm_frac": bytes_s / (kms_s * 1e-3) / 1e9 / HBM_PEAK_GBS}}


def cpu_baseline(inp, target_s=10.0):
    """fp64 oracle on the host cores over the prefill workload (all heads): a prefix
    sized to about target_s seconds, or the whole workload repeated until then."""
    import oracle

    threads = oracle.max_threads()
    s0 = None if inp.initial_state is None else inp.initial_state[:1].astype("float64")

    def run(Tp):
        t = time.perf_counter()
        oracle.forward(inp.q32()[:Tp], inp.k32()[:Tp], inp.v32()[:Tp], inp.g[:Tp], inp.beta[:Tp], [0, Tp],
                       inp.H_q, inp.H_v, inp.scale, initial_state=s0)
        return time.perf_counter() - t

    probe_T = min(256, inp.T)
    tp = run(probe_T)
    Ts = int(min(inp.T, max(probe_T, probe_T * target_s / max(tp, 1e-6))))
    Ts = max(CHUNK, Ts // CHUNK * CHUNK) if inp.T >= CHUNK else inp.T
    reps, total = 0, 0.0
    while True:
        total += run(Ts)
        reps += 1
        if total >= target_s or reps >= 1000:
            break
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return dict(value=reps * Ts / total, unit="tokens/s", cores=threads, kind="oracle", cpu_model=cpu_model(),
                sample=f"fp64 token recurrence (oracle/gdn_recurrence.c, OpenMP over value heads) on the first "
                       f"{Ts} of {inp.T} tokens, all {inp.H_v} value heads, run {reps} times in {total:.2f} s wall; "
                       f"{avail} host cores visible, {threads} OpenMP threads")


def cpu_model() -> str:
    """The host CPU's model name (first processor entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def copy_calibration(torch, gdn, device, gib=1.0):
    """The library's streaming copy (gdn_stream_copy, kernel stream_copy_kernel) of
    known size, run under rocprofv3 --pmc to calibrate the HBM byte counters."""
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        gdn.stream_copy(src, dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="prefill_T4096",
                    choices=["prefill_T4096", "varlen_8seq", "long_T65536", "many_256req", "tiny_f32_T100"])
    ap.add_argument("--only", choices=["all", "prefill", "decode", "copy", "many"], default="all",
                    help="restrict the run (used for counter collection): prefill = the workload's plain and gated "
                         "steps only; many = the 256-request batch only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures a single GPU; --gpus {args.gpus} is not supported (the GDN core shards over "
              f"sequences and value heads with no exchange between GPUs).", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_deltanet_state_chunk_amd as gdn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    gdn.load_library()
    hip = Hip()
    if args.only == "copy":
        copy_calibration(torch, gdn, device)
        return
    if args.only == "many":
        print(json.dumps({"prefill_many": bench_prefill_many(args, torch, gdn, hip, device)}), flush=True)
        return

    res = {}
    pre = pre_g = dec = decf = decg = decp = None
    hbm = None
    if args.only in ("all", "prefill", "decode"):
        hbm = hbm_probe(torch, gdn, hip, device)
        print(f"[bench] achievable HBM (1 GiB streaming copy): {hbm['gb_per_s']:.0f} GB/s median, "
              f"{hbm['gb_per_s_best']:.0f} best", file=sys.stderr, flush=True)
        res["achievable_hbm"] = hbm
    if args.only in ("all", "prefill"):
        pre = bench_prefill(args, torch, gdn, hip, device)
        print(f"[bench] prefill {args.workload}: {pre['ms_step']:.4f} ms/step, stages "
              + ", ".join(f"{s} {pre['stage_ms'][s] * 1e3:.1f} us" for s in pre["stages"]), file=sys.stderr,
              flush=True)
        pre_g = bench_prefill(args, torch, gdn, hip, device, gated=True)
        print(f"[bench] prefill {args.workload} + gated read-out: {pre_g['ms_step']:.4f} ms/step, "
              + ", ".join(f"{s} {pre_g['stage_ms'][s] * 1e3:.1f} us" for s in pre_g["stages"]), file=sys.stderr,
              flush=True)
    if args.only == "all":
        pre_s = bench_prefill_serving(args, torch, gdn, device)
        print(f"[bench] prefill {args.workload} from raw inputs + gated read-out: {pre_s['ms_per_step']:.4f} ms/step",
              file=sys.stderr, flush=True)
        res["prefill_serving"] = pre_s
        if args.workload == "prefill_T4096":
            many = bench_prefill_many(args, torch, gdn, hip, device)
            print(f"[bench] prefill of 256 short requests: host cu_seqlens {many['gdn_chunk_fwd']['median_us']:.1f} us, "
                  f"device cu_seqlens {many['gdn_chunk_fwd_dev']['median_us']:.1f} us", file=sys.stderr, flush=True)
            res["prefill_many"] = many
    if args.only in ("all", "decode"):
        dec = bench_decode(args, torch, gdn, hip, device)
        print(f"[bench] decode: {dec['ms_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        decf = bench_decode(args, torch, gdn, hip, device, fused=True)
        print(f"[bench] decode (fused front end): {decf['ms_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        decp = bench_decode(args, torch, gdn, hip, device, fused=True, pooled=True)
        print(f"[bench] decode (fused front end, state pool): {decp['ms_step'] * 1e3:.1f} us/step", file=sys.stderr,
              flush=True)
        decg = bench_decode(args, torch, gdn, hip, device, fused=True, gated=True)
        print(f"[bench] decode (front end + gated read-out): {decg['ms_step'] * 1e3:.1f} us/step", file=sys.stderr,
              flush=True)

    if pre is not None:
        inp = pre["inp"]
        ms = pre["ms_step"]
        tokens = inp.T
        STAGES = pre["stages"]
        dom = max(STAGES, key=lambda s: pre["stage_ms"][s])
        dom_s = pre["stage_ms"][dom] * 1e-3
        achieved = pre["bytes"][dom] / dom_s / 1e9
        traffic = _traffic_from_profiles(dom, args.workload)
        total_flops = sum(pre["flops"].values())
        mfma_peak = BF16_MFMA_PEAK_TFLOPS if inp.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
        res.update({
            "metric": METRIC,
            "value": tokens / (ms * 1e-3),
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": ms,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": inp.dtype,
            "data": "synthetic",
            "config": {"workload": args.workload, "seqlens": [int(x) for x in
                                                             (inp.cu_seqlens[1:] - inp.cu_seqlens[:-1])],
                       "T": inp.T, "H_q": inp.H_q, "H_v": inp.H_v, "d_k": inp.d_k, "d_v": inp.d_v,
                       "chunk": CHUNK, "initial_state": inp.initial_state is not None,
                       "scan_operands": pre["form"], "query_copy": pre["qcopy"]},
            "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS,
                         "frac_of_achievable": achieved / hbm["gb_per_s"] if hbm else None,
                         "traffic": traffic},
            "step_ms": pre["warm"],
            "step_ms_cold": pre["cold"],
            "tokens_per_s_median": tokens / (pre["warm"]["median_ms"] * 1e-3),
            "tokens_per_s_cold_median": tokens / (pre["cold"]["median_ms"] * 1e-3),
            "whole_step": {"algorithmic_mbytes": sum(pre["bytes"].values()) / 1e6,
                           "gb_per_s": sum(pre["bytes"].values()) / (ms * 1e-3) / 1e9,
                           "frac_of_peak": sum(pre["bytes"].values()) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "stages_us": {s: pre["stage_ms"][s] * 1e3 for s in STAGES},
            "ms_per_step_with_kernel_events": pre["ms_step_with_events"],
            "stage_hbm_frac": {s: pre["bytes"][s] / (pre["stage_ms"][s] * 1e-3) / 1e9 / HBM_PEAK_GBS
                               for s in STAGES if pre["bytes"][s] > 0},
            "mfma_util": {"whole_step": total_flops / (ms * 1e-3) / 1e12 / mfma_peak,
                          **{s: pre["flops"][s] / (pre["stage_ms"][s] * 1e-3) / 1e12 / mfma_peak for s in STAGES
                             if pre["flops"][s] > 0}},
            "algorithmic": {"gflop": total_flops / 1e9, "mbytes": {s: pre["bytes"][s] / 1e6 for s in STAGES}},
        })
    if dec is not None:
        gbs = dec["bytes"] / (dec["ms_step"] * 1e-3) / 1e9
        kgbs = dec["bytes"] / (dec["kernel_ms"] * 1e-3) / 1e9
        decode = {"workload": "decode_256x1", "us_per_step": dec["ms_step"] * 1e3, "state_gb_per_s": gbs,
                  "kernel_us": dec["kernel_ms"] * 1e3, "kernel_us_median": dec["kernel_stats"]["median_ms"] * 1e3,
                  "kernel_us_min": dec["kernel_stats"]["min_ms"] * 1e3,
                  "tokens_per_s": dec["N"] / (dec["ms_step"] * 1e-3), "steps": dec["steps"],
                  "roofline": {"bound": "hbm", "kernel": "recurrent_step", "achieved": kgbs, "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": kgbs / HBM_PEAK_GBS,
                               "traffic": _traffic_from_profiles("recurrent_step", "decode_256x1")}}
        if pre is None:
            res.update({"metric": METRIC, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": dec["steps"],
                        "warmup": args.warmup, "ms_per_step": dec["ms_step"], "higher_is_better": True,
                        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                        "config": {"workload": "decode_256x1"}, "roofline": decode["roofline"]})
        res["decode"] = decode
    if pre_g is not None:
        ro = pre_g["stages"][2]  # the kernel that applies the read-out
        og = pre_g["stage_ms"][ro] * 1e-3
        res["prefill_gated"] = {
            "workload": args.workload + " with the gated RMSNorm read-out",
            "ms_per_step": pre_g["ms_step"], "tokens_per_s": pre_g["inp"].T / (pre_g["ms_step"] * 1e-3),
            "stages_us": {s: pre_g["stage_ms"][s] * 1e3 for s in pre_g["stages"]},
            "readout_kernel": ro, "readout_hbm_frac": pre_g["bytes"][ro] / og / 1e9 / HBM_PEAK_GBS}
    if decg is not None:
        kg = decg["bytes"] / (decg["kernel_ms"] * 1e-3) / 1e9
        res["decode_fused_gated"] = {
            "workload": "decode_256x1 from raw inputs, with the gated RMSNorm read-out (nodes 7 and 8 in one pass)",
            "us_per_step": decg["ms_step"] * 1e3, "kernel_us": decg["kernel_ms"] * 1e3,
            "tokens_per_s": decg["N"] / (decg["ms_step"] * 1e-3),
            "roofline": {"bound": "hbm", "achieved": kg, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": kg / HBM_PEAK_GBS, "traffic": None}}
    if decf is not None:
        kgbs = decf["bytes"] / (decf["kernel_ms"] * 1e-3) / 1e9
        res["decode_fused"] = {
            "workload": "decode_256x1 from raw q, k, a, b (q/k L2 norm, gate and beta inside the step)",
            "us_per_step": decf["ms_step"] * 1e3, "kernel_us": decf["kernel_ms"] * 1e3,
            "state_gb_per_s": decf["bytes"] / (decf["ms_step"] * 1e-3) / 1e9,
            "tokens_per_s": decf["N"] / (decf["ms_step"] * 1e-3), "steps": decf["steps"],
            "roofline": {"bound": "hbm", "kernel": "recurrent_step_fused", "achieved": kgbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": kgbs / HBM_PEAK_GBS, "traffic": None}}
    if decp is not None:
        kp = decp["bytes"] / (decp["kernel_ms"] * 1e-3) / 1e9
        res["decode_fused_pooled"] = {
            "workload": "decode_256x1 from raw q, k, a, b over a 512-row state pool, each sequence's row from a "
                        "seeded permutation (gdn_recurrent_step_fused_pooled)",
            "us_per_step": decp["ms_step"] * 1e3, "kernel_us": decp["kernel_ms"] * 1e3,
            "tokens_per_s": decp["N"] / (decp["ms_step"] * 1e-3),
            "roofline": {"bound": "hbm", "achieved": kp, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": kp / HBM_PEAK_GBS, "traffic": None}}
    if args.only == "all":
        conv = bench_conv(args, torch, gdn, hip, device)
        print(f"[bench] conv1d+SiLU: prefill {conv['prefill']['kernel_us']:.1f} us, decode step "
              f"{conv['decode_step']['kernel_us']:.1f} us (back-to-back calls {conv['decode_step']['us']:.1f} us)",
              file=sys.stderr, flush=True)
        res["conv1d_silu"] = conv
    if pre is not None and args.only == "all" and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(pre["inp"])
    res["source_sha"] = _source_sha()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
