"""ORACLE (test infrastructure only): fp64 chunk-wise form of Gated DeltaNet.

Written from "实验三：GDN Prefill 前向优化", section "计算过程描述" (the four
stages and the chunk equations) and section "输入输出定义" (the in-chunk
inclusive cumulative gate that restarts at every chunk; GVA head mapping).
For chunk c with valid length ell = min(C, L - cC), with Q, K, V the chunk's
valid rows, Gamma = Diag(exp(g_cumsum)), B = Diag(beta):

    A       = (I + StrictLower(B Gamma K K^T Gamma^{-1}))^{-1}
    U       = A B V,          W = A B Gamma K
    S_{c+1} = gamma_ell S_c + gamma_ell K^T Gamma^{-1} (U - W S_c)
    O_c     = scale [Gamma Q S_c + Gamma Lower(Q K^T) Gamma^{-1} (U - W S_c)]

StrictLower drops the diagonal, Lower keeps it.  The inverse is a general
dense inverse (numpy.linalg.inv); Gamma and Gamma^{-1} are formed as the
diagonal matrices the formulas name.  The chunk size C is a parameter so that
C = 1 (the token recurrence) and C >= L (the fully parallel form) can be
checked, as the "Chunk-wise Parallel" section of the same page describes.

This module is independent of oracle/gdn_recurrence.c and of the HIP library:
it shares no code with either.  Only tests/ and the smoke check import it.
For small inputs only (pure numpy, per (sequence, head, chunk) loops).
"""
from __future__ import annotations

import numpy as np


def chunk_forward(q, k, v, g, beta, cu_seqlens, H_q, H_v, scale, initial_state=None, C=64,
                  keep_intermediates=False):
    """Chunk-form forward over a packed batch.

    q, k: [T, H_q, d_k]; v: [T, H_v, d_v]; g, beta: [T, H_v] (any float dtype,
    promoted to float64); cu_seqlens: [N+1]; initial_state: [N, H_v, d_k, d_v] or None.

    Returns dict with 'out' [T, H_v, d_v], 'final_state' [N, H_v, d_k, d_v] and,
    when keep_intermediates, per-chunk lists keyed by (n, h):
      'gc' (cumulative gate, length ell), 'A' (ell x ell), 'W' (ell x d_k),
      'U' (ell x d_v), 'h' (state at chunk start, d_k x d_v), 'X' (U - W S, ell x d_v).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, _, d_k = k.shape
    d_v = v.shape[2]
    N = len(cu) - 1
    G = H_v // H_q
    out = np.zeros((T, H_v, d_v))
    final = np.zeros((N, H_v, d_k, d_v))
    inter = {}
    for n in range(N):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        L = t1 - t0
        for h in range(H_v):
            hq = h // G  # GVA: value head h reads query/key head floor(h / G)
            S = np.zeros((d_k, d_v)) if initial_state is None else np.array(initial_state[n, h], dtype=np.float64)
            recs = []
            n_chunks = -(-L // C)
            for c in range(n_chunks):
                a = t0 + c * C
                ell = min(C, L - c * C)
                Q = q[a:a + ell, hq, :]
                K = k[a:a + ell, hq, :]
                V = v[a:a + ell, h, :]
                gcum = np.cumsum(g[a:a + ell, h])  # inclusive, restarts per chunk
                Gam = np.diag(np.exp(gcum))
                Gin = np.diag(np.exp(-gcum))
                Bm = np.diag(beta[a:a + ell, h])
                I = np.eye(ell)
                A = np.linalg.inv(I + np.tril(Bm @ Gam @ K @ K.T @ Gin, -1))
                U = A @ Bm @ V
                W = A @ Bm @ Gam @ K
                X = U - W @ S
                O = scale * (Gam @ Q @ S + Gam @ np.tril(Q @ K.T) @ Gin @ X)
                out[a:a + ell, h, :] = O
                if keep_intermediates:
                    recs.append(dict(gc=gcum.copy(), A=A, W=W, U=U, h=S.copy(), X=X))
                gl = np.exp(gcum[-1])
                S = gl * S + gl * (K.T @ Gin @ X)
            final[n, h] = S
            if keep_intermediates:
                inter[(n, h)] = recs
    res = dict(out=out, final_state=final)
    if keep_intermediates:
        res["chunks"] = inter
    return res
