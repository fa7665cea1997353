// Chunk-wise Gated DeltaNet prefill for gfx950.
//
// Four kernels, one per stage of the chunk form in "实验三：GDN Prefill 前向优化"
// (section "计算过程描述"):
//   1. kkt_solve     g^cumsum and A = (I + StrictLower(B Gamma K K^T Gamma^-1))^-1
//   2. recompute_w_u W = A B Gamma K, U = A B V
//   3. chunk_state_h S_{c+1} = gamma_l S_c + gamma_l K^T Gamma^-1 (U - W S_c), serial over chunks
//   4. chunk_output_o O = scale [Gamma Q S_c + Gamma Lower(Q K^T) Gamma^-1 (U - W S_c)]
// Stage names follow the Prefill-GDN kernel graph of the "Qwen3.5-397B-A17B"
// trace page (nodes chunk_gate_cumsum, chunk_kkt_solve, chunk_recompute_w_u,
// chunk_state_h, chunk_output_o), whose zero-init nodes are folded in here:
// every workspace entry and output row is written exactly once.
//
// Every ratio gamma_i / gamma_j is formed as exp(gc_i - gc_j) with i >= j, so
// nothing overflows however strong the decay (Gamma^-1 alone would).
// Positions past a tail chunk's valid length carry beta = 0 and zero K/V rows,
// which makes their rows of A (masked to zero), W, U and U - W S vanish.
#include "gdn_device.h"
#include "gdn_params.h"

namespace gdn {

namespace {

struct ChunkPos {
    int ci;   // global chunk index
    int n;    // sequence (index within the launch's table)
    int t0;   // first token
    int ell;  // valid length, 1..64
};

// Sequence owning global chunk ci: the largest n with choff[n] <= ci (empty
// sequences own no chunk and are skipped by taking the largest).
__device__ __forceinline__ ChunkPos locate_chunk(const SeqTable& tab, int ci) {
    int lo = 0, hi = tab.num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tab.choff[mid] <= ci)
            lo = mid;
        else
            hi = mid - 1;
    }
    ChunkPos c;
    c.ci = ci;
    c.n = lo;
    c.t0 = tab.cu[lo] + (ci - tab.choff[lo]) * CHUNK;
    c.ell = min(CHUNK, tab.cu[lo + 1] - c.t0);
    return c;
}

constexpr int LPAD = 65;  // fp32 64x64 LDS matrices, padded row

// acc += X[xr:xr+16, xc:xc+16] @ Y[yr:yr+16, yc:yc+16], fp32 operands in LDS,
// four v_mfma_f32_16x16x4_f32 (lane (m, a) supplies X[m][4s+a] and Y[4s+a][m]).
__device__ __forceinline__ f32x4 mm16_lds(const float (*X)[LPAD], int xr, int xc, const float (*Y)[LPAD], int yr,
                                          int yc, f32x4 acc, int r16, int grp) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const float a = X[xr + r16][xc + 4 * s + grp];
        const float b = Y[yr + 4 * s + grp][yc + r16];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    return acc;
}

// Store a D tile (lane: column r16, rows 4*grp + i) into an LDS matrix at (r0, c0), times s.
__device__ __forceinline__ void tile_to_lds(float (*M)[LPAD], int r0, int c0, const f32x4& t, float s, int r16,
                                            int grp) {
#pragma unroll
    for (int i = 0; i < 4; ++i) M[r0 + 4 * grp + i][c0 + r16] = s * t[i];
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. kkt_solve: one workgroup (4 waves) per (chunk, value head).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void kkt_solve_kernel(const ChunkParams p, int padded) {
    const int wid = xcd_remap(blockIdx.x, padded);
    if (wid >= p.tab.n_chunks * p.H_v) return;
    const int h = wid % p.H_v;
    const ChunkPos cp = locate_chunk(p.tab, p.tab.chunk_begin + wid / p.H_v);
    const int hq = h / p.G;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int ell = cp.ell;

    __shared__ float s_gc[CHUNK], s_beta[CHUNK];
    __shared__ float s_L[CHUNK][LPAD];
    __shared__ float s_A[CHUNK][LPAD];
    __shared__ float s_T[4][16][LPAD];

    // In-chunk inclusive cumsum of the log gate ("输入输出定义": restarts every chunk).
    if (w == 0) {
        const size_t gi = (size_t)(cp.t0 + lane) * p.H_v + h;
        float gv = lane < ell ? p.g[gi] : 0.f;
        const float bv = lane < ell ? p.beta[gi] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(gv, off, 64);
            if (lane >= off) gv += o;
        }
        s_gc[lane] = gv;
        s_beta[lane] = bv;
        p.gc[((size_t)cp.ci * p.H_v + h) * CHUNK + lane] = lane < ell ? gv : 0.f;
    }

    // K K^T: wave w forms row block w against all four column blocks.
    const T* kb = reinterpret_cast<const T*>(p.k) + (size_t)cp.t0 * p.H_q * D + (size_t)hq * D;
    const size_t kstride = (size_t)p.H_q * D;
    f32x4 acc[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) acc[J] = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        Frag<T> a;
        const int ra = 16 * w + r16;
        load8_masked(a, kb + (size_t)ra * kstride + 32 * ks + 8 * grp, ra < ell);
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            Frag<T> b;
            const int rb = 16 * J + r16;
            load8_masked(b, kb + (size_t)rb * kstride + 32 * ks + 8 * grp, rb < ell);
            acc[J] = mma(a, b, acc[J]);
        }
    }
    __syncthreads();
    // L_ij = beta_i exp(gc_i - gc_j) (k_i . k_j) for i > j; zero elsewhere.
#pragma unroll
    for (int J = 0; J < 4; ++J) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int i = 16 * w + 4 * grp + i4, j = 16 * J + r16;
            s_L[i][j] = (i > j) ? s_beta[i] * __expf(s_gc[i] - s_gc[j]) * acc[J][i4] : 0.f;
        }
    }
    __syncthreads();

    // (I + L)^-1 by blocks of 16.  Diagonal blocks: forward substitution, lane owns column c.
    {
        const int base = 16 * w, c = r16;
        float a[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < r; ++kk) s -= s_L[base + r][base + kk] * a[kk];
            a[r] = s;
        }
        if (grp == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s_A[base + r][base + c] = a[r];
        }
    }
    __syncthreads();
    // 32x32 diagonal blocks: A10 = -A11 L10 A00 (wave 0), A32 = -A33 L32 A22 (wave 1).
    if (w < 2) {
        const int o = 32 * w;
        const f32x4 t = mm16_lds(s_L, o + 16, o, s_A, o, o, zero4(), r16, grp);
        tile_to_lds(s_T[w], 0, 0, t, 1.f, r16, grp);
    }
    __syncthreads();
    if (w < 2) {
        const int o = 32 * w;
        const f32x4 t = mm16_lds(s_A, o + 16, o + 16, s_T[w], 0, 0, zero4(), r16, grp);
        tile_to_lds(s_A, o + 16, o, t, -1.f, r16, grp);
    }
    __syncthreads();
    // Lower-left 32x32 block: A_LL = -A_hi (L_LL A_lo).  Wave w owns block (I, J) =
    // (2 + w/2, w%2); first T_IJ = sum_{K=J..1} L_IK A_KJ ...
    {
        const int I = 2 + (w >> 1), J = w & 1;
        f32x4 t = zero4();
        for (int K = J; K <= 1; ++K) t = mm16_lds(s_L, 16 * I, 16 * K, s_A, 16 * K, 16 * J, t, r16, grp);
        tile_to_lds(s_T[w], 0, 0, t, 1.f, r16, grp);
    }
    __syncthreads();
    // ... then A_IJ = -sum_{K=2..I} A_IK T_KJ (T_KJ sits in s_T[2*(K-2) + J]).
    {
        const int I = 2 + (w >> 1), J = w & 1;
        f32x4 t = zero4();
        for (int K = 2; K <= I; ++K) t = mm16_lds(s_A, 16 * I, 16 * K, s_T[2 * (K - 2) + J], 0, 0, t, r16, grp);
        tile_to_lds(s_A, 16 * I, 16 * J, t, -1.f, r16, grp);
    }
    __syncthreads();

    // Write A, zero outside the valid lower triangle: thread -> row tid/4, 16 columns.
    {
        T* Ab = reinterpret_cast<T*>(p.A) + ((size_t)cp.ci * p.H_v + h) * CHUNK * CHUNK;
        const int i = tid >> 2, j0 = (tid & 3) * 16;
#pragma unroll
        for (int j4 = 0; j4 < 16; j4 += 4) {
            float v4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = j0 + j4 + e;
                v4[e] = (j <= i && i < ell) ? s_A[i][j] : 0.f;
            }
            store4(Ab + (size_t)i * CHUNK + j0 + j4, v4[0], v4[1], v4[2], v4[3]);
        }
    }
}

// ---------------------------------------------------------------------------
// 2. recompute_w_u: one workgroup per (chunk, value head).
//    W^T = (B Gamma K)^T A^T  -> W stored [pos][perm32(d_k)]
//    U   = A (B V)            -> Ut stored [d_v][pos]
//    Kt  = K^T                -> [d_k][perm32(pos)], written once per key head
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void recompute_w_u_kernel(const ChunkParams p, int padded) {
    const int wid = xcd_remap(blockIdx.x, padded);
    if (wid >= p.tab.n_chunks * p.H_v) return;
    const int h = wid % p.H_v;
    const ChunkPos cp = locate_chunk(p.tab, p.tab.chunk_begin + wid / p.H_v);
    const int hq = h / p.G;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int ell = cp.ell;
    constexpr int SP = D + 2;  // padded LDS row

    __shared__ T s_K[CHUNK][SP];
    __shared__ T s_V[CHUNK][SP];
    __shared__ float s_sk[CHUNK], s_sv[CHUNK];

    if (tid < CHUNK) {
        const size_t gi = (size_t)(cp.t0 + tid) * p.H_v + h;
        const float b = tid < ell ? p.beta[gi] : 0.f;
        const float gcv = p.gc[((size_t)cp.ci * p.H_v + h) * CHUNK + tid];
        s_sk[tid] = b * __expf(gcv);
        s_sv[tid] = b;
    }
    // Stage the chunk's K and V rows (zeros past the valid length).
    {
        const T* kb = reinterpret_cast<const T*>(p.k) + (size_t)cp.t0 * p.H_q * D + (size_t)hq * D;
        const T* vb = reinterpret_cast<const T*>(p.v) + (size_t)cp.t0 * p.H_v * D + (size_t)h * D;
        constexpr int PER_ROW = D / 4;  // 4-element groups per row
        for (int e = tid; e < CHUNK * PER_ROW; e += 256) {
            const int r = e / PER_ROW, c4 = (e % PER_ROW) * 4;
            float k0 = 0.f, k1 = 0.f, k2 = 0.f, k3 = 0.f, v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
            if (r < ell) {
                load4(kb + (size_t)r * p.H_q * D + c4, k0, k1, k2, k3);
                load4(vb + (size_t)r * p.H_v * D + c4, v0, v1, v2, v3);
            }
            s_K[r][c4 + 0] = from_f32<T>(k0);
            s_K[r][c4 + 1] = from_f32<T>(k1);
            s_K[r][c4 + 2] = from_f32<T>(k2);
            s_K[r][c4 + 3] = from_f32<T>(k3);
            s_V[r][c4 + 0] = from_f32<T>(v0);
            s_V[r][c4 + 1] = from_f32<T>(v1);
            s_V[r][c4 + 2] = from_f32<T>(v2);
            s_V[r][c4 + 3] = from_f32<T>(v3);
        }
    }
    __syncthreads();

    // Fragments of A (rows pos, contiguous columns), shared by both products:
    // Af[mt][ks] is the A operand of U = A (B V) for row tile mt and the B
    // operand of W^T = (B Gamma K)^T A^T for column tile mt.
    const T* Ab = reinterpret_cast<const T*>(p.A) + ((size_t)cp.ci * p.H_v + h) * CHUNK * CHUNK;
    Frag<T> Af[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) load8(Af[mt][ks], Ab + (size_t)(16 * mt + r16) * CHUNK + 32 * ks + 8 * grp);

    constexpr int TPW = D / 64;  // 16-wide tiles of d_k (or d_v) per wave
    // W^T tiles: rows d_k (this wave's tiles), columns pos.  A is lower triangular,
    // so column tile nt only needs contraction steps ks with 32 ks <= 16 nt + 15.
    T* Wb = reinterpret_cast<T*>(p.W) + ((size_t)cp.ci * p.H_v + h) * CHUNK * D;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int mt = w * TPW + tt;
        const int dk = 16 * mt + r16;
        Frag<T> kf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 32 * ks + 8 * grp + j;
                frag_set(kf[ks], j, s_sk[r] * to_f32<T>(s_K[r][dk]));
            }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            f32x4 c = zero4();
            c = mma(kf[0], Af[nt][0], c);
            if (nt >= 2) c = mma(kf[1], Af[nt][1], c);
            // lane: column pos = 16 nt + r16, rows d_k = 16 mt + 4 grp + i
            const int pos = 16 * nt + r16;
            store4(Wb + (size_t)pos * D + perm32(16 * mt + 4 * grp), c[0], c[1], c[2], c[3]);
        }
    }
    // U tiles: rows pos, columns d_v (this wave's tiles).
    T* Ub = reinterpret_cast<T*>(p.Ut) + ((size_t)cp.ci * p.H_v + h) * D * CHUNK;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int nt = w * TPW + tt;
        const int dv = 16 * nt + r16;
        Frag<T> vf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 32 * ks + 8 * grp + j;
                frag_set(vf[ks], j, s_sv[r] * to_f32<T>(s_V[r][dv]));
            }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x4 c = zero4();
            c = mma(Af[mt][0], vf[0], c);
            if (mt >= 2) c = mma(Af[mt][1], vf[1], c);
            // lane: column d_v, rows pos = 16 mt + 4 grp + i
            store4(Ub + (size_t)dv * CHUNK + 16 * mt + 4 * grp, c[0], c[1], c[2], c[3]);
        }
    }
    // K^T of the chunk, once per key head.
    if (h % p.G == 0) {
        T* Kb = reinterpret_cast<T*>(p.Kt) + ((size_t)cp.ci * p.H_q + hq) * D * CHUNK;
        for (int e = tid; e < D * (CHUNK / 4); e += 256) {
            const int dk = e / (CHUNK / 4), r4 = (e % (CHUNK / 4)) * 4;
            store4(Kb + (size_t)dk * CHUNK + perm32(r4), to_f32<T>(s_K[r4][dk]), to_f32<T>(s_K[r4 + 1][dk]),
                   to_f32<T>(s_K[r4 + 2][dk]), to_f32<T>(s_K[r4 + 3][dk]));
        }
    }
}

// ---------------------------------------------------------------------------
// 3. chunk_state_h: one wave per (sequence, value head, 16-column tile of d_v),
//    serial over the sequence's chunks.  The fp32 state slice S[:, tile] lives
//    in MFMA accumulators for the whole sequence; its bf16/fp32 copy feeds the
//    next product directly through the perm32 fragment convention, so the
//    serial chain has no LDS traffic and no barrier.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void chunk_state_h_kernel(const ChunkParams p, int padded) {
    constexpr int NT = D / 16;  // d_k row tiles of S (= d_v column tiles per head)
    constexpr int KS = D / 32;  // contraction steps over d_k
    const int wid = xcd_remap(blockIdx.x, padded);
    if (wid >= p.tab.num_seqs * p.H_v * NT) return;
    const int tile = wid % NT;
    const int u = wid / NT;
    const int h = u % p.H_v, n = u / p.H_v;
    const int hq = h / p.G;
    const int lane = threadIdx.x, r16 = lane & 15, grp = lane >> 4;
    const int col = 16 * tile + r16;
    const size_t state_off = ((size_t)(p.tab.seq_base + n) * p.H_v + h) * D * D;

    f32x4 S[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[mt][i] = p.s0 ? p.s0[state_off + (size_t)(16 * mt + 4 * grp + i) * D + col] : 0.f;
    }

    const int L = p.tab.cu[n + 1] - p.tab.cu[n];
    const int nch = p.tab.choff[n + 1] - p.tab.choff[n];
    for (int c = 0; c < nch; ++c) {
        const int ci = p.tab.choff[n] + c;
        const int ell = min(CHUNK, L - c * CHUNK);
        const size_t ch = (size_t)ci * p.H_v + h;

        // Chunk-start state h_c, stored transposed [d_v][d_k].
        T* Hb = reinterpret_cast<T*>(p.Ht) + (ch * D + col) * D;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) store4(Hb + 16 * mt + 4 * grp, S[mt][0], S[mt][1], S[mt][2], S[mt][3]);

        // Operands of this chunk.
        const T* Wb = reinterpret_cast<const T*>(p.W) + ch * CHUNK * D;
        const T* Kb = reinterpret_cast<const T*>(p.Kt) + ((size_t)ci * p.H_q + hq) * D * CHUNK;
        const T* Ub = reinterpret_cast<const T*>(p.Ut) + (ch * D + col) * CHUNK;
        const float* gcb = p.gc + ch * CHUNK;
        Frag<T> Wf[4][KS];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) load8(Wf[mt][ks], Wb + (size_t)(16 * mt + r16) * D + 32 * ks + 8 * grp);
        f32x4 X[4];
        float gcv[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            float u0, u1, u2, u3;
            load4(Ub + 16 * mt + 4 * grp, u0, u1, u2, u3);
            X[mt] = f32x4{u0, u1, u2, u3};
            const float4 gg = *reinterpret_cast<const float4*>(gcb + 16 * mt + 4 * grp);
            gcv[mt][0] = gg.x; gcv[mt][1] = gg.y; gcv[mt][2] = gg.z; gcv[mt][3] = gg.w;
        }
        const float gl = gcb[ell - 1];

        // X = U - W S.
        Frag<T> Sb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) Sb[ks] = pack_perm32<T>(S[2 * ks], S[2 * ks + 1], -1.f);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) X[mt] = mma(Wf[mt][ks], Sb[ks], X[mt]);

        // Store (U - W S)^T with perm32 positions; zero past the valid length.
        T* Xb = reinterpret_cast<T*>(p.Xt) + (ch * D + col) * CHUNK;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * mt + 4 * grp + i >= ell) X[mt][i] = 0.f;
            store4(Xb + perm32(16 * mt + 4 * grp), X[mt][0], X[mt][1], X[mt][2], X[mt][3]);
        }

        // S <- gamma_l S + K^T diag(gamma_l / gamma_r) (U - W S).
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) X[mt][i] *= __expf(gl - gcv[mt][i]);
        Frag<T> Xf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) Xf[ks] = pack_perm32<T>(X[2 * ks], X[2 * ks + 1], 1.f);
        const float eg = __expf(gl);
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
            S[mt] *= eg;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                Frag<T> kf;
                load8(kf, Kb + (size_t)(16 * mt + r16) * CHUNK + 32 * ks + 8 * grp);
                S[mt] = mma(kf, Xf[ks], S[mt]);
            }
        }
    }
    if (p.sfinal) {
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) p.sfinal[state_off + (size_t)(16 * mt + 4 * grp + i) * D + col] = S[mt][i];
    }
}

// ---------------------------------------------------------------------------
// 4. chunk_output_o: one workgroup per (chunk, value head).  Computes
//    O^T = scale [ (H^T Q^T) diag(gamma) + (U - W S)^T P^T ],
//    P^T[j][i] = (k_j . q_i) exp(gc_i - gc_j) for j <= i  (Lower keeps the diagonal).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void chunk_output_o_kernel(const ChunkParams p, int padded) {
    const int wid = xcd_remap(blockIdx.x, padded);
    if (wid >= p.tab.n_chunks * p.H_v) return;
    const int h = wid % p.H_v;
    const ChunkPos cp = locate_chunk(p.tab, p.tab.chunk_begin + wid / p.H_v);
    const int hq = h / p.G;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int ell = cp.ell;
    constexpr int KS = D / 32;
    constexpr int TPW = D / 64;
    constexpr int PP = CHUNK + 2;

    __shared__ float s_gc[CHUNK];
    __shared__ T s_Pt[CHUNK][PP];  // P^T [pos'][pos]

    const size_t ch = (size_t)cp.ci * p.H_v + h;
    if (tid < CHUNK) s_gc[tid] = p.gc[ch * CHUNK + tid];

    const T* qb = reinterpret_cast<const T*>(p.q) + (size_t)cp.t0 * p.H_q * D + (size_t)hq * D;
    const T* kb = reinterpret_cast<const T*>(p.k) + (size_t)cp.t0 * p.H_q * D + (size_t)hq * D;
    const size_t qstride = (size_t)p.H_q * D;

    // Q fragments (B operand, rows pos): Qf[nt][ks].
    Frag<T> Qf[4][KS];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int r = 16 * nt + r16;
            load8_masked(Qf[nt][ks], qb + (size_t)r * qstride + 32 * ks + 8 * grp, r < ell);
        }
    __syncthreads();  // s_gc

    // P^T tiles (I, J = w) for I <= w: rows pos' (keys), columns pos (queries).
    Frag<T> qw[KS];  // query fragments of column tile w (runtime index: load, do not index Qf)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int r = 16 * w + r16;
        load8_masked(qw[ks], qb + (size_t)r * qstride + 32 * ks + 8 * grp, r < ell);
    }
    for (int I = 0; I < 4; ++I) {
        f32x4 c = zero4();
        if (I <= w) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Frag<T> kf;
                const int r = 16 * I + r16;
                load8_masked(kf, kb + (size_t)r * qstride + 32 * ks + 8 * grp, r < ell);
                c = mma(kf, qw[ks], c);
            }
        }
        const int pos = 16 * w + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pj = 16 * I + 4 * grp + i;
            const float val = (pj <= pos && pos < ell) ? c[i] * __expf(s_gc[pos] - s_gc[pj]) : 0.f;
            s_Pt[pj][pos] = from_f32<T>(val);
        }
    }
    __syncthreads();

    // Output tiles: rows d_v (this wave's tiles), columns pos.
    const T* Hb = reinterpret_cast<const T*>(p.Ht) + ch * D * D;
    const T* Xb = reinterpret_cast<const T*>(p.Xt) + ch * D * CHUNK;
    T* ob = reinterpret_cast<T*>(p.out) + (size_t)cp.t0 * p.H_v * D + (size_t)h * D;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int mt = w * TPW + tt;
        const int dv = 16 * mt + r16;
        Frag<T> hf[KS], xf[2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load8(hf[ks], Hb + (size_t)dv * D + 32 * ks + 8 * grp);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) load8(xf[ks], Xb + (size_t)dv * CHUNK + 32 * ks + 8 * grp);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            f32x4 inter = zero4(), intra = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) inter = mma(hf[ks], Qf[nt][ks], inter);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (32 * ks > 16 * nt + 15) continue;  // P^T rows all beyond this column tile
                Frag<T> pf;  // perm32 slots: pos' = 32 ks + 16 hh + 4 grp + b
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int b = 0; b < 4; ++b) pf.v[4 * hh + b] = s_Pt[32 * ks + 16 * hh + 4 * grp + b][16 * nt + r16];
                intra = mma(xf[ks], pf, intra);
            }
            const int pos = 16 * nt + r16;
            if (pos < ell) {
                const float eg = __expf(s_gc[pos]);
                float o4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o4[i] = p.scale * (eg * inter[i] + intra[i]);
                store4(ob + (size_t)pos * p.H_v * D + 16 * mt + 4 * grp, o4[0], o4[1], o4[2], o4[3]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Pipeline launcher: the four stages in stream order.
// ---------------------------------------------------------------------------
static inline int pad8(int x) { return (x + 7) & ~7; }

template <typename T, int D>
hipError_t launch_chunk_pipeline(const ChunkParams& p, hipStream_t stream, hipEvent_t const* events) {
    const int work_ch = p.tab.n_chunks * p.H_v;
    const int grid_ch = pad8(work_ch);
    const int work_st = p.tab.num_seqs * p.H_v * (D / 16);
    const int grid_st = pad8(work_st);
    auto mark = [&](int i) {
        if (events) (void)hipEventRecord(events[i], stream);
    };
    mark(0);
    if (work_ch > 0) hipLaunchKernelGGL((kkt_solve_kernel<T, D>), dim3(grid_ch), dim3(256), 0, stream, p, grid_ch);
    mark(1);
    if (work_ch > 0)
        hipLaunchKernelGGL((recompute_w_u_kernel<T, D>), dim3(grid_ch), dim3(256), 0, stream, p, grid_ch);
    mark(2);
    if (work_st > 0)
        hipLaunchKernelGGL((chunk_state_h_kernel<T, D>), dim3(grid_st), dim3(64), 0, stream, p, grid_st);
    mark(3);
    if (work_ch > 0)
        hipLaunchKernelGGL((chunk_output_o_kernel<T, D>), dim3(grid_ch), dim3(256), 0, stream, p, grid_ch);
    mark(4);
    return hipGetLastError();
}

template hipError_t launch_chunk_pipeline<bf16, 128>(const ChunkParams&, hipStream_t, hipEvent_t const*);
template hipError_t launch_chunk_pipeline<bf16, 64>(const ChunkParams&, hipStream_t, hipEvent_t const*);
template hipError_t launch_chunk_pipeline<float, 128>(const ChunkParams&, hipStream_t, hipEvent_t const*);
template hipError_t launch_chunk_pipeline<float, 64>(const ChunkParams&, hipStream_t, hipEvent_t const*);

}  // namespace gdn
