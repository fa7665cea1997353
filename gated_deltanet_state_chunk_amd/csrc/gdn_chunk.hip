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

// Fragment-order offsets (in elements) of the per-(chunk, value head) blocks
// written by recompute_w_u and read by chunk_state_h.  A fragment holds 8
// values per lane; lane = 16 a + r with r the row (A operand) and a the lane
// group; "perm32" slot 4 h + b stands for contraction index 16 h + 4 a + b.
//   W  (rows pos, contraction d_k): fragment (pos / 16, K-step), lane, slot
template <int D>
__host__ __device__ __forceinline__ int frag_w_offset(int pos_tile, int ks, int lane) {
    return ((pos_tile * (D / 32) + ks) * 64 + lane) * 8;
}
//   Kd^T (rows d_k, contraction pos): element (dk, pos) with pos a multiple of 4
__host__ __device__ __forceinline__ int frag_k_offset(int dk, int pos4) {
    const int m = dk >> 4, r = dk & 15, ks = pos4 >> 5, h = (pos4 >> 4) & 1, a = (pos4 >> 2) & 3;
    return ((m * 2 + ks) * 64 + 16 * a + r) * 8 + 4 * h;
}
//   U (accumulator order): column tile of d_v, row tile of pos, lane -> 4 rows
__host__ __device__ __forceinline__ int frag_u_offset(int col_tile, int pos_tile, int lane) {
    return ((col_tile * 4 + pos_tile) * 64 + lane) * 4;
}

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
//    W^T = (B Gamma K)^T A^T,  U = A (B V),  Kd^T = (diag(gamma_l / gamma_r) K)^T
//    (the keys of the state update, already carrying the decay to the end of
//    the chunk).  All three are written in the MFMA fragment order in which
//    chunk_state_h consumes them (frag_w / frag_k / frag_u below), so that
//    stage can copy each chunk's block into LDS with contiguous 1 KiB loads.
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
    __shared__ float s_sk[CHUNK], s_sv[CHUNK], s_kd[CHUNK];

    if (tid < CHUNK) {
        const size_t gi = (size_t)(cp.t0 + tid) * p.H_v + h;
        const float* gcb = p.gc + ((size_t)cp.ci * p.H_v + h) * CHUNK;
        const float b = tid < ell ? p.beta[gi] : 0.f;
        const float gcv = gcb[tid];
        s_sk[tid] = b * __expf(gcv);
        s_sv[tid] = b;
        s_kd[tid] = tid < ell ? __expf(gcb[ell - 1] - gcv) : 0.f;  // gamma_l / gamma_r
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
    constexpr int KS = D / 32;
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
            // lane: column pos = 16 nt + r16, rows d_k = 16 mt + 4 grp + i: in fragment
            // order this is fragment (pos tile nt, K-step mt / 2), same lane, slots 4 (mt % 2) + i
            store4(Wb + frag_w_offset<D>(nt, mt >> 1, lane) + 4 * (mt & 1), c[0], c[1], c[2], c[3]);
        }
    }
    // U tiles: rows pos, columns d_v (this wave's tiles).
    T* Ub = reinterpret_cast<T*>(p.Ut) + ((size_t)cp.ci * p.H_v + h) * D * CHUNK;
    (void)KS;
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
            // lane: column d_v = 16 nt + r16, rows pos = 16 mt + 4 grp + i (accumulator order)
            store4(Ub + frag_u_offset(nt, mt, lane), c[0], c[1], c[2], c[3]);
        }
    }
    // Decayed keys of the state update, transposed.
    {
        T* Kb = reinterpret_cast<T*>(p.Kt) + ((size_t)cp.ci * p.H_v + h) * D * CHUNK;
        for (int e = tid; e < D * (CHUNK / 4); e += 256) {
            const int dk = e / (CHUNK / 4), r4 = (e % (CHUNK / 4)) * 4;
            store4(Kb + frag_k_offset(dk, r4), s_kd[r4] * to_f32<T>(s_K[r4][dk]),
                   s_kd[r4 + 1] * to_f32<T>(s_K[r4 + 1][dk]), s_kd[r4 + 2] * to_f32<T>(s_K[r4 + 2][dk]),
                   s_kd[r4 + 3] * to_f32<T>(s_K[r4 + 3][dk]));
        }
    }
}

// ---------------------------------------------------------------------------
// 3. chunk_state_h: one workgroup per (sequence, value head, 16-column tile of
//    d_v), serial over the sequence's chunks; four compute waves (one per SIMD)
//    and one producer wave.
//
//    Compute waves.  The fp32 state slice S[:, tile] (d_k x 16) stays in MFMA
//    accumulators, split by rows over the waves.  Per chunk:
//      X = U - W S          wave w: positions 16w..16w+15, contraction over d_k
//      S = gamma_l S + Kd^T X   wave w: its rows of S, contraction over positions
//    The two products exchange bf16 copies of -S and X through LDS in MFMA
//    operand order (one 16-byte access per lane and fragment), two barriers a
//    chunk, and read their operands from the LDS stage of that chunk.
//
//    Producer wave.  Streams each chunk's W, Kd, U and gate blocks (stored by
//    recompute_w_u in exactly the LDS stage order) into a ring of stages with
//    direct global->LDS loads, NST - 1 chunks ahead, so the compute waves never
//    issue a global load: the per-chunk operands (about 34 KiB) would otherwise
//    stall their instruction stream on the CU's vector-memory path.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct StateStage {
    static constexpr int W_BYTES = CHUNK * D * (int)sizeof(T);
    static constexpr int K_BYTES = D * CHUNK * (int)sizeof(T);
    static constexpr int U_BYTES = 4 * 64 * 4 * (int)sizeof(T);  // one 16-column tile
    static constexpr int G_BYTES = CHUNK * 4;
    static constexpr int BYTES = W_BYTES + K_BYTES + U_BYTES + G_BYTES;
    static constexpr int NDMA = (W_BYTES + K_BYTES + U_BYTES) / 1024 + 1;  // loads per chunk
    static constexpr int EXCH = (D / 32 + 2) * 64 * 8 * (int)sizeof(T);    // -S and X exchange
    static constexpr int NST = (3 * BYTES + EXCH <= 150 * 1024 && NDMA <= 63) ? 3 : 2;
};

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// Wave-wide copy of 1 KiB (64 lanes x 16 B) from global `src` to LDS `dst`.
__device__ __forceinline__ void dma_1k(const char* src, char* dst, int lane) {
    __builtin_amdgcn_global_load_lds((gptr_t)(src + 16 * lane), (lptr_t)dst, 16, 0, 0);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <typename T, int D>
__device__ __forceinline__ void state_issue(char* stage, const ChunkParams& p, size_t ch, int tile, int lane) {
    using SS = StateStage<T, D>;
    constexpr int NT = D / 16;
    const char* wg = reinterpret_cast<const char*>(p.W) + ch * SS::W_BYTES;
    const char* kg = reinterpret_cast<const char*>(p.Kt) + ch * SS::K_BYTES;
    const char* ug = reinterpret_cast<const char*>(p.Ut) + (ch * NT + tile) * SS::U_BYTES;
#pragma unroll
    for (int j = 0; j < SS::W_BYTES / 1024; ++j) dma_1k(wg + 1024 * j, stage + 1024 * j, lane);
#pragma unroll
    for (int j = 0; j < SS::K_BYTES / 1024; ++j) dma_1k(kg + 1024 * j, stage + SS::W_BYTES + 1024 * j, lane);
#pragma unroll
    for (int j = 0; j < SS::U_BYTES / 1024; ++j)
        dma_1k(ug + 1024 * j, stage + SS::W_BYTES + SS::K_BYTES + 1024 * j, lane);
    __builtin_amdgcn_global_load_lds((gptr_t)(p.gc + ch * CHUNK + lane),
                                     (lptr_t)(stage + SS::W_BYTES + SS::K_BYTES + SS::U_BYTES), 4, 0, 0);
}

// Write a D tile's four values (rows 4 grp + i of one 16-row tile) into the
// perm32 fragment they belong to: even tile -> slots 0..3, odd -> slots 4..7.
template <typename T>
__device__ __forceinline__ void lds_put4(Frag<T>& f, int half, const f32x4& v, float s) {
    if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(&f) + 4 * half) = cvt4_bf16(v, s);
    } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(&f) + 4 * half) =
            make_float4(s * v[0], s * v[1], s * v[2], s * v[3]);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(320) void chunk_state_h_kernel(const ChunkParams p, int padded) {
    using SS = StateStage<T, D>;
    constexpr int NT = D / 16;   // column tiles of d_v per head
    constexpr int KS = D / 32;   // contraction steps over d_k
    constexpr int TPW = D / 64;  // S row tiles per compute wave
    constexpr int NST = SS::NST;
    const int wid = xcd_remap(blockIdx.x, padded);
    if (wid >= p.tab.num_seqs * p.H_v * NT) return;
    const int tile = wid % NT;
    const int u = wid / NT;
    const int h = u % p.H_v, n = u / p.H_v;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int col = 16 * tile + r16;
    const size_t state_off = ((size_t)(p.tab.seq_base + n) * p.H_v + h) * D * D;
    const int L_n = p.tab.cu[n + 1] - p.tab.cu[n];
    const int nch = p.tab.choff[n + 1] - p.tab.choff[n];
    const int c0 = p.tab.choff[n];

    __shared__ __attribute__((aligned(16))) char smem[NST * SS::BYTES + SS::EXCH];
    Frag<T>(*LS)[64] = reinterpret_cast<Frag<T>(*)[64]>(smem + NST * SS::BYTES);           // [KS][64]: -S
    Frag<T>(*LX)[64] = reinterpret_cast<Frag<T>(*)[64]>(smem + NST * SS::BYTES + KS * 64 * sizeof(Frag<T>));  // [2][64]: X

    if (w == 4) {
        // ---------------- producer ----------------
#pragma unroll
        for (int b = 0; b < NST - 1; ++b)
            if (b < nch) state_issue<T, D>(smem + b * SS::BYTES, p, (size_t)(c0 + b) * p.H_v + h, tile, lane);
        wait_vmcnt<0>();
        // The producer's barriers are plain s_barrier: a workgroup release fence
        // would wait for the direct-to-LDS loads just issued, and the whole point
        // is that they stay in flight.  Visibility is ensured explicitly: chunk c
        // is complete (vmcnt) before this wave arrives at B1(c).  The asm's memory
        // clobber keeps the compiler from moving loads across the barrier.
        for (int c = 0; c < nch; ++c) {
            asm volatile("s_barrier" ::: "memory");  // B1(c): stage c % NST is complete and visible
            const int cn = c + NST - 1;
            if (cn < nch) state_issue<T, D>(smem + (cn % NST) * SS::BYTES, p, (size_t)(c0 + cn) * p.H_v + h, tile, lane);
            asm volatile("s_barrier" ::: "memory");  // B2(c)
            // chunk c + 1 must be in LDS before B1(c + 1); the chunk issued above may stay in flight
            if (NST == 3 && cn < nch)
                wait_vmcnt<(NST == 3 ? SS::NDMA : 0)>();
            else
                wait_vmcnt<0>();
        }
        return;
    }

    // ---------------- compute waves ----------------
    f32x4 S[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int m = w * TPW + tt;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[tt][i] = p.s0 ? p.s0[state_off + (size_t)(16 * m + 4 * grp + i) * D + col] : 0.f;
        lds_put4(LS[m >> 1][lane], m & 1, S[tt], -1.f);
    }
    for (int c = 0; c < nch; ++c) {
        const int ci = c0 + c;
        const int ell = min(CHUNK, L_n - c * CHUNK);
        const size_t ch = (size_t)ci * p.H_v + h;
        const char* st = smem + (c % NST) * SS::BYTES;
        const Frag<T>* Wst = reinterpret_cast<const Frag<T>*>(st);
        const Frag<T>* Kst = reinterpret_cast<const Frag<T>*>(st + SS::W_BYTES);
        const Raw4<T>* Ust = reinterpret_cast<const Raw4<T>*>(st + SS::W_BYTES + SS::K_BYTES);
        const float* Gst = reinterpret_cast<const float*>(st + SS::W_BYTES + SS::K_BYTES + SS::U_BYTES);
        __syncthreads();  // B1(c): -S in LS, stage c ready
        Frag<T> wf[KS], sb[KS], kf[TPW][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            wf[ks] = Wst[(w * KS + ks) * 64 + lane];
            sb[ks] = LS[ks][lane];
        }
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) kf[tt][ks] = Kst[((w * TPW + tt) * 2 + ks) * 64 + lane];
        const Raw4<T> uf = Ust[w * 64 + lane];
        const float eg = __expf(Gst[ell - 1]);

        // h_c = S (this wave's rows), stored transposed [d_v][d_k]
        T* Hb = reinterpret_cast<T*>(p.Ht) + (ch * D + col) * D;
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
            store4(Hb + 16 * (w * TPW + tt) + 4 * grp, S[tt][0], S[tt][1], S[tt][2], S[tt][3]);
        // X = U - W S for positions 16 w .. 16 w + 15
        f32x4 X = raw4_to_f32(uf);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) X = mma(wf[ks], sb[ks], X);
        T* Xb = reinterpret_cast<T*>(p.Xt) + (ch * D + col) * CHUNK;
        store4(Xb + perm32(16 * w + 4 * grp), X[0], X[1], X[2], X[3]);
        lds_put4(LX[w >> 1][lane], w & 1, X, 1.f);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) S[tt] *= eg;
        __syncthreads();  // B2(c): all of X in LX
        const Frag<T> xb0 = LX[0][lane], xb1 = LX[1][lane];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            S[tt] = mma(kf[tt][0], xb0, S[tt]);
            S[tt] = mma(kf[tt][1], xb1, S[tt]);
        }
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int m = w * TPW + tt;
            lds_put4(LS[m >> 1][lane], m & 1, S[tt], -1.f);
        }
    }
    if (p.sfinal) {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int m = w * TPW + tt;
#pragma unroll
            for (int i = 0; i < 4; ++i) p.sfinal[state_off + (size_t)(16 * m + 4 * grp + i) * D + col] = S[tt][i];
        }
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
        hipLaunchKernelGGL((chunk_state_h_kernel<T, D>), dim3(grid_st), dim3(320), 0, stream, p, grid_st);
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
