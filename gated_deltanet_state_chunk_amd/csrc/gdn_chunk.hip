// Chunk-wise Gated DeltaNet prefill for gfx950.
//
// The four stages of the chunk form in "实验三：GDN Prefill 前向优化" (section
// "计算过程描述") in three kernels:
//   1. chunk_prep     g^cumsum, A = (I + StrictLower(B Gamma K K^T Gamma^-1))^-1,
//                     W = A B Gamma K, U = A B V          (stages 1 and 2)
//   2. chunk_state_h  S_{c+1} = gamma_l S_c + gamma_l K^T Gamma^-1 (U - W S_c), serial over chunks
//   3. chunk_output_o O = scale [Gamma Q S_c + Gamma Lower(Q K^T) Gamma^-1 (U - W S_c)]
// The Prefill-GDN kernel graph of the "Qwen3.5-397B-A17B" trace page runs the
// first kernel as three (chunk_gate_cumsum, chunk_kkt_solve,
// chunk_recompute_w_u); here they share one pass over the chunk's keys, which
// saves re-reading K and the round trip of A.  Its zero-init nodes are folded
// in: every workspace entry and output row is written exactly once.
//
// Every ratio gamma_i / gamma_j is formed as exp(gc_i - gc_j) with i >= j, so
// nothing overflows however strong the decay (Gamma^-1 alone would).
// Positions past a tail chunk's valid length carry beta = 0 and zero K/V rows,
// which makes their rows of A (masked to zero), W, U and U - W S vanish.
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

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

// The chunks of the sequences of one state-scan bin (order[kb .. ke) of the
// launch table), sequence after sequence, empty sequences skipped.  All its
// values are uniform across a workgroup.
struct BinCursor {
    const SeqTable* tab;
    int k, ke;      // position in order[], end of the bin
    int n, c, nch;  // sequence, chunk within it, its chunk count
    int c0, t0, L;  // its first global chunk, first token and length
    __device__ void at_seq() {
        n = tab->order[k];
        c = 0;
        c0 = tab->choff[n];
        nch = tab->choff[n + 1] - c0;
        t0 = tab->cu[n];
        L = tab->cu[n + 1] - t0;
    }
    __device__ void skip_empty() {
        while (k < ke && nch == 0)
            if (++k < ke) at_seq();
    }
    __device__ void begin(const SeqTable& t, int kb, int kend) {
        tab = &t;
        k = kb;
        ke = kend;
        nch = 0;
        if (k < ke) {
            at_seq();
            skip_empty();
        }
    }
    __device__ bool valid() const { return k < ke; }
    __device__ void next() {
        if (++c == nch && ++k < ke) {
            at_seq();
            skip_empty();
        }
    }
    __device__ int ci() const { return c0 + c; }                      // global chunk index
    __device__ int ell() const { return min(CHUNK, L - c * CHUNK); }  // valid length
    __device__ int token() const { return t0 + c * CHUNK; }           // first token
    __device__ bool last() const { return c + 1 == nch; }
};

// acc += X[0:16, 0:16] @ Y[0:16, 0:16] for fp32 blocks in LDS with row strides
// XS and YS: four v_mfma_f32_16x16x4_f32 (lane (m, a) supplies X[m][4s+a] and Y[4s+a][m]).
template <int XS, int YS>
__device__ __forceinline__ f32x4 mm16_lds(const float* X, const float* Y, f32x4 acc, int r16, int grp) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const float a = X[r16 * XS + 4 * s + grp];
        const float b = Y[(4 * s + grp) * YS + r16];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    return acc;
}

// Store a D tile (lane: column r16, rows 4*grp + i) into an LDS block with row stride MS, times s.
template <int MS>
__device__ __forceinline__ void tile_to_lds(float* M, const f32x4& t, float s, int r16, int grp) {
#pragma unroll
    for (int i = 0; i < 4; ++i) M[(4 * grp + i) * MS + r16] = s * t[i];
}

}  // namespace

// Fragment-order offsets (in elements) of the per-(chunk, value head) blocks
// written by chunk_prep and read by chunk_state_h.  A fragment holds 8
// values per lane; lane = 16 a + r with r the row (A operand) and a the lane
// group; "perm32" slot 4 h + b stands for contraction index 16 h + 4 a + b.
//   W  (rows pos, contraction d_k): fragment (pos / 16, K-step), lane, slot
template <int D>
__host__ __device__ __forceinline__ int frag_w_offset(int pos_tile, int ks, int lane) {
    return ((pos_tile * (D / 32) + ks) * 64 + lane) * 8;
}
//   U (accumulator order): column tile of d_v, pair of row tiles of pos, lane ->
//   8 values, the 4 rows of the even tile then the 4 of the odd one
__host__ __device__ __forceinline__ int frag_u_offset(int col_tile, int pos_pair, int lane) {
    return ((col_tile * 2 + pos_pair) * 64 + lane) * 8;
}

// Permutation of the 16-byte pieces of K row `row` in Kc and in a state-scan
// stage: piece i is stored at i ^ kswz(row), so that the column reads of the
// state update hit distinct LDS banks.  bf16: the 32-byte window of 16
// columns that one transposed read covers moves with row % (pieces / 2);
// fp32: the 64-byte window moves with (row / 4) % (pieces / 4), the rows 4
// apart that one scalar column read touches.
template <typename T, int D>
__host__ __device__ constexpr int kswz(int row) {
    constexpr int CPR = D * (int)sizeof(T) / 16;
    return sizeof(T) == 2 ? (row & (CPR / 2 - 1)) * 2 : ((row >> 2) & (CPR / 4 - 1)) * 4;
}


// P, the masked and decayed Q K^T of a (chunk, value head), is kept as the six
// B-operand fragments of X^T P^T its query tiles need: (tile, K-step) =
// (0,0), (1,0), (2,0), (2,1), (3,0), (3,1) (query tiles 0 and 1 see keys < 32 only).
constexpr int P_FRAGS = 6;

// ---------------------------------------------------------------------------
// 1. chunk_prep: one workgroup (4 waves) per (chunk, value head); the first
//    stages of the chunk form in one pass over the chunk's keys:
//      gc = in-chunk inclusive cumsum of g          ("输入输出定义")
//      L  = StrictLower(B Gamma K K^T Gamma^-1),  A = (I + L)^-1   (fp32)
//    and the per-chunk operands of the state scan: the six fragments of A it
//    multiplies B (V - Gamma K S) by, the gate block (gc, kf = gamma_l / gamma,
//    beta and beta gamma per position), the key rows (Kc, once per key head)
//    and, for bf16, P = masked, decayed Q K^T.  The scan never sees W or U:
//    U - W S = A B V - A B Gamma K S = A B (V - Gamma K S), so it forms X from
//    A and the raw K and V rows (section "计算过程描述" gives U and W as
//    A B V and A B Gamma K; the product is only regrouped).  W and U are
//    still formed, from the same A, when the caller asks for them
//    (inspection), and A itself under keep_A.
// ---------------------------------------------------------------------------
// Lower-triangular 64x64 fp32 matrices are kept as their ten 16x16 blocks
// (I >= J), block (I, J) at index I (I + 1) / 2 + J, rows padded to BS floats.
constexpr int BS = 20;
constexpr int BLK = 16 * BS;
__host__ __device__ constexpr int blk(int I, int J) { return (I * (I + 1) / 2 + J) * BLK; }

// A (lower triangular) as the A operand of X = A (B Y) in the state scan: the
// fragments (row tile t, K-step s) with 32 s <= 16 t + 15, in the order of
// P_FRAGS, lane 16 a + r, slot 4 h + b holding A[16 t + r][32 s + 16 h + 4 a + b]
// (perm32: the B operand B Y is two stacked accumulator tiles).
constexpr int A_FRAGS = 6;
__host__ __device__ constexpr int a_frag_first(int t) { return t < 2 ? t : 2 * t - 2; }

template <typename T, int D>
struct PrepLds {
    static constexpr int KP = D + 32 / (int)sizeof(T);  // padded row (32 bytes: the transposed column reads hit distinct banks)
    T K[CHUNK][KP];
    union {
        struct {
            // Strictly lower part of B Gamma K K^T Gamma^-1, overwritten block by
            // block with (I + L)^-1 as the solve finishes with each L block.
            float LA[10 * BLK];
            float Tm[4 * BLK];  // products of the block solve
        } sv;                   // during the solve
        T V[CHUNK][KP];         // W and U for inspection: after it (once A is in registers)
    } u;
    float gc[CHUNK], beta[CHUNK], sk[CHUNK], svb[CHUNK], kd[CHUNK];
};

// DEV: the sequence table is read from device memory (p.dtab) instead of the
// kernel arguments (same for the two kernels below).  WU: also form W and U
// (a separate instantiation, so that the inspection path's registers do not
// weigh on the hot one).
template <typename T, int D, bool DEV, bool WU>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 4 : 2) void chunk_prep_kernel(const ChunkParams p, int padded) {
    using PL = PrepLds<T, D>;
    using PT = ProdT<T>;  // element type of the A fragments (and of the W and U products)
    constexpr int VEC = 16 / (int)sizeof(T);                  // elements per 16-byte access
    constexpr int NV = CHUNK * D / VEC / 256;                 // 16-byte pieces per thread
    const SeqTable& tab = DEV ? *p.dtab : p.tab;
    const int work = tab.n_chunks * p.H_v;
    if constexpr (DEV) padded = (work + 7) & ~7;  // the grid was sized by a bound
    // Items (chunk, value head) of this workgroup: virtual indices blockIdx.x,
    // blockIdx.x + gridDim.x, ... mapped XCD-aware (gridDim.x is a multiple of 8,
    // so every item of a workgroup stays on its XCD).  The next item's K and
    // gate rows are loaded into registers as soon as this item's are staged, so
    // they land while K K^T, the solve and P are formed.
    int v = blockIdx.x;
    if (v >= padded) return;
    int wid = xcd_remap(v, padded);
    if (wid >= work) return;  // padding items come last, so all later ones are padding too

    __shared__ __attribute__((aligned(16))) PL s;
    float* const Ls = s.u.sv.LA;
    float* const Tm = s.u.sv.Tm;
    float* const As = s.u.sv.LA;  // block (I, J) of A replaces block (I, J) of L

    // Rows of K (zero past the valid length) and wave 0's gate inputs, in
    // registers; with W and U also the rows of V (fetched at the start of their
    // own item: they are not read before the solve is done).
    float4 kreg[NV], vreg[WU ? NV : 1];
    float graw = 0.f, braw = 0.f;
    auto load_k = [&](int it) {
        const int tid = threadIdx.x, lane = tid & 63;
        const int hh = it % p.H_v;
        const ChunkPos c = locate_chunk(tab, tab.chunk_begin + it / p.H_v);
        const T* kb = reinterpret_cast<const T*>(p.k) + (size_t)c.t0 * p.H_q * D + (size_t)(hh / p.G) * D;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = tid + 256 * j, r = e / (D / VEC), cc = (e % (D / VEC)) * VEC;
            kreg[j] = r < c.ell ? *reinterpret_cast<const float4*>(kb + (size_t)r * p.H_q * D + cc)
                                : make_float4(0, 0, 0, 0);
        }
        if (tid < 64) {
            const size_t gi = (size_t)(c.t0 + lane) * p.H_v + hh;
            if (p.fa) {  // raw gate inputs (front end)
                graw = lane < c.ell ? to_f32<T>(reinterpret_cast<const T*>(p.fa)[gi]) : 0.f;
                braw = lane < c.ell ? to_f32<T>(reinterpret_cast<const T*>(p.fb)[gi]) : 0.f;
            } else {
                graw = lane < c.ell ? p.g[gi] : 0.f;
                braw = lane < c.ell ? p.beta[gi] : 0.f;
            }
        }
    };
    load_k(wid);

    for (;;) {
    // Thread indices re-read per item: the empty asm hides that they do not change,
    // so the address arithmetic of the body is not hoisted out of the loop (where it
    // would stay live in registers across the whole item).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, grp = lane >> 4;
    const int h = wid % p.H_v;
    const ChunkPos cp = locate_chunk(tab, tab.chunk_begin + wid / p.H_v);
    const int ell = cp.ell;
    const size_t ch = (size_t)cp.ci * p.H_v + h;

    if constexpr (WU) {  // V rows into registers (staged in LDS after the solve)
        const T* vb = reinterpret_cast<const T*>(p.v) + (size_t)cp.t0 * p.H_v * D + (size_t)h * D;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = tid + 256 * j, r = e / (D / VEC), c = (e % (D / VEC)) * VEC;
            vreg[j] = r < ell ? *reinterpret_cast<const float4*>(vb + (size_t)r * p.H_v * D + c)
                              : make_float4(0, 0, 0, 0);
        }
    }
    // Query fragments of this wave's 16 positions for P (bf16): rows 16 w + r16,
    // contraction indices 32 ks + 8 grp .. + 7 (zero past the valid length).
    // Loaded here, used after the solve, so the load latency overlaps K K^T
    // and the solve.
    Frag<T> qw[D / 32];
    if constexpr (sizeof(T) == 2) {
        if (p.Pf) {
            const int row = 16 * w + r16;
            const T* qb = reinterpret_cast<const T*>(p.q) + ((size_t)(cp.t0 + row) * p.H_q + h / p.G) * D + 8 * grp;
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) load8_masked(qw[ks], qb + 32 * ks, row < ell);
        }
    }
    // With the front end, each K row is L2-normalised on the way (rows past the
    // valid length are zero and stay zero).  The first value head of each key
    // head also writes the rows to Kc, the state scan's copy of the chunk's keys
    // (contiguous, 16-byte pieces in the stage order of kswz).
    const bool write_kc = h % p.G == 0;
    T* Kcb = reinterpret_cast<T*>(p.Kc) + ((size_t)cp.ci * p.H_q + h / p.G) * CHUNK * D;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int e = tid + 256 * j, r = e / (D / VEC), c = (e % (D / VEC)) * VEC;
        const float4 kv = p.fa ? l2norm_piece<T, D>(kreg[j]) : kreg[j];
        *reinterpret_cast<float4*>(&s.K[r][c]) = kv;
        if (write_kc) *reinterpret_cast<float4*>(Kcb + r * D + VEC * ((c / VEC) ^ kswz<T, D>(r))) = kv;
    }
    // In-chunk inclusive cumsum of the log gate (front end: g and beta from the
    // raw inputs first), and the chunk's gate block for the state scan: gc, kf =
    // gamma_l / gamma, beta and beta gamma, all zero past the valid length.
    if (w == 0) {
        float gv = graw, bv = braw;
        if (p.fa) {
            gv = lane < ell ? front_gate(gv, p.A_log[h], p.dt_bias[h]) : 0.f;
            bv = lane < ell ? front_beta<T>(bv) : 0.f;
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(gv, off, 64);
            if (lane >= off) gv += o;
        }
        const float gl = __shfl(gv, ell - 1, 64);
        const float kd = lane < ell ? __expf(gl - gv) : 0.f;  // gamma_l / gamma
        const float sk = bv * __expf(gv);                     // beta gamma
        s.gc[lane] = gv;
        s.beta[lane] = bv;
        s.sk[lane] = sk;
        s.svb[lane] = bv;
        s.kd[lane] = kd;
        float* G = p.gates + ch * 4 * CHUNK;
        G[lane] = lane < ell ? gv : 0.f;
        G[CHUNK + lane] = kd;
        G[2 * CHUNK + lane] = bv;
        G[3 * CHUNK + lane] = sk;
    }
    // Without W and U the next item's K and gate loads go out now (this item's
    // are staged), to land while K K^T, the solve and P are formed; with them
    // they wait until A is in registers (the V rows hold those registers until then).
    v += gridDim.x;
    const int next = v < padded ? xcd_remap(v, padded) : work;
    if constexpr (!WU) {
        if (next < work) load_k(next);
    }
    lds_sync();

    // K K^T: wave w forms row block w against column blocks J <= w (fragments from LDS);
    // L_ij = beta_i exp(gc_i - gc_j) (k_i . k_j) for i > j, zero elsewhere.
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        if (J > w) break;
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            Frag<T> a, b;
            load8(a, &s.K[16 * w + r16][32 * ks + 8 * grp]);
            load8(b, &s.K[16 * J + r16][32 * ks + 8 * grp]);
            acc = mma(a, b, acc);
        }
        float* Lb = Ls + blk(w, J);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int i = 16 * w + 4 * grp + i4, j = 16 * J + r16;
            Lb[(4 * grp + i4) * BS + r16] = (i > j) ? s.beta[i] * __expf(s.gc[i] - s.gc[j]) * acc[i4] : 0.f;
        }
    }
    lds_sync();

    // (I + L)^-1 by blocks of 16, each A block stored over the L block of the same
    // index once no later step reads that L block.  Diagonal blocks: forward
    // substitution, lane owns column c (the wave reads all of L_ww before writing A_ww).
    {
        const float* Lb = Ls + blk(w, w);
        const int c = r16;
        float a[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < r; ++kk) acc -= Lb[r * BS + kk] * a[kk];
            a[r] = acc;
        }
        if (grp == 0) {
            float* Ab = As + blk(w, w);
#pragma unroll
            for (int r = 0; r < 16; ++r) Ab[r * BS + c] = a[r];
        }
    }
    lds_sync();
    // 32x32 diagonal blocks: A10 = -A11 L10 A00 (wave 0), A32 = -A33 L32 A22 (wave 1).
    if (w < 2) {
        const int o = 2 * w;
        const f32x4 t = mm16_lds<BS, BS>(Ls + blk(o + 1, o), As + blk(o, o), zero4(), r16, grp);
        tile_to_lds<BS>(Tm + w * BLK, t, 1.f, r16, grp);
    }
    lds_sync();
    if (w < 2) {
        const int o = 2 * w;
        const f32x4 t = mm16_lds<BS, BS>(As + blk(o + 1, o + 1), Tm + w * BLK, zero4(), r16, grp);
        tile_to_lds<BS>(As + blk(o + 1, o), t, -1.f, r16, grp);
    }
    lds_sync();
    // Lower-left 32x32 block: A_LL = -A_hi (L_LL A_lo).  Wave w owns block (I, J) =
    // (2 + w/2, w%2); first T_IJ = sum_{K=J..1} L_IK A_KJ ...
    {
        const int I = 2 + (w >> 1), J = w & 1;
        f32x4 t = zero4();
        for (int K = J; K <= 1; ++K) t = mm16_lds<BS, BS>(Ls + blk(I, K), As + blk(K, J), t, r16, grp);
        tile_to_lds<BS>(Tm + w * BLK, t, 1.f, r16, grp);
    }
    lds_sync();
    // ... then A_IJ = -sum_{K=2..I} A_IK T_KJ (T_KJ sits in Tm block 2*(K-2) + J).
    {
        const int I = 2 + (w >> 1), J = w & 1;
        f32x4 t = zero4();
        for (int K = 2; K <= I; ++K) t = mm16_lds<BS, BS>(As + blk(I, K), Tm + (2 * (K - 2) + J) * BLK, t, r16, grp);
        tile_to_lds<BS>(As + blk(I, J), t, -1.f, r16, grp);
    }
    lds_sync();

    // A's fragments for the state scan that forms X from them: wave w writes
    // those of row tile w.  Rows past the valid length are unit rows e_i (their L
    // rows vanish with beta), which meet the zero rows of B Y there, so X
    // vanishes on them unmasked.
    if (!WU || p.write_af) {
        PT* Ab = reinterpret_cast<PT*>(p.Af) + ch * A_FRAGS * 512;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (ks == 1 && w < 2) break;
            Frag<PT> f;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int J = 2 * ks + hh;  // column block: columns 32 ks + 16 hh + 4 grp .. + 3
                float4 x = make_float4(0, 0, 0, 0);
                if (J <= w) x = *reinterpret_cast<const float4*>(As + blk(w, J) + r16 * BS + 4 * grp);
                frag_set(f, 4 * hh + 0, x.x);
                frag_set(f, 4 * hh + 1, x.y);
                frag_set(f, 4 * hh + 2, x.z);
                frag_set(f, 4 * hh + 3, x.w);
            }
            *reinterpret_cast<Frag<PT>*>(Ab + ((a_frag_first(w) + ks) * 64 + lane) * 8) = f;
        }
    }

    // P (bf16): the P^T tiles (J, w) = K_J Q_w^T of this wave's query positions
    // i = 16 w + r16, P^T[j][i] = (k_j . q_i) exp(gc_i - gc_j) for j <= i < ell
    // (Lower keeps the diagonal), K_J from the staged keys.  With the front end
    // the query rows are L2-normalised first (the row spread over the four lanes
    // of lane % 16).  Where the state scan reads them (the launcher passes Qc:
    // one column tile a workgroup, or the front end), the first value head of
    // each key head keeps the rows for its output waves, as the B operands of their h^T Q^T
    // product: wave w's fragment (w, ks) holds, in lane 16 a + r, slot 4 hh + b,
    // q[16 w + r][32 ks + 16 hh + 4 a + b] (the exchanged -S fragments' d_k
    // order), so that each output wave loads a step's query operand as four
    // 1 KiB pieces straight into registers.  This lane's 8 values are d_k
    // 32 ks + 8 grp .. + 7: two 4-value halves, each a half of another lane's slots.
    if constexpr (sizeof(T) == 2) {
        if (p.Pf) {
            const int row = 16 * w + r16;
            if (p.fa) {
                float ss = 0.f;
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
                    for (int j = 0; j < 8; ++j) ss += frag_get(qw[ks], j) * frag_get(qw[ks], j);
                const float r = 1.f / sqrtf(sum_over_rows(ss) + 1e-6f);
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
                    for (int j = 0; j < 8; ++j) frag_set(qw[ks], j, frag_get(qw[ks], j) * r);
            }
            if (p.Qc && h % p.G == 0) {
                T* Qcb = reinterpret_cast<T*>(p.Qc) + (((size_t)cp.ci * p.H_q + h / p.G) * 4 + w) * (D / 32) * 64 * 8;
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int e = 8 * grp + 4 * hf;  // first d_k offset of the half within the step
                        const int a = (e & 15) >> 2, hh = e >> 4;
                        *reinterpret_cast<bf16x4*>(Qcb + ((ks * 64 + 16 * a + r16) * 8 + 4 * hh)) =
                            bf16x4{qw[ks].v[4 * hf], qw[ks].v[4 * hf + 1], qw[ks].v[4 * hf + 2], qw[ks].v[4 * hf + 3]};
                    }
            }
            f32x4 pt[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                if (J > w) break;
                f32x4 pacc = zero4();
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    Frag<T> b;
                    load8(b, &s.K[16 * J + r16][32 * ks + 8 * grp]);
                    pacc = mma(b, qw[ks], pacc);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * J + 4 * grp + e;
                    pt[J][e] = (j <= row && row < ell) ? pacc[e] * __expf(s.gc[row] - s.gc[j]) : 0.f;
                }
            }
            // to the workspace as the B operands of X^T P^T: query tile w, K-steps
            // s = 0 (and 1 for w >= 2), two stacked P^T tiles per fragment (perm32)
            T* Pb = reinterpret_cast<T*>(p.Pf) + ch * P_FRAGS * 512;
            const int f0 = w < 2 ? w : 2 * w - 2;
            *reinterpret_cast<Frag<T>*>(Pb + (f0 * 64 + lane) * 8) = pack_perm32<T>(pt[0], pt[1], 1.f);
            if (w >= 2) *reinterpret_cast<Frag<T>*>(Pb + ((f0 + 1) * 64 + lane) * 8) = pack_perm32<T>(pt[2], pt[3], 1.f);
        }
    }

    // A to the workspace on request, zero outside the valid lower triangle.
    if (p.keep_A) {
        T* Ab = reinterpret_cast<T*>(p.A) + ch * CHUNK * CHUNK;
        const int i = tid >> 2, jb = tid & 3;  // row i, column block jb
        const float* src = As + blk(i >> 4, jb) + (i & 15) * BS;
#pragma unroll
        for (int j4 = 0; j4 < 16; j4 += 4) {
            float v4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * jb + j4 + e;
                v4[e] = (jb <= (i >> 4) && j <= i && i < ell) ? src[j4 + e] : 0.f;
            }
            store4(Ab + (size_t)i * CHUNK + 16 * jb + j4, v4[0], v4[1], v4[2], v4[3]);
        }
    }

    // W = A B Gamma K and U = A B V, for the state scan that reads them (and on
    // request, for inspection), with the operand types and fragment orders
    // documented for the workspace.
    if constexpr (WU) {
        // Fragments of A (rows pos, contiguous columns): Af[mt][ks] is the A operand
        // of U = A (B V) for row tile mt and the B operand of W^T = (B Gamma K)^T A^T
        // for column tile mt.  Rows past the valid length are unit rows e_i, which
        // meet zero rows of B Gamma K and B V, so W and U vanish there unmasked.
        Frag<PT> Af[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int J = 2 * ks + (grp >> 1);  // column block of this lane's 8 columns
                float4 lo = make_float4(0, 0, 0, 0), hi = lo;
                if (J <= mt) {
                    const float4* src = reinterpret_cast<const float4*>(As + blk(mt, J) + r16 * BS + 8 * (grp & 1));
                    lo = src[0];
                    hi = src[1];
                }
                frag_set(Af[mt][ks], 0, lo.x); frag_set(Af[mt][ks], 1, lo.y);
                frag_set(Af[mt][ks], 2, lo.z); frag_set(Af[mt][ks], 3, lo.w);
                frag_set(Af[mt][ks], 4, hi.x); frag_set(Af[mt][ks], 5, hi.y);
                frag_set(Af[mt][ks], 6, hi.z); frag_set(Af[mt][ks], 7, hi.w);
            }
        lds_sync();  // A is in registers: its LDS takes V (read after W is done)
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = tid + 256 * j, r = e / (D / VEC), c = (e % (D / VEC)) * VEC;
            *reinterpret_cast<float4*>(&s.u.V[r][c]) = vreg[j];
        }
        // The next item's K and gate loads go out now; they land while W and U are formed.
        if (next < work) load_k(next);

        constexpr int TPW = D / 64;  // 16-wide tiles of d_k (or d_v) per wave
        // A fragment of 8 consecutive positions (32 ks + 8 grp ..) of one column of a
        // staged [pos][col] matrix, each value scaled by its position's factor and
        // rounded to the product type (fp16 for bf16 inputs: rounding the scaled
        // values B V to bf16 was the largest single error of the output).  For
        // bf16 the columns come from LDS with transposed reads (two per fragment);
        // for fp32 element by element.
        auto col_frag = [&](Frag<PT>& f, const T* M, const float* sc, int ks, int c) {
            const int r0 = 32 * ks + 8 * grp;
            if constexpr (sizeof(T) == 2) {
                const bf16x4 lo = lds_col4<PL::KP>(M, r0, c & ~15, lane), hi = lds_col4<PL::KP>(M, r0 + 4, c & ~15, lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    frag_set(f, j, sc[r0 + j] * (float)lo[j]);
                    frag_set(f, 4 + j, sc[r0 + 4 + j] * (float)hi[j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) frag_set(f, j, sc[r0 + j] * to_f32<T>(M[(r0 + j) * PL::KP + c]));
            }
        };
        auto w_kfrag = [&](Frag<PT>(&kf)[2], int mt) {  // (B Gamma K)^T rows of d_k tile mt, contraction pos
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) col_frag(kf[ks], &s.K[0][0], s.sk, ks, 16 * mt + r16);
        };
        // W^T tiles: rows d_k (this wave's tiles), columns pos; column tile nt only
        // needs contraction steps ks with 32 ks <= 16 nt + 15.  lane: column pos =
        // 16 nt + r16, rows d_k = 16 mt + 4 grp + i: fragment (pos tile nt, K-step
        // mt / 2), same lane, slots 4 (mt % 2) + i.
        T* Wb = reinterpret_cast<T*>(p.W) + ch * CHUNK * D;
        if constexpr (TPW == 2) {  // this wave's two d_k tiles fill whole fragments: 16-byte stores
            Frag<PT> k0[2], k1[2];
            w_kfrag(k0, 2 * w);
            w_kfrag(k1, 2 * w + 1);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                f32x4 c0 = mma(k0[0], Af[nt][0], zero4()), c1 = mma(k1[0], Af[nt][0], zero4());
                if (nt >= 2) {
                    c0 = mma(k0[1], Af[nt][1], c0);
                    c1 = mma(k1[1], Af[nt][1], c1);
                }
                store8(Wb + frag_w_offset<D>(nt, w, lane), c0, c1);
            }
        } else {
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int mt = w * TPW + tt;
                Frag<PT> kf[2];
                w_kfrag(kf, mt);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    f32x4 c = zero4();
                    c = mma(kf[0], Af[nt][0], c);
                    if (nt >= 2) c = mma(kf[1], Af[nt][1], c);
                    store4(Wb + frag_w_offset<D>(nt, mt >> 1, lane) + 4 * (mt & 1), c[0], c[1], c[2], c[3]);
                }
            }
        }
        lds_sync();  // V staged
        // U tiles: rows pos, columns d_v (this wave's tiles), stored in the product type.
        PT* Ub = reinterpret_cast<PT*>(p.Ut) + ch * D * CHUNK;
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int nt = w * TPW + tt;
            const int dv = 16 * nt + r16;
            Frag<PT> vf[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) col_frag(vf[ks], &s.u.V[0][0], s.svb, ks, dv);
            // lane: column d_v = 16 nt + r16, rows pos = 16 mt + 4 grp + i (accumulator
            // order); row tiles 2 m and 2 m + 1 share one 16-byte store
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                f32x4 c0 = mma(Af[2 * m][0], vf[0], zero4()), c1 = mma(Af[2 * m + 1][0], vf[0], zero4());
                if (m == 1) {
                    c0 = mma(Af[2][1], vf[1], c0);
                    c1 = mma(Af[3][1], vf[1], c1);
                }
                store8(Ub + frag_u_offset(nt, m, lane), c0, c1);
            }
        }
    }
    if (next >= work) break;
    lds_sync();  // every read of this item's LDS is done before the next item's K lands
    wid = next;
    }
}
// ---------------------------------------------------------------------------
// 3. chunk_state_h: one workgroup per (sequence, value head, 16-column tile of
//    d_v), serial over the sequence's chunks: four compute waves (one per
//    SIMD), NPW producer waves (one) and one store wave.
//
//    Compute waves.  The fp32 state slice S[:, tile] (d_k x 16) stays in MFMA
//    accumulators, split by rows over the waves.  Per chunk:
//      B Y = B (V - Gamma K S)     wave w: positions 16w..16w+15, contraction over d_k
//      X   = A (B Y)               wave w: positions 16w..16w+15, contraction over positions
//      S   = gamma_l S + K^T (kf X)  wave w: its rows of S, contraction over positions
//    X is U - W S of the chunk form, regrouped as A B (V - Gamma K S), so the
//    chunk's operands are its raw key rows (Kc, with the front end the
//    L2-normalised ones), its value rows, the 64 x 64 A and the gates; kf =
//    gamma_l / gamma per position applies the chunk form's decayed keys to X
//    rather than to K.  The products exchange bf16 copies of -S, X and kf X
//    (and B Y in the type of A's fragments) through LDS in MFMA operand order
//    (one 16-byte access per lane and fragment), three barriers a chunk (B1
//    before K S, Bm before the A product, B2 before the state update).  A
//    chunk's operand fragments are copied from its LDS stage into registers
//    during the previous step (K's column fragments with transposed reads):
//    with three stages between Bm and B2, where the compute waves would
//    otherwise wait for the output waves, with two after B2.  The compute
//    waves issue no global memory instruction inside the loop: a
//    vector-memory instruction stalls its wave whenever the CU's memory
//    pipeline is backed up, and on this serial path every stall delays the
//    next barrier for all waves.
//
//    Producer waves.  Stream each chunk's K rows (Kc, one copy per key head),
//    A fragments, gate block (stored by chunk_prep in exactly the LDS stage
//    order) and the value rows of the workgroup's column tiles (gathered from
//    v) into a ring of NST stages (three where they fit) with direct
//    global->LDS loads.  A stage is free once its chunk is in registers (B1
//    of that chunk's step); chunk c + NST goes out in two halves, at B1(c) and
//    B2(c); vmcnt waits make chunk c + 1 land before B1(c) (three stages) or
//    B2(c) (two) and keep at most 63 loads in flight per wave.
//
//    Store wave.  Writes the output tiles (bf16) or copies h_c (the
//    sign-flipped -S of LS, between B1(c) and B2(c)) and X_c (LX, between
//    B2(c) and B1(c + 1)) to HBM.
// ---------------------------------------------------------------------------
// Loads producer wave pw of NPW issues in part 0 / part 1 of a chunk of NPIECE
// 1 KiB pieces.
__host__ __device__ constexpr int stage_part_loads(int npiece, int npw, int pw, int part) {
    int n = 0;
    for (int j = 0; j < npiece; ++j) n += (j % npw == pw && (j < npiece / 2) == (part == 0)) ? 1 : 0;
    return n;
}
// Producer waves' vmcnt bound at B2(c) (chunks c + 2 .. c + nst - 1 whole plus
// part 0 of chunk c + nst issued after chunk c + 1's last load) for wave pw.
__host__ __device__ constexpr int stage_wait_b2(int npiece, int npw, int nst, int pw) {
    return (nst - 2) * (stage_part_loads(npiece, npw, pw, 0) + stage_part_loads(npiece, npw, pw, 1)) +
           stage_part_loads(npiece, npw, pw, 0);
}
// Fewest producer waves (1, 2 or 4) whose outstanding loads stay within the
// 63 a wave's vmcnt can count.
__host__ __device__ constexpr int stage_producers(int npiece, int nst) {
    for (int npw = 1; npw < 4; npw *= 2) {
        bool ok = true;
        for (int pw = 0; pw < npw; ++pw) {
            const int r0 = 63 - stage_part_loads(npiece, npw, pw, 0);
            ok = ok && stage_wait_b2(npiece, npw, nst, pw) < 64 && r0 - stage_part_loads(npiece, npw, pw, 1) >= 0;
        }
        if (ok) return npw;
    }
    return 4;
}

// One chunk's LDS stage, each part a whole number of 1 KiB pieces.
//   W form (AF false): W fragments | K rows | U of the CT column tiles | gate
//     block | (FO) P fragments.
//   A form (AF true): K rows | (FO) P fragments | A fragments | gate block |
//     value rows of the CT column tiles.  Everything from A on lies in the
//     second half of the pieces, which the producer issues for chunk c + NST
//     only at B2(c) (see below), so the compute waves may read A, the gates
//     and the value rows of chunk c from its stage in step c itself.
// FO: the output is formed in the scan; the stage also carries the chunk's P
// fragments (for the output waves) and the workgroup keeps an output tile
// buffer through which the store wave writes O.
template <typename T, int D, int CT = 1, bool FO = false, bool AF = false>
struct StateStage {
    using PT = ProdT<T>;
    static constexpr int K_BYTES = CHUNK * D * (int)sizeof(T);            // K rows, row-major (pieces permuted by kswz)
    static constexpr int G_BYTES = 4 * CHUNK * 4;                         // gc, kf, beta, beta gamma
    static constexpr int P_BYTES = FO ? P_FRAGS * 1024 : 0;               // P fragments (bf16)
    static constexpr int W_BYTES = AF ? 0 : CHUNK * D * (int)sizeof(T);   // W fragments
    static constexpr int U1_BYTES = CHUNK * 16 * (int)sizeof(PT);         // U of one 16-column tile
    static constexpr int U_BYTES = AF ? 0 : CT * U1_BYTES;
    static constexpr int A_BYTES = AF ? A_FRAGS * 64 * 8 * (int)sizeof(PT) : 0;  // A's six fragments
    static constexpr int V1_BYTES = CHUNK * 16 * (int)sizeof(T);          // value rows of one tile, [64][16]
    static constexpr int V_BYTES = AF ? CT * V1_BYTES : 0;
    static constexpr int W_OFF = 0;
    static constexpr int K_OFF = AF ? 0 : W_BYTES;
    static constexpr int U_OFF = K_OFF + K_BYTES;
    static constexpr int P_OFF = AF ? K_BYTES : U_OFF + U_BYTES + G_BYTES;
    static constexpr int A_OFF = AF ? P_OFF + P_BYTES : 0;
    static constexpr int G_OFF = AF ? A_OFF + A_BYTES : U_OFF + U_BYTES;
    static constexpr int V_OFF = AF ? G_OFF + G_BYTES : 0;
    static constexpr int BYTES = W_BYTES + K_BYTES + U_BYTES + G_BYTES + P_BYTES + A_BYTES + V_BYTES;
    static_assert(BYTES % 1024 == 0 && V1_BYTES % 1024 == 0 && U1_BYTES % 1024 == 0, "stage pieces are 1 KiB");
    static constexpr int NPIECE = BYTES / 1024;  // 1 KiB loads per chunk
    static_assert(!AF || A_OFF / 1024 >= NPIECE / 2, "A, the gates and V must lie in the second half of the pieces");
    // Exchange blocks (-S, X, kf X and, in the A form, B Y): one fragment per
    // lane, 16 bytes of padding after every 16 lanes so that the store wave's
    // column gathers spread over the LDS banks.
    static constexpr int XPAD = 16;
    static constexpr int XBLK = 64 * 8 * (int)sizeof(T) + 4 * XPAD;
    static_assert(sizeof(PT) == sizeof(T), "B Y shares the exchange block size");
    static constexpr int EXCH = (D / 32 + (AF ? 6 : 4)) * CT * XBLK;
    static constexpr int OBUF = FO ? 4 * CT * 64 * 8 : 0;  // output tiles (bf16: 4 values a lane, per wave and tile)
    static constexpr int QBUF = FO && CT > 1 ? 4 * 16 * D * (int)sizeof(T) : 0;  // each output wave's 16 query rows
    // Three stages where they fit and one producer wave can keep them fed (a
    // chunk is issued two steps and a half before it is read), else two.  The
    // third stage pays where the stream comes from HBM (T = 65536: 991 -> 902
    // us) and costs nothing at T = 4096.  A second producer wave costs more
    // than it brings (T = 4096: 48.6 -> 61.9 us), so a stage that only two
    // producers could keep three deep gets two.
    static constexpr int LDS_CAP = 160 * 1024;
    static constexpr int NST = (3 * BYTES + EXCH + OBUF + QBUF + 256 <= LDS_CAP &&  // + the L2-prefetch sink
                                (FO ? stage_producers(NPIECE, 3) == 1 : true))
                                   ? 3
                                   : 2;
    // A wave can keep at most 63 vector-memory operations in flight, so the
    // stream is split over NPW producer waves, each owning every NPW-th piece.
    // The compute waves copy chunk c into registers before B1(c), so stage
    // c % NST is refilled with chunk c + NST from B1(c) on.
    static constexpr int NPW = stage_producers(NPIECE, NST);
    static constexpr int NOUT = FO ? 4 : 0;       // output waves
    static constexpr int WAVES = 5 + NPW + NOUT;  // compute, producers, store, output
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

// LDS reads the compiler does not track.  The producer reads the compute
// waves' exchange buffers while its own direct-to-LDS loads are in flight; a
// plain LDS load there makes the compiler wait for all of those loads (it
// cannot tell the buffers apart), so the producer reads with inline asm and
// waits for the results itself (lds_wait_untracked) before using them.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// N 16-byte reads: piece i of element j at addr + j * stride + 16 * i (n pieces an element).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <int N>
__device__ __forceinline__ void lds_read_untracked(u32x4* r, unsigned addr, unsigned stride, int n) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const unsigned a = addr + (k / n) * stride + 16 * (k % n);
        asm volatile("ds_read_b128 %0, %1" : "=v"(r[k]) : "v"(a));
    }
}

template <int N>
__device__ __forceinline__ void lds_wait_untracked(u32x4* r) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int k = 0; k < N; ++k) asm volatile("" : "+v"(r[k]));  // uses of r stay after the wait
}

// Issue this producer wave's share (pieces j with j % NPW == pw) of one
// chunk's direct-to-LDS loads, in stage order; part 0 issues the first half
// of the share, part 1 the rest.  ch: (chunk, value head) index; kch: (chunk,
// key head) index of Kc; tok, ell: the chunk's first token and valid length.
// A form: the value rows of column tile ct come straight from v, one 16-byte
// piece a lane: a 1 KiB piece covers 32 rows (bf16; 16 for fp32) of the
// tile's 16 columns, and rows past the valid length repeat the last valid row
// (finite values that meet beta = 0).
template <typename T, int D, int CT, bool FO, bool AF>
__device__ __forceinline__ void state_issue(char* stage, const ChunkParams& p, size_t ch, size_t kch, int tok,
                                            int ell, int h, int tile, int lane, int pw, int part) {
    using SS = StateStage<T, D, CT, FO, AF>;
    constexpr int NT = D / 16;
    constexpr int NW = SS::W_BYTES / 1024, NK = SS::K_BYTES / 1024, NU = SS::U_BYTES / 1024;
    constexpr int NA = SS::A_BYTES / 1024, NPF = SS::P_BYTES / 1024;
    constexpr int NP = SS::NPIECE;
    constexpr int VPT = SS::V1_BYTES / 1024;       // pieces per column tile of V
    constexpr int LPR = 16 * (int)sizeof(T) / 16;  // lanes per row of a V tile (2 bf16, 4 fp32)
    constexpr int RPP = 64 / LPR;                  // rows per piece
    const char* wg = reinterpret_cast<const char*>(p.W) + ch * SS::W_BYTES;
    const char* kg = reinterpret_cast<const char*>(p.Kc) + kch * SS::K_BYTES;
    const char* ug = reinterpret_cast<const char*>(p.Ut) + (ch * NT + CT * tile) * SS::U1_BYTES;
    const char* pg = reinterpret_cast<const char*>(p.Pf) + ch * SS::P_BYTES;
    const char* ag = reinterpret_cast<const char*>(p.Af) + ch * SS::A_BYTES;
    const char* gg = reinterpret_cast<const char*>(p.gates + ch * 4 * CHUNK);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        if (j % SS::NPW != pw) continue;
        if ((j < NP / 2) != (part == 0)) continue;
        char* dst = stage + 1024 * j;  // the stage's parts follow one another in piece order
        if constexpr (!AF) {
            if (j < NW)
                dma_1k(wg + 1024 * j, dst, lane);
            else if (j < NW + NK)
                dma_1k(kg + 1024 * (j - NW), dst, lane);
            else if (j < NW + NK + NU)
                dma_1k(ug + 1024 * (j - NW - NK), dst, lane);
            else if (j < NW + NK + NU + 1)
                dma_1k(gg, dst, lane);
            else
                dma_1k(pg + 1024 * (j - NW - NK - NU - 1), dst, lane);
        } else {
            if (j < NK) {
                dma_1k(kg + 1024 * j, dst, lane);
            } else if (j < NK + NPF) {
                dma_1k(pg + 1024 * (j - NK), dst, lane);
            } else if (j < NK + NPF + NA) {
                dma_1k(ag + 1024 * (j - NK - NPF), dst, lane);
            } else if (j < NK + NPF + NA + 1) {
                dma_1k(gg, dst, lane);
            } else {
                const int vj = j - NK - NPF - NA - 1, ct = vj / VPT, row = (vj % VPT) * RPP + lane / LPR;
                const char* src = reinterpret_cast<const char*>(p.v) +
                                  (((size_t)(tok + min(row, ell - 1)) * p.H_v + h) * D + 16 * (CT * tile + ct)) * sizeof(T) +
                                  16 * (lane % LPR);
                __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)dst, 16, 0, 0);
            }
        }
    }
}

template <typename SS>
__host__ __device__ constexpr int state_part_loads(int pw, int part) {
    return stage_part_loads(SS::NPIECE, SS::NPW, pw, part);
}
template <typename SS>
__host__ __device__ constexpr int state_wait_b2(int pw) {
    return stage_wait_b2(SS::NPIECE, SS::NPW, SS::NST, pw);
}
// Write a D tile's four values (rows 4 grp + i of one 16-row tile) into the
// perm32 fragment they belong to: even tile -> slots 0..3, odd -> slots 4..7.
template <typename T>
__device__ __forceinline__ void lds_put4(Frag<T>& f, int half, const f32x4& v, float s) {
    if constexpr (std::is_same_v<T, bf16>) {
        *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(&f) + 4 * half) = cvt4_bf16(v, s);
    } else if constexpr (std::is_same_v<T, f16>) {
        *reinterpret_cast<f16x4*>(reinterpret_cast<f16*>(&f) + 4 * half) = __builtin_convertvector(v * s, f16x4);
    } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(&f) + 4 * half) =
            make_float4(s * v[0], s * v[1], s * v[2], s * v[3]);
    }
}

// A operand of the state update K^T (kf X) for rows 16 m .. 16 m + 15 of S
// (columns of K) and contraction step ks (positions 32 ks .. 32 ks + 31 in
// perm32 slots: slot b <- position 32 ks + 4 g + b, slot 4 + b <- 32 ks + 16 +
// 4 g + b, g = lane / 16), read from a stage's K rows (pieces permuted by kswz).
template <typename T, int D>
__device__ __forceinline__ Frag<T> k_col_frag(const char* kst, int m, int ks, int lane) {
    constexpr int RB = D * (int)sizeof(T);  // bytes per K row
    const int g = (lane >> 4) & 3, j = lane & 15;
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        typedef short v4i16 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            // transposed read: lane j names row r0 + j / 4, columns 16 m + 4 (j % 4) .. + 3;
            // lane i receives column 16 m + i of rows r0 .. r0 + 3
            const int row = 32 * ks + 16 * half + 4 * g + (j >> 2);
            const int piece = (2 * m + ((j & 3) >> 1)) ^ kswz<T, D>(row);
            const char* a = kst + row * RB + 16 * piece + 8 * (j & 1);
            const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)a);
            const bf16x4 b = __builtin_bit_cast(bf16x4, r);
#pragma unroll
            for (int i = 0; i < 4; ++i) f.v[4 * half + i] = b[i];
        }
    } else {
        const int colb = 4 * (16 * m + j);  // byte of column 16 m + j in an unpermuted row
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            const int row = 32 * ks + (sl < 4 ? 4 * g + sl : 16 + 4 * g + sl - 4);
            const int piece = (colb >> 4) ^ kswz<T, D>(row);
            f.v[sl] = *reinterpret_cast<const float*>(kst + row * RB + 16 * piece + (colb & 15));
        }
    }
    return f;
}

// A operand of K S for the 16 positions r0 .. r0 + 15 (row r0 + lane % 16) and
// contraction step ks over d_k in the perm32 order of the exchanged -S
// fragments (slot 4 h + b <- d_k 32 ks + 16 h + 4 g + b, g = lane / 16), read
// from a stage's K rows (pieces permuted by kswz): two 4-value reads a fragment.
template <typename T, int D>
__device__ __forceinline__ Frag<T> k_row_frag(const char* kst, int r0, int ks, int lane) {
    constexpr int RB = D * (int)sizeof(T);  // bytes per K row
    const int g = lane >> 4, row = r0 + (lane & 15);
    Frag<T> f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int col = 32 * ks + 16 * hh + 4 * g;                  // first of the four d_k indices
        const int piece = (col * (int)sizeof(T) / 16) ^ kswz<T, D>(row);
        const char* a = kst + row * RB + 16 * piece + (col * (int)sizeof(T)) % 16;
        if constexpr (sizeof(T) == 2) {
            const bf16x4 x = *reinterpret_cast<const bf16x4*>(a);
#pragma unroll
            for (int i = 0; i < 4; ++i) f.v[4 * hh + i] = x[i];
        } else {
            const float4 x = *reinterpret_cast<const float4*>(a);
            f.v[4 * hh + 0] = x.x; f.v[4 * hh + 1] = x.y; f.v[4 * hh + 2] = x.z; f.v[4 * hh + 3] = x.w;
        }
    }
    return f;
}

// Value rows r0 .. r0 + 3 (r0 = 16 w + 4 (lane / 16)) of column lane % 16 of a
// stage's [64][16] tile: the accumulator layout of the wave's K S tile.
template <typename T>
__device__ __forceinline__ f32x4 v_acc4(const char* vst, int r0, int lane) {
    if constexpr (sizeof(T) == 2) {
        const bf16x4 x = lds_col4<16>(reinterpret_cast<const bf16*>(vst), r0, 0, lane);
        return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    } else {
        const float* b = reinterpret_cast<const float*>(vst) + r0 * 16 + (lane & 15);
        return f32x4{b[0], b[16], b[32], b[48]};
    }
}

// ---------------------------------------------------------------------------
// Output waves of chunk_state_h with the output formed in the scan (stage 4 of
// the chunk form computed beside stage 3).  Wave o forms the outputs of
// positions 16 o .. 16 o + 15 of every chunk for the workgroup's CT column
// tiles of d_v:
//   O^T = scale [ (h^T Q^T) diag(gamma) + X^T P^T ]
// from the scan's own operands: h_c from LS (which holds -h_c between B1(c)
// and B2(c)), X_c from LX (between B2(c) and B1(c + 1)), P and the gates from
// the chunk's stage (read after B2(c - 1), before the stage is released at
// B1(c)), and this wave's query rows, copied into LDS a chunk ahead (with the
// front end from chunk_prep's normalised copy Qc).  LS and LX fragments serve as the A
// operands h^T and X^T unchanged; the query fragments list d_k in the same
// (perm32) order.  The bf16 tile goes to LO, from where the store wave writes
// it after the next barrier, so these waves issue no global store.  Nothing
// on the serial chain waits for them except the two barriers of a step.
// ---------------------------------------------------------------------------
template <typename T, int D, int CT, bool AF>
__device__ __forceinline__ void chunk_output_waves(const ChunkParams& p, const char* smem, const char* LS,
                                                   const char* LX, char* LO, char* LQ, int o, int lane,
                                                   const SeqTable& tab, int kb, int ke, int hq, int nch) {
    static_assert(sizeof(T) == 2, "the output waves are bf16");
    using SS = StateStage<T, D, CT, true, AF>;
    constexpr int KS = D / 32;
    constexpr int NST = SS::NST;
    o = __builtin_amdgcn_readfirstlane(o);
    const int r16 = lane & 15, grp = lane >> 4;
    const int pos = 16 * o + r16;  // this lane's query position (column of its O^T tiles)
    auto xfr = [&](const char* buf, int b) {
        return *reinterpret_cast<const Frag<T>*>(buf + b * SS::XBLK + lane * (int)sizeof(Frag<T>) +
                                                 (lane >> 4) * SS::XPAD);
    };
    // Query operand.  One column tile a workgroup: this wave's four fragments
    // of the chunk's rows come from chunk_prep's copy Qc, already in operand
    // order (four 1 KiB loads), straight into registers a step ahead, so none
    // of it passes through LDS, which the first half of a step is short of
    // (T = 65536: scan 1034 -> 962 us for 25 us more in chunk_prep).  With more
    // tiles, where the copy costs chunk_prep more than the scan saves, each wave
    // copies its 16 rows into its own LDS buffer with 1 KiB direct-to-LDS
    // loads, issued a step ahead right after the previous chunk's fragments
    // have been read out: from Qc with the front end (normalised, in operand
    // order), else from q, the 16-byte pieces of row r permuted by r so that
    // the fragment reads spread over the banks (rows past the valid length
    // re-read the last valid row; their outputs are never stored).
    constexpr bool QREG = CT == 1;
    constexpr int RB = D * (int)sizeof(T), PPR = RB / 16;  // row bytes, 16-byte pieces a row
    char* const lq = LQ + o * 16 * RB;
    BinCursor cq;  // the chunk whose query rows are loaded next
    cq.begin(tab, kb, ke);
    Frag<T> qn[KS];
    auto qc_block = [&]() {  // this wave's fragments in Qc (16 RB bytes)
        return reinterpret_cast<const char*>(p.Qc) + (((size_t)cq.ci() * p.H_q + hq) * 4 + o) * 16 * RB;
    };
    auto load_q = [&]() {
        if constexpr (QREG) {
            const Frag<T>* q0 = reinterpret_cast<const Frag<T>*>(qc_block());
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qn[ks] = q0[ks * 64 + lane];
        } else if (p.Qc) {
            const char* q0 = qc_block();
#pragma unroll
            for (int i = 0; i < 16 * PPR / 64; ++i) dma_1k(q0 + 1024 * i, lq + 1024 * i, lane);
        } else {
            const int ell = cq.ell();
            const char* q0 = reinterpret_cast<const char*>(p.q) + ((size_t)cq.token() * p.H_q + hq) * RB;
#pragma unroll
            for (int i = 0; i < 16 * PPR / 64; ++i) {
                const int e = 64 * i + lane, r = e / PPR, pc = (e % PPR) ^ (r % PPR);
                const char* src = q0 + (size_t)min(16 * o + r, ell - 1) * p.H_q * RB + 16 * pc;
                __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)(lq + 1024 * i), 16, 0, 0);
            }
        }
        cq.next();
    };
    // fragment ks of this lane's row: slots 0..3 <- d_k 32 ks + 4 grp .. + 3,
    // slots 4..7 <- 32 ks + 16 + 4 grp .. + 3 (the exchange fragments' d_k order)
    auto q_frag = [&](int ks) -> Frag<T> {
        if constexpr (QREG) {
            return qn[ks];
        } else {
            if (p.Qc) return *reinterpret_cast<const Frag<T>*>(lq + (ks * 64 + lane) * 16);
            const char* row = lq + r16 * RB + 8 * (grp & 1);
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 16 * ((4 * ks + (grp >> 1)) ^ (r16 % PPR)));
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16 * ((4 * ks + 2 + (grp >> 1)) ^ (r16 % PPR)));
            Frag<T> f;
            f.v = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return f;
        }
    };
    Frag<T> pf0, pf1;
    float gq = 0.f;
    auto read_stage = [&](int c) {
        const char* st = smem + (c % NST) * SS::BYTES;
        const Frag<T>* P = reinterpret_cast<const Frag<T>*>(st + SS::P_OFF);
        const int f0 = o < 2 ? o : 2 * o - 2;  // fragments of query tile o (see P_FRAGS)
        pf0 = P[f0 * 64 + lane];
        if (o >= 2) pf1 = P[(f0 + 1) * 64 + lane];
        gq = reinterpret_cast<const float*>(st + SS::G_OFF)[pos];
    };
    if (nch > 0) load_q();
    wait_lgkmcnt0();
    asm volatile("s_barrier" ::: "memory");  // B0
    if (nch > 0) read_stage(0);
    for (int c = 0; c < nch; ++c) {
        wait_lgkmcnt0();
        asm volatile("s_barrier" ::: "memory");  // B1(c): LS holds -h_c
        // Bm(c), the compute waves' exchange of B Y in the A form: these waves
        // have no part in it and pass at once, so it never waits for their work.
        if constexpr (AF) asm volatile("s_barrier" ::: "memory");
        wait_vmcnt<0>();  // chunk c's query rows (this wave's only loads)
        Frag<T> qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = q_frag(ks);
        if constexpr (!QREG) wait_lgkmcnt0();  // read out before the next chunk's rows overwrite them
        if (c + 1 < nch) load_q();
        // -(h^T Q^T) from LS (which holds -h_c until B2(c))
        f32x4 inter[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            inter[ct] = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) inter[ct] = mma(xfr(LS, ks * CT + ct), qf[ks], inter[ct]);
        }
        const float eg = __expf(gq);
        wait_lgkmcnt0();
        asm volatile("s_barrier" ::: "memory");  // B2(c): LX holds X_c
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            f32x4 acc = mma(xfr(LX, ct), pf0, zero4());
            if (o >= 2) acc = mma(xfr(LX, CT + ct), pf1, acc);  // P^T rows 32..63 vanish for queries < 32
            *reinterpret_cast<bf16x4*>(LO + ((ct * 4 + o) * 64 + lane) * 8) = cvt4_bf16(acc - eg * inter[ct], p.scale);
        }
        if (c + 1 < nch) read_stage(c + 1);
    }
    wait_lgkmcnt0();
    asm volatile("s_barrier" ::: "memory");  // B_end: the last output tile is in LO
}

template <typename T, int D, bool DEV, int CT, bool FO, bool AF>
__global__ __launch_bounds__((64 * StateStage<T, D, CT, FO, AF>::WAVES)) void chunk_state_h_kernel(const ChunkParams p,
                                                                                                int padded) {
    using SS = StateStage<T, D, CT, FO, AF>;
    constexpr int NT = D / 16;   // column tiles of d_v per head
    constexpr int NTW = NT / CT; // workgroups per head (CT column tiles each)
    constexpr int KS = D / 32;   // contraction steps over d_k
    constexpr int TPW = D / 64;  // S row tiles per compute wave
    constexpr int NST = SS::NST;
    // Work groups of NTW workgroups, one per (bin, value head), the bins
    // heaviest first; group g runs on XCD g % 8 (workgroup i lands on XCD i % 8)
    // with its tiles in consecutive slots, so the tiles of a head share an L2
    // and every XCD gets an even share of heavy and light bins.  A bin is a run
    // of sequences the workgroup scans one after another (one sequence, unless
    // the launch has more sequences than fit on the chip side by side).
    (void)padded;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int gi = (slot / NTW) * 8 + xcd;
    // All of the workgroup's LDS is one array: the stage ring first (at LDS
    // offset 0; with another __shared__ object ahead of it the scan ran 50 ->
    // 73 us at T = 4096 on MI355X), then the exchange, output and query-row
    // buffers, the L2-prefetch sink and, for a device table, its copy.
    constexpr int SINK_OFF = NST * SS::BYTES + SS::EXCH + SS::OBUF + SS::QBUF;
    constexpr int DTAB_OFF = SINK_OFF + 256;
    constexpr int LDS_BYTES = DTAB_OFF + (DEV ? (int)((sizeof(SeqTable) + 15) & ~size_t(15)) : 0);
    static_assert(LDS_BYTES <= SS::LDS_CAP, "LDS of the state scan");
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
    // A device table is copied into LDS first: read from global memory, which
    // the kernel also writes, its entries would be vector loads, and a vector
    // load in a producer wave's cursor would count against the vmcnt that
    // paces the stage loads (its wait would drain the stages in flight).
    if constexpr (DEV) {
        static_assert(sizeof(SeqTable) % 4 == 0, "table copied in words");
        const int32_t* src = reinterpret_cast<const int32_t*>(p.dtab);
        int32_t* dst = reinterpret_cast<int32_t*>(smem + DTAB_OFF);
        for (int i = threadIdx.x; i < (int)(sizeof(SeqTable) / 4); i += blockDim.x) dst[i] = src[i];
        __syncthreads();
    }
    const SeqTable& tab = [&]() -> const SeqTable& {
        if constexpr (DEV)
            return *reinterpret_cast<const SeqTable*>(smem + DTAB_OFF);
        else
            return p.tab;
    }();
    if (gi >= tab.n_bins * p.H_v) return;
    const int tile = slot % NTW;  // column tiles CT tile .. CT tile + CT - 1
    const int h = gi % p.H_v, bin = gi / p.H_v;
    const int kb = tab.bin_first[bin], ke = tab.bin_first[bin + 1];
    int nch = 0;  // chunks of the bin
    for (int k = kb; k < ke; ++k) nch += tab.choff[tab.order[k] + 1] - tab.choff[tab.order[k]];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, grp = lane >> 4;
    const int hq = h / p.G;
    // (chunk, value head) and (chunk, key head) indices of the chunk a cursor is at
    auto vch = [&](const BinCursor& cu) { return (size_t)cu.ci() * p.H_v + h; };
    auto kch = [&](const BinCursor& cu) { return (size_t)cu.ci() * p.H_q + hq; };

    char* const LS = smem + NST * SS::BYTES;  // KS x CT blocks: -S (block ks CT + ct)
    char* const LX = LS + KS * CT * SS::XBLK; // 2 x CT blocks: X (block j CT + ct)
    char* const LY = LX + 2 * CT * SS::XBLK;  // 2 x CT blocks: kf X
    char* const LB = LY + 2 * CT * SS::XBLK;  // A form: 2 x CT blocks: B Y (A's operand type)
    char* const LO = LB + (AF ? 2 : 0) * CT * SS::XBLK;  // FO: output tiles, 8 bytes per (tile ct, wave, lane)
    static_assert(SS::EXCH == (KS + (AF ? 6 : 4)) * CT * SS::XBLK, "exchange blocks: LS, LX, LY (and LB)");
    char* const LQ = LO + SS::OBUF;           // FO, more than one tile: each output wave's query rows
    char* const sink = smem + SINK_OFF;       // L2-prefetch sink
    static_assert(SINK_OFF == (NST * SS::BYTES + SS::EXCH) + SS::OBUF + SS::QBUF, "buffers in order");
    // fragment of lane ln in block b of an exchange buffer
    auto xf = [](char* buf, int b, int ln) -> Frag<T>& {
        return *reinterpret_cast<Frag<T>*>(buf + b * SS::XBLK + ln * (int)sizeof(Frag<T>) + (ln >> 4) * SS::XPAD);
    };
    // Whether the store wave writes h and X (always without the output waves;
    // with them only for inspection).
    const bool store_hx = !FO || p.keep_hx;

    if constexpr (FO) {
        if (w > 4 + SS::NPW) {
            chunk_output_waves<T, D, CT, AF>(p, smem, LS, LX, LO, LQ, w - (5 + SS::NPW), lane, tab, kb, ke, hq, nch);
            return;
        }
    }
    if (w >= 4 + SS::NPW) {
        // ---------------- store wave ----------------
        // Writes the chunk-start states and X to HBM from the compute waves'
        // exchange buffers, so that no global store sits in the compute waves'
        // instruction stream: between B1(c) and B2(c) LS holds bf16(-h_c),
        // between B2(c) and B1(c + 1) LX holds X_c, both in the perm32
        // fragment order (slots 0..3: rows 4g..4g+3 of a 32-row block, slots
        // 4..7: rows 16+4g..16+4g+3, g = lane / 16; column lane % 16).
        constexpr int FQ = sizeof(Frag<T>) / 16;  // 16-byte pieces per fragment
        const unsigned sgn = sizeof(T) == 2 ? 0x80008000u : 0x80000000u;
        // Ht and Xt are written in the fragment order chunk_output_o reads them
        // in (its A operands H^T and X^T, rows d_v: block (d_v tile, K-step),
        // lane 16 g + r holding row r, contraction indices 8 g .. 8 g + 7 of the
        // block), so every store instruction writes 1 KiB of consecutive bytes
        // (whole cache lines) and every load of chunk_output_o reads them the
        // same way.  The pieces are gathered from the fragment-ordered exchange
        // buffers (perm32 contraction order) by lane-permuted LDS reads; bf16:
        // the two 8-byte halves of a piece come from lanes 16 apart, one
        // ds_read2_b64.
        constexpr int EB = (int)sizeof(T);
        constexpr int HPL = KS * FQ, XPL = 2 * FQ;  // 16-byte pieces per lane per chunk
        const unsigned ls0 = lds_addr(LS), lx0 = lds_addr(LX);
        auto xoff = [](int b, int ln) {
            return (unsigned)(b * SS::XBLK + ln * (int)sizeof(Frag<T>) + (ln >> 4) * SS::XPAD);
        };
        unsigned hla[CT][HPL], xla[CT][XPL];  // LDS byte addresses
        unsigned hgo[CT][HPL], xgo[CT][XPL];  // byte offsets in the chunk-head's Ht / Xt block
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int ctile = CT * tile + ct;  // d_v tile
#pragma unroll
            for (int t = 0; t < HPL; ++t) {
                const int ks = t / FQ, e = t % FQ;  // piece: d_k 32 ks + 8 grp + 4 e .. (bf16: 8 values, e = 0)
                if constexpr (EB == 2)
                    hla[ct][t] = ls0 + xoff(ks * CT + ct, 32 * (grp & 1) + r16) + 8 * (grp >> 1);
                else
                    hla[ct][t] = ls0 + xoff(ks * CT + ct, 16 * (2 * (grp & 1) + e) + r16) + 16 * (grp >> 1);
                hgo[ct][t] = (unsigned)(((ctile * KS + ks) * 64 + lane) * 8 * EB + 16 * e);
            }
#pragma unroll
            for (int t = 0; t < XPL; ++t) {
                const int j = t / FQ, e = t % FQ;  // piece: stored positions 32 j + 8 grp + 4 e ..
                xla[ct][t] = lx0 + xoff(j * CT + ct, 16 * grp + r16) + 16 * e;
                xgo[ct][t] = (unsigned)(((ctile * 2 + j) * 64 + lane) * 8 * EB + 16 * e);
            }
        }
        // L2 prefetch: once a step, this workgroup's share of lines of chunk
        // c + PF (4 bytes per line, into a sink nobody reads); the workgroups of
        // a head together touch every line, so by the time the producers stream
        // that chunk it is in L2.  W form: the W and K lines (chunk_prep's
        // output, which the Infinity Cache usually still holds) pay only where
        // the stream comes from HBM (long or many sequences) and cost a few per
        // cent where it does not, so the launcher enables them by size; with one
        // tile a workgroup the output waves' query rows are prefetched too (read
        // only one step ahead, their HBM latency otherwise holds up the first
        // half of every step: T = 65536 scan 1151 -> 1000 us), and so are the
        // tile's share of P, its U block and the gate block (1000 -> 978 us).
        // With four tiles those extra lines cost more than they save.  A form:
        // the K and A lines likewise by size, and the value rows always: nothing
        // upstream reads them, so they come cold from HBM, and the stage ring
        // alone issues them only two steps and a half ahead; with one tile the
        // query rows, P and the gate blocks too where the stream is twice that
        // size (T = 65536 in the A form: 1472 -> 1356 us a call; at T = 8192,
        // below that size, they cost 5 us).
        constexpr int PF = 6;
        constexpr bool XPF = FO && CT == 1;
        constexpr int VRL = D * (int)sizeof(T) / 128;                // lines per value row
        constexpr int VLT = AF ? CHUNK * VRL / NTW : 0;              // value-row lines per workgroup
        constexpr int WLT = SS::W_BYTES / 128 / NTW;                 // lines of W per workgroup
        constexpr int KLT = SS::K_BYTES / 128 / NTW;                 // lines of K (and of the query rows) per workgroup
        constexpr int ALT = SS::A_BYTES / 128 / NTW;                 // lines of A per workgroup
        static_assert(KLT * NTW * 128 == SS::K_BYTES && ALT * NTW * 128 == SS::A_BYTES &&
                          WLT * NTW * 128 == SS::W_BYTES && (!AF || VLT * NTW == CHUNK * VRL),
                      "whole lines per workgroup");
        constexpr int QLT = XPF ? KLT : 0;
        constexpr int PLT = XPF ? SS::P_BYTES / 128 / NTW : 0;
        constexpr int ULT = XPF ? SS::U_BYTES / 128 : 0;
        constexpr int GLT = XPF ? SS::G_BYTES / 128 : 0;
        constexpr int XLT = QLT + PLT + ULT + GLT;                   // the lines for the output waves
        constexpr int NLT = VLT + WLT + KLT + ALT + XLT;
        constexpr int NPL = (NLT + 63) / 64;                         // prefetch loads per lane
        // Output tile of chunk c (FO) from LO to O.  A row of the tile is 32 CT
        // contiguous bytes of O, so 2 CT lanes share a row, 16 bytes each (column
        // tile ct, half hf), and an instruction covers 64 / (2 CT) whole row
        // pieces: every cache line it touches receives all of the workgroup's
        // bytes of that line at once.  (Row by row, 16 bytes of 64 rows an
        // instruction, the stores cost the serial chain about 9 us at T = 4096.)
        // Each piece is gathered from LO, where output wave o's lane 16 g + r
        // holds columns 4 g .. 4 g + 3 of row 16 o + r: the lanes of groups 2 hf
        // and 2 hf + 1, 128 bytes apart.
        BinCursor co, cs, cpf;  // chunks of the next output store, of the step, of the next prefetch
        co.begin(tab, kb, ke);
        cs.begin(tab, kb, ke);
        cpf.begin(tab, kb, ke);
        for (int i = 0; i < PF; ++i) cpf.next();
        auto store_o = [&]() {
            if constexpr (FO) {
                constexpr int LPRW = 2 * CT, RPI = 64 / LPRW;  // lanes per row, rows per instruction
                const int ell = co.ell();
                const int pc = lane % LPRW, ct = pc >> 1, hf = pc & 1;
                u32x4 ov[LPRW];
#pragma unroll
                for (int i = 0; i < LPRW; ++i) {
                    const int row = RPI * i + lane / LPRW;
                    const unsigned a = lds_addr(LO) + (unsigned)((((ct * 4 + (row >> 4)) * 64) + 32 * hf + (row & 15)) * 8);
                    asm volatile("ds_read2_b64 %0, %1 offset1:16" : "=v"(ov[i]) : "v"(a));
                }
                lds_wait_untracked<LPRW>(ov);
                char* o0 = reinterpret_cast<char*>(p.out) +
                           (((size_t)co.token() * p.H_v + h) * D + 16 * (CT * tile + ct) + 8 * hf) * EB;
#pragma unroll
                for (int i = 0; i < LPRW; ++i) {
                    const int row = RPI * i + lane / LPRW;
                    if (row < ell) *reinterpret_cast<u32x4*>(o0 + (size_t)row * p.H_v * D * EB) = ov[i];
                }
                co.next();
            }
        };
        asm volatile("s_barrier" ::: "memory");  // B0
        for (int c = 0; c < nch; ++c) {
            const size_t ch = vch(cs);
            cs.next();
            asm volatile("s_barrier" ::: "memory");  // B1(c)
            if constexpr (AF) asm volatile("s_barrier" ::: "memory");  // Bm(c): passed at once
            if (cpf.valid() && (AF || p.l2_prefetch)) {
                const size_t chp = vch(cpf), kchp = kch(cpf);
                const int nlt = p.l2_prefetch == 0 ? VLT : AF && p.l2_prefetch == 1 ? NLT - XLT : NLT;
#pragma unroll
                for (int q = 0; q < NPL; ++q) {
                    int x = lane + 64 * q;
                    if (x >= nlt) continue;
                    const char* a;
                    if (x < VLT) {  // line li of the head's value rows: row li / VRL, piece li % VRL
                        const int li = tile * VLT + x, row = min(li / VRL, cpf.ell() - 1);
                        a = reinterpret_cast<const char*>(p.v) +
                            ((size_t)(cpf.token() + row) * p.H_v + h) * D * sizeof(T) + 128 * (li % VRL);
                    } else if ((x -= VLT) < WLT) {
                        a = reinterpret_cast<const char*>(p.W) + chp * SS::W_BYTES + (tile * WLT + x) * 128;
                    } else if ((x -= WLT) < KLT) {
                        a = reinterpret_cast<const char*>(p.Kc) + kchp * SS::K_BYTES + (tile * KLT + x) * 128;
                    } else if ((x -= KLT) < ALT) {
                        a = reinterpret_cast<const char*>(p.Af) + chp * SS::A_BYTES + (tile * ALT + x) * 128;
                    } else if ((x -= ALT) < QLT) {  // line of the chunk's query fragments (Qc)
                        a = reinterpret_cast<const char*>(p.Qc) + kchp * SS::K_BYTES + (tile * QLT + x) * 128;
                    } else if ((x -= QLT) < PLT) {
                        a = reinterpret_cast<const char*>(p.Pf) + chp * SS::P_BYTES + (tile * PLT + x) * 128;
                    } else if ((x -= PLT) < ULT) {
                        a = reinterpret_cast<const char*>(p.Ut) + (chp * NT + CT * tile) * SS::U1_BYTES + x * 128;
                    } else {
                        x -= ULT;
                        a = reinterpret_cast<const char*>(p.gates + chp * 4 * CHUNK) + x * 128;
                    }
                    __builtin_amdgcn_global_load_lds((gptr_t)a, (lptr_t)sink, 4, 0, 0);
                }
            }
            cpf.next();
            if constexpr (FO) {
                if (c > 0) store_o();
            }
            if (!store_hx) {
                asm volatile("s_barrier" ::: "memory");  // B2(c)
                continue;
            }
            // h_c = -(LS): a sign flip, exact
            u32x4 hv[CT * HPL];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < HPL; ++t) {
                    if constexpr (EB == 2 && SS::XPAD == 16)  // the two halves, 16 lanes (272 bytes) apart, in one read
                        asm volatile("ds_read2_b64 %0, %1 offset1:34" : "=v"(hv[ct * HPL + t]) : "v"(hla[ct][t]));
                    else if constexpr (EB == 2)  // unpadded: 256 bytes apart
                        asm volatile("ds_read2_b64 %0, %1 offset1:32" : "=v"(hv[ct * HPL + t]) : "v"(hla[ct][t]));
                    else
                        asm volatile("ds_read_b128 %0, %1" : "=v"(hv[ct * HPL + t]) : "v"(hla[ct][t]));
                }
            lds_wait_untracked<CT * HPL>(hv);
            char* Hb = reinterpret_cast<char*>(p.Ht) + ch * D * D * EB;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < HPL; ++t) *reinterpret_cast<u32x4*>(Hb + hgo[ct][t]) = hv[ct * HPL + t] ^ sgn;
            asm volatile("s_barrier" ::: "memory");  // B2(c)
            u32x4 xv[CT * XPL];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < XPL; ++t)
                    asm volatile("ds_read_b128 %0, %1" : "=v"(xv[ct * XPL + t]) : "v"(xla[ct][t]));
            lds_wait_untracked<CT * XPL>(xv);
            char* Xb = reinterpret_cast<char*>(p.Xt) + ch * D * CHUNK * EB;  // X_c, already in the stored perm32 order
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < XPL; ++t) *reinterpret_cast<u32x4*>(Xb + xgo[ct][t]) = xv[ct * XPL + t];
        }
        if constexpr (FO) {
            asm volatile("s_barrier" ::: "memory");  // B_end: the last output tile is in LO
            if (nch > 0) store_o();
        }
        wait_vmcnt<0>();  // no prefetch may land in LDS after the workgroup has ended
        return;
    }
    if (w >= 4) {
        // ---------------- producer waves ----------------
        const int pw = __builtin_amdgcn_readfirstlane(w - 4);  // wave-uniform: scalar branches
        // Outstanding-load bounds (vmcnt counts at most 63): before k loads go
        // out at most 63 - k may be in flight (R*_), and at B2(c) chunk c + 1
        // must have landed (WB_).
        static_assert(SS::NPW <= 2, "the producer code below handles one or two waves");
        constexpr int WB_0 = state_wait_b2<SS>(0), WB_1 = state_wait_b2<SS>(1);
        constexpr int R0_0 = 63 - state_part_loads<SS>(0, 0), R0_1 = 63 - state_part_loads<SS>(1, 0);
        constexpr int R1_0 = 63 - state_part_loads<SS>(0, 1), R1_1 = 63 - state_part_loads<SS>(1, 1);
        constexpr int RC_0 = R0_0 - state_part_loads<SS>(0, 1), RC_1 = R0_1 - state_part_loads<SS>(1, 1);
        static_assert(WB_0 < 64 && WB_1 < 64 && RC_0 >= 0 && RC_1 >= 0, "producer loads exceed the vmcnt range");

        BinCursor cp;  // the chunk whose loads go out next
        cp.begin(tab, kb, ke);
        // Chunks 0 .. NST-1 up front; chunk 0 lands before B0.
#pragma unroll
        for (int b = 0; b < NST; ++b) {
            if (b == 1) wait_vmcnt<0>();
            if (b == 2) {
                if (pw == 0) wait_vmcnt<RC_0>(); else wait_vmcnt<RC_1>();
            }
            if (b < nch) {
                state_issue<T, D, CT, FO, AF>(smem + b * SS::BYTES, p, vch(cp), kch(cp), cp.token(), cp.ell(), h, tile,
                                          lane, pw, 0);
                state_issue<T, D, CT, FO, AF>(smem + b * SS::BYTES, p, vch(cp), kch(cp), cp.token(), cp.ell(), h, tile,
                                          lane, pw, 1);
                cp.next();
            }
        }
        // The producers' barriers are plain s_barrier: a workgroup release fence
        // would wait for the direct-to-LDS loads just issued, and the whole point
        // is that they stay in flight.  Visibility is ensured explicitly: a
        // chunk's loads have completed (vmcnt) before the producer arrives at
        // the barrier after which the compute waves read it.  The asm's memory
        // clobber keeps the compiler from moving loads across a barrier.
        asm volatile("s_barrier" ::: "memory");  // B0: chunks 0 and 1 in LDS
        // A chunk's loads go out in two halves, one in each phase of a step.
        // With three stages the compute waves copy chunk c + 1 into registers
        // between B1(c) and B2(c), so it has landed before B1(c): only chunk
        // c + 2's loads may then be in flight (LA_).  With two stages it is read
        // after B2(c) and lands before that barrier (WB_).
        constexpr int LA_0 = state_part_loads<SS>(0, 0) + state_part_loads<SS>(0, 1);
        constexpr int LA_1 = state_part_loads<SS>(1, 0) + state_part_loads<SS>(1, 1);
        for (int c = 0; c < nch; ++c) {
            if constexpr (NST == 3) {
                if (c + 2 < nch) {
                    if (pw == 0) wait_vmcnt<LA_0>(); else wait_vmcnt<LA_1>();
                } else {
                    wait_vmcnt<0>();
                }
            }
            asm volatile("s_barrier" ::: "memory");  // B1(c): chunk c is in registers, its stage free
            const int cn = c + NST;
            char* stn = smem + (cn % NST) * SS::BYTES;
            const size_t chn = vch(cp), kchn = kch(cp);  // chunk cn
            const int tokn = cp.token(), elln = cp.ell();
            if (cn < nch) {
                if (pw == 0) wait_vmcnt<R0_0>(); else wait_vmcnt<R0_1>();
                state_issue<T, D, CT, FO, AF>(stn, p, chn, kchn, tokn, elln, h, tile, lane, pw, 0);
            }
            if constexpr (AF) asm volatile("s_barrier" ::: "memory");  // Bm(c): after the first half went out
            if (cn < nch) {
                if constexpr (NST != 3) {
                    if (pw == 0) wait_vmcnt<WB_0>(); else wait_vmcnt<WB_1>();
                }
            } else if constexpr (NST != 3) {
                wait_vmcnt<0>();
            }
            asm volatile("s_barrier" ::: "memory");  // B2(c)
            if (cn < nch) {
                if (pw == 0) wait_vmcnt<R1_0>(); else wait_vmcnt<R1_1>();
                state_issue<T, D, CT, FO, AF>(stn, p, chn, kchn, tokn, elln, h, tile, lane, pw, 1);
                cp.next();
            }
        }
        if constexpr (FO) asm volatile("s_barrier" ::: "memory");  // B_end
        return;
    }

    // ---------------- compute waves ----------------
    // This wave's rows of S for the workgroup's column tiles: entry i of
    // [tt][ct] is row 16 (w TPW + tt) + 4 grp + i, column 16 (CT tile + ct) + r16.
    auto s_index = [&](int tt, int ct, int i) {
        return (size_t)(16 * (w * TPW + tt) + 4 * grp + i) * D + 16 * (CT * tile + ct) + r16;
    };
    // initial state of sequence n (zeros without a row)
    auto load_s = [&](int n, f32x4 (&dst)[TPW][CT]) {
        const int si = tab.s_in[n];
        const float* src = p.s0 + ((size_t)max(si, 0) * p.H_v + h) * D * D;
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                if (si < 0) {
                    dst[tt][ct] = zero4();
                    continue;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[tt][ct][i] = src[s_index(tt, ct, i)];
            }
    };
    // final state of sequence n, if it has a row
    auto store_s = [&](int n, const f32x4 (&src)[TPW][CT]) {
        const int so = tab.s_out[n];
        if (so < 0) return;
        float* dst = p.sfinal + ((size_t)so * p.H_v + h) * D * D;
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[s_index(tt, ct, i)] = src[tt][ct][i];
    };
    f32x4 S[TPW][CT];
    // Sequences without tokens end in the state they start from.
    for (int k = kb; k < ke; ++k) {
        const int n = tab.order[k];
        if (tab.choff[n + 1] == tab.choff[n] && tab.s_out[n] >= 0) {
            f32x4 S0[TPW][CT];
            load_s(n, S0);
            store_s(n, S0);
        }
    }
    BinCursor rd;  // the chunk whose stage is read next
    rd.begin(tab, kb, ke);
    auto put_s = [&]() {  // -S into LS, the operand of the next step
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int m = w * TPW + tt;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) lds_put4(xf(LS, (m >> 1) * CT + ct, lane), m & 1, S[tt][ct], -1.f);
        }
    };
    if (nch > 0) {
        load_s(rd.n, S);
        put_s();
    }
    // Operand fragments of one chunk, copied from its LDS stage into registers
    // during the previous step: K's columns (the A operand of K^T (kf X)) and
    // the A operand of the step's first product over d_k, W's rows (W form) or
    // K's rows (A form).
    using PT = ProdT<T>;
    Frag<T> kr[KS], kfg[TPW][2];
    int rell = CHUNK;  // valid length of the chunk last read
    // The rest of a chunk's operands of this wave.  W form: U of its positions,
    // kf of its positions and gamma_l, a step ahead.  A form: its row tile of A,
    // the value rows, beta, beta gamma and kf of its positions, and gamma_l;
    // with one column tile and three stages a step ahead too, so that nothing
    // but the exchanges sits on the serial chain after B1; with more tiles the
    // registers are not there, and they are read from the chunk's own stage at
    // the start of its step (the second half of an A-form stage is refilled
    // only from B2 on).
    constexpr bool AHEAD = !AF || (CT == 1 && NST == 3);
    struct ChunkOps {
        Frag<PT> a0, a1;
        f32x4 v[CT];
        Raw4<PT> u[CT];
        float4 fb, fbg, fx;
        float gl;
    } ops;
    auto read_ops = [&](const char* st, int ell, ChunkOps& o) {
        const float* Gst = reinterpret_cast<const float*>(st + SS::G_OFF);
        if constexpr (AF) {
            const Frag<PT>* Ast = reinterpret_cast<const Frag<PT>*>(st + SS::A_OFF);
            o.a0 = Ast[a_frag_first(w) * 64 + lane];
            if (w >= 2) o.a1 = Ast[(a_frag_first(w) + 1) * 64 + lane];
            if constexpr (AHEAD) {  // else read where they are used (registers)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    o.v[ct] = v_acc4<T>(st + SS::V_OFF + ct * SS::V1_BYTES, 16 * w + 4 * grp, lane);
            }
            o.fb = *reinterpret_cast<const float4*>(Gst + 2 * CHUNK + 16 * w + 4 * grp);
            o.fbg = *reinterpret_cast<const float4*>(Gst + 3 * CHUNK + 16 * w + 4 * grp);
        } else {
            const Raw4<PT>* Ust = reinterpret_cast<const Raw4<PT>*>(st + SS::U_OFF);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                o.u[ct] = Ust[ct * (SS::U1_BYTES / (int)sizeof(Raw4<PT>)) + ((w >> 1) * 64 + lane) * 2 + (w & 1)];
        }
        o.fx = *reinterpret_cast<const float4*>(Gst + CHUNK + 16 * w + 4 * grp);
        o.gl = Gst[ell - 1];
    };
    auto read_stage = [&](int c) {  // chunk c of the bin, at cursor rd
        const char* st = smem + (c % NST) * SS::BYTES;
        if constexpr (AF) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kr[ks] = k_row_frag<T, D>(st + SS::K_OFF, 16 * w, ks, lane);
        } else {
            const Frag<T>* Wst = reinterpret_cast<const Frag<T>*>(st + SS::W_OFF);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kr[ks] = Wst[(w * KS + ks) * 64 + lane];
        }
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) kfg[tt][ks] = k_col_frag<T, D>(st + SS::K_OFF, w * TPW + tt, ks, lane);
        rell = rd.ell();
        if constexpr (AHEAD) read_ops(st, rell, ops);
        rd.next();
    };
    auto bar = [] {  // the compute waves' LDS traffic is all a barrier waits for
        wait_lgkmcnt0();
        asm volatile("s_barrier" ::: "memory");
    };
    // A form: fragment of lane ln in block b of the B Y exchange buffer (A's operand type)
    auto xfb = [&](int b, int ln) -> Frag<PT>& {
        return *reinterpret_cast<Frag<PT>*>(LB + b * SS::XBLK + ln * (int)sizeof(Frag<PT>) + (ln >> 4) * SS::XPAD);
    };
    bar();  // B0: stages 0 and 1 ready
    if (nch > 0) read_stage(0);
    // The bin's sequences one after another (the inner loop is one sequence's
    // chunks; the sequence change stays out of it).  c counts the bin's chunks.
    int c = 0;
    for (int k = kb; k < ke; ++k) {
        const int n = tab.order[k];
        const int nc = tab.choff[n + 1] - tab.choff[n];
        for (int j = 0; j < nc; ++j, ++c) {
            bar();  // B1(c): -S in LS; the first half of chunk c's stage may be refilled
            if constexpr (!AHEAD) read_ops(smem + (c % NST) * SS::BYTES, rell, ops);
            const float gl = ops.gl;
            const float4 fx = ops.fx;
            f32x4 X[CT];
            if constexpr (AF) {
                const Frag<PT> a0 = ops.a0, a1 = ops.a1;
                const f32x4 b4 = f32x4{ops.fb.x, ops.fb.y, ops.fb.z, ops.fb.w};
                const f32x4 bg4 = f32x4{ops.fbg.x, ops.fbg.y, ops.fbg.z, ops.fbg.w};
                // B Y = B (V - Gamma K S) for positions 16 w .. 16 w + 15: LS holds -S,
                // so the product is -(K S) (one independent chain per column tile)
                f32x4 Y[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) Y[ct] = zero4();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) Y[ct] = mma(kr[ks], xf(LS, ks * CT + ct, lane), Y[ct]);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const f32x4 v4 = AHEAD ? ops.v[ct]
                                           : v_acc4<T>(smem + (c % NST) * SS::BYTES + SS::V_OFF + ct * SS::V1_BYTES,
                                                       16 * w + 4 * grp, lane);
                    // beta v + (beta gamma) (-K S), as one rounding of beta v and one
                    // fused multiply-add (fixed, so every work split rounds alike)
                    f32x4 by;
#pragma unroll
                    for (int i = 0; i < 4; ++i) by[i] = __builtin_fmaf(bg4[i], Y[ct][i], b4[i] * v4[i]);
                    lds_put4(xfb((w >> 1) * CT + ct, lane), w & 1, by, 1.f);
                }
                // X = A (B Y) for positions 16 w .. 16 w + 15 (A is lower triangular:
                // row tiles 0 and 1 see positions < 32 only)
                bar();  // Bm(c): all of B Y in LB
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    X[ct] = mma(a0, xfb(ct, lane), zero4());
                    if (w >= 2) X[ct] = mma(a1, xfb(CT + ct, lane), X[ct]);
                }
            } else {
                // X = U - W S for positions 16 w .. 16 w + 15 (one independent chain per column tile)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) X[ct] = raw4_to_f32(ops.u[ct]);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) X[ct] = mma(kr[ks], xf(LS, ks * CT + ct, lane), X[ct]);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                lds_put4(xf(LX, (w >> 1) * CT + ct, lane), w & 1, X[ct], 1.f);
                const f32x4 Yk = f32x4{X[ct][0] * fx.x, X[ct][1] * fx.y, X[ct][2] * fx.z, X[ct][3] * fx.w};
                lds_put4(xf(LY, (w >> 1) * CT + ct, lane), w & 1, Yk, 1.f);
            }
            const float eg = __expf(gl);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) S[tt][ct] *= eg;
            Frag<T> kc[TPW][2];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                kc[tt][0] = kfg[tt][0];
                kc[tt][1] = kfg[tt][1];
            }
            // Three stages: chunk c + 1 has landed before B1(c), and its
            // fragments are read here, while the output waves still work on
            // h_c; two stages: after B2(c).
            if constexpr (NST == 3) {
                if (c + 1 < nch) read_stage(c + 1);
            }
            bar();  // B2(c): all of X in LX and kf X in LY
            if constexpr (NST != 3) {
                if (c + 1 < nch) read_stage(c + 1);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const Frag<T> xb0 = xf(LY, ct, lane), xb1 = xf(LY, CT + ct, lane);
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) {
                    S[tt][ct] = mma(kc[tt][0], xb0, S[tt][ct]);
                    S[tt][ct] = mma(kc[tt][1], xb1, S[tt][ct]);
                }
            }
            if (j + 1 < nc) put_s();
        }
        if (nc == 0) continue;  // (its final state was written above)
        // Sequence end, after B2 of its last chunk: its final state leaves, and
        // the initial state of the bin's next sequence with tokens becomes S
        // before B1 of the next step.  Loads go out before the stores: vmcnt
        // counts stores too, so loads issued after them would also wait for
        // the stores' acknowledgements.
        if (c < nch) {
            int k2 = k + 1;  // exists: chunks remain
            while (tab.choff[tab.order[k2] + 1] == tab.choff[tab.order[k2]]) ++k2;
            f32x4 S0[TPW][CT];
            load_s(tab.order[k2], S0);
            store_s(n, S);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) S[tt][ct] = S0[tt][ct];
            put_s();
        } else {
            store_s(n, S);
        }
    }
    if constexpr (FO) bar();  // B_end
}

// ---------------------------------------------------------------------------
// 4. chunk_output_o: one workgroup (4 waves) per (chunk, value head).  Computes
//    O^T = scale [ (H^T Q^T) diag(gamma) + (U - W S)^T P^T ],
//    P^T[j][i] = (k_j . q_i) exp(gc_i - gc_j) for j <= i  (Lower keeps the diagonal).
//    Q and K are staged in LDS once; wave w forms the P^T tiles of query block w
//    and publishes them in operand order; then each wave produces its 16-row
//    tiles of O^T (d_v rows) for all 64 positions, one 16-position tile at a
//    time, which goes through LDS and leaves as rows of O.  With the read-out
//    epilogue (trace page, Decode-GDN node 8; node 18 of the prefill graph)
//    each position's sum of squares over d_v is reduced across the lanes and
//    waves on the way, and out = o / sqrt(mean o^2 + eps) * weight * silu(z)
//    is stored instead of o.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct OutLds {
    static constexpr int KP = D + 16 / (int)sizeof(T);
    T Q[CHUNK][KP];
    union {
        T K[CHUNK][KP];  // until the P tiles are formed
        struct {
            Frag<T> P[4][2][64];  // B operand of (U - W S)^T P^T: [query tile][K-step][lane]
            float ss[4][CHUNK];   // gated read-out: per-wave sums of o^2 per position
            T os[2][16][D];       // one position tile of O (rows: positions), two buffers;
                                  // 16-byte piece i of row r stored at i ^ (r % pieces)
        } pr;
    } u;
    float gc[CHUNK];
};

template <typename T, int D, bool GATED, bool DEV>
__global__ __launch_bounds__(256) void chunk_output_o_kernel(const ChunkParams p, int padded) {
    using OL = OutLds<T, D>;
    constexpr int KS = D / 32;
    constexpr int TPW = D / 64;
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int NV = CHUNK * D / VEC / 256;
    const SeqTable& tab = DEV ? *p.dtab : p.tab;
    const int work = tab.n_chunks * p.H_v;
    if constexpr (DEV) padded = (work + 7) & ~7;  // the grid was sized by a bound
    if ((int)blockIdx.x >= padded) return;
    const int wid = xcd_remap(blockIdx.x, padded);
    if (wid >= work) return;
    const int h = wid % p.H_v;
    const ChunkPos cp = locate_chunk(tab, tab.chunk_begin + wid / p.H_v);
    const int hq = h / p.G;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int ell = cp.ell;
    const size_t ch = (size_t)cp.ci * p.H_v + h;

    __shared__ __attribute__((aligned(16))) OL s;

    // Q and K rows into LDS (zeros past the valid length), gates.  K comes from
    // chunk_prep's contiguous copy Kc (already L2-normalised with the front end,
    // zero past the valid length); Q rows are L2-normalised on the way with the
    // front end, as in chunk_prep.
    const T* qb = reinterpret_cast<const T*>(p.q) + (size_t)cp.t0 * p.H_q * D + (size_t)hq * D;
    const T* kcb = reinterpret_cast<const T*>(p.Kc) + ((size_t)cp.ci * p.H_q + hq) * CHUNK * D;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int e = tid + 256 * j, r = e / (D / VEC), c = (e % (D / VEC)) * VEC;
        float4 qv = r < ell ? *reinterpret_cast<const float4*>(qb + (size_t)r * p.H_q * D + c) : make_float4(0, 0, 0, 0);
        const float4 kv = *reinterpret_cast<const float4*>(kcb + r * D + VEC * ((c / VEC) ^ kswz<T, D>(r)));
        if (p.fa) qv = l2norm_piece<T, D>(qv);
        *reinterpret_cast<float4*>(&s.Q[r][c]) = qv;
        *reinterpret_cast<float4*>(&s.u.K[r][c]) = kv;
    }
    if (tid < CHUNK) s.gc[tid] = p.gates[ch * 4 * CHUNK + tid];
    lds_sync();
    // This wave's operand fragments of H^T and (U - W S)^T (rows d_v), straight to
    // registers; issued after the Q/K staging (needed first, by the P tiles), so
    // they land while the P tiles are formed (36.6 -> 35 us at T = 4096).
    const T* Hb = reinterpret_cast<const T*>(p.Ht) + ch * D * D;
    const T* Xb = reinterpret_cast<const T*>(p.Xt) + ch * D * CHUNK;
    Frag<T> hf[TPW][KS], xf[TPW][2];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int m = w * TPW + tt;  // d_v tile
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load8(hf[tt][ks], Hb + ((size_t)(m * KS + ks) * 64 + lane) * 8);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) load8(xf[tt][ks], Xb + ((size_t)(m * 2 + ks) * 64 + lane) * 8);
    }
    // Read-out: each position tile of O is staged in LDS and leaves as whole
    // 16-byte pieces of rows, wave w storing rows 4 w .. 4 w + 3 (piece q of
    // the wave: row 4 w + q / PPR, piece q % PPR), so a store instruction
    // writes consecutive bytes of a row.  With the gated read-out the same
    // lanes load the matching pieces of z (rows past the valid length re-read
    // the last valid row; they are never stored) and apply the norm there; a
    // lane's pieces all have the same columns, so its norm weights are loaded
    // once.  Tile 0's z goes out after the Q/K staging (so those loads are not
    // queued behind it); each later tile's while the previous one is computed.
    constexpr int VE = 16 / (int)sizeof(T);         // elements per piece
    constexpr int PPR = D / VE;                     // pieces per row
    constexpr int PL = (4 * PPR + 63) / 64;         // pieces per lane
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    u32x4_t zc[GATED ? PL : 1], zn[GATED ? PL : 1];
    float wvp[GATED ? VE : 1];
    const T* zb = GATED ? reinterpret_cast<const T*>(p.gz) + (size_t)cp.t0 * p.H_v * D + (size_t)h * D : nullptr;
    auto load_z = [&](u32x4_t(&zz)[GATED ? PL : 1], int nt) {
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            const int q = lane + 64 * u;
            if (q < 4 * PPR) {
                const int pos = min(16 * nt + 4 * w + q / PPR, ell - 1);
                zz[u] = *reinterpret_cast<const u32x4_t*>(zb + (size_t)pos * p.H_v * D + (q % PPR) * VE);
            }
        }
    };
    if constexpr (GATED) {
        load_z(zc, 0);
#pragma unroll
        for (int e = 0; e < VE; ++e) wvp[e] = p.gw[(lane % PPR) * VE + e];
    }

    // P^T tiles (I, J = w) for I <= w, held in registers until every wave is
    // done with K, then published over K as B fragments for query tile w.
    f32x4 pt[4];
    {
        Frag<T> qw[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load8(qw[ks], &s.Q[16 * w + r16][32 * ks + 8 * grp]);
        const int pos = 16 * w + r16;
        const float gq = s.gc[pos];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 c = zero4();
            if (I <= w) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    Frag<T> kf;
                    load8(kf, &s.u.K[16 * I + r16][32 * ks + 8 * grp]);
                    c = mma(kf, qw[ks], c);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pj = 16 * I + 4 * grp + i;
                pt[I][i] = (pj <= pos && pos < ell) ? c[i] * __expf(gq - s.gc[pj]) : 0.f;
            }
        }
    }
    lds_sync();  // K is dead
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        // rows pos' 16 I + 4 grp + i: K-step I / 2, slots 4 (I % 2) + i
        if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(&s.u.pr.P[w][I >> 1][lane]) + 4 * (I & 1)) =
                cvt4_bf16(pt[I], 1.f);
        } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(&s.u.pr.P[w][I >> 1][lane]) + 4 * (I & 1)) =
                make_float4(pt[I][0], pt[I][1], pt[I][2], pt[I][3]);
        }
    }
    lds_sync();

    // Output tiles: rows d_v (this wave's tiles), columns pos, one position tile
    // at a time.  With the read-out epilogue, each position's sum of o^2 is
    // reduced over this lane's values, the four lanes sharing a position (grp)
    // and the four waves (through LDS, behind the tile's one barrier).
    T* ob = reinterpret_cast<T*>(p.out) + (size_t)cp.t0 * p.H_v * D + (size_t)h * D;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        if constexpr (GATED) {
            if (nt + 1 < 4) load_z(zn, nt + 1);
        }
        Frag<T> qf[KS], pf[2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load8(qf[ks], &s.Q[16 * nt + r16][32 * ks + 8 * grp]);
        pf[0] = s.u.pr.P[nt][0][lane];
        pf[1] = s.u.pr.P[nt][1][lane];
        const int pos = 16 * nt + r16;
        const float eg = __expf(s.gc[pos]);
        float ssq = 0.f;
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            f32x4 inter = zero4(), intra = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) inter = mma(hf[tt][ks], qf[ks], inter);
            intra = mma(xf[tt][0], pf[0], intra);
            if (nt >= 2) intra = mma(xf[tt][1], pf[1], intra);  // P^T rows 32..63 vanish for queries < 32
            f32x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = p.scale * (eg * inter[i] + intra[i]);
            if constexpr (GATED) {
#pragma unroll
                for (int i = 0; i < 4; ++i) ssq += ov[i] * ov[i];
            }
            // 4 values of row r16 (position), columns 16 (w TPW + tt) + 4 grp ..
            const int col = 16 * (w * TPW + tt) + 4 * grp;
            store4(&s.u.pr.os[nt & 1][r16][((col / VE) ^ (r16 % PPR)) * VE + col % VE], ov[0], ov[1], ov[2], ov[3]);
        }
        if constexpr (GATED) {  // this wave's share of each position's sum of o^2 over d_v
            ssq += wave_shfl_xor(ssq, 16);
            ssq += wave_shfl_xor(ssq, 32);
            if (grp == 0) s.u.pr.ss[w][pos] = ssq;
        }
        // One barrier a tile: buffer nt & 1 is rewritten two tiles later, after
        // the next tile's barrier.
        lds_sync();
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            const int q = lane + 64 * u;
            if (q < 4 * PPR) {
                const int row = 4 * w + q / PPR, pc = q % PPR, pr = 16 * nt + row;
                const float4 raw = *reinterpret_cast<const float4*>(&s.u.pr.os[nt & 1][row][(pc ^ (row % PPR)) * VE]);
                float4 outv = raw;
                if constexpr (GATED) {
                    const float rstd =
                        1.f / sqrtf((s.u.pr.ss[0][pr] + s.u.pr.ss[1][pr] + s.u.pr.ss[2][pr] + s.u.pr.ss[3][pr]) *
                                        (1.f / D) + p.geps);
                    float o[VE], zf[VE];
                    if constexpr (sizeof(T) == 2) {
                        const bf16x8 ob8 = __builtin_bit_cast(bf16x8, raw), zb8 = __builtin_bit_cast(bf16x8, zc[u]);
#pragma unroll
                        for (int e = 0; e < VE; ++e) {
                            o[e] = (float)ob8[e];
                            zf[e] = (float)zb8[e];
                        }
                    } else {
                        const float4 zz = __builtin_bit_cast(float4, zc[u]);
                        o[0] = raw.x; o[1] = raw.y; o[2] = raw.z; o[3] = raw.w;
                        zf[0] = zz.x; zf[1] = zz.y; zf[2] = zz.z; zf[3] = zz.w;
                    }
                    float y[VE];
#pragma unroll
                    for (int e = 0; e < VE; ++e) y[e] = o[e] * rstd * wvp[e] * silu_f32(zf[e]);
                    if constexpr (sizeof(T) == 2) {
                        bf16x8 yb;
#pragma unroll
                        for (int e = 0; e < VE; ++e) yb[e] = (bf16)y[e];
                        outv = __builtin_bit_cast(float4, yb);
                    } else {
                        outv = make_float4(y[0], y[1], y[2], y[3]);
                    }
                }
                if (pr < ell) *reinterpret_cast<float4*>(ob + (size_t)pr * p.H_v * D + pc * VE) = outv;
            }
        }
        if constexpr (GATED) {
#pragma unroll
            for (int u = 0; u < PL; ++u) zc[u] = zn[u];
        }
    }
}

// ---------------------------------------------------------------------------
// Gated read-out after the fused output (trace page, node 18 of the prefill
// graph; Decode-GDN node 8): in place over the rows of the launch's tokens,
//     out = o / sqrt(mean o^2 + eps) * weight * silu(z)
// over the d_v values of one (token, value head) row, o being the output as
// stored (rounded to the output dtype, the value the unfused pair of nodes
// hands over).  A row is held by D / 8 (bf16) lanes, 16 bytes each; HBM bound.
// ---------------------------------------------------------------------------
template <typename T, int D, bool DEV>
__global__ __launch_bounds__(256) void chunk_gate_kernel(const ChunkParams p) {
    constexpr int VE = 16 / (int)sizeof(T);  // elements per lane
    constexpr int LPR = D / VE;              // lanes per row
    constexpr int RPB = 256 / LPR;           // rows per workgroup
    const SeqTable& tab = DEV ? *p.dtab : p.tab;
    const int tbeg = tab.cu[0], tend = tab.cu[tab.num_seqs];
    const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;  // (token - tbeg) * H_v + head
    if (row >= (size_t)(tend - tbeg) * p.H_v) return;                 // whole rows leave together
    const int li = threadIdx.x % LPR;
    const size_t off = ((size_t)tbeg * p.H_v + row) * D + (size_t)li * VE;
    T* const ob = reinterpret_cast<T*>(p.out) + off;
    const float4 raw = *reinterpret_cast<const float4*>(ob);
    const float4 zraw = *reinterpret_cast<const float4*>(reinterpret_cast<const T*>(p.gz) + off);
    float o[VE], z[VE];
    if constexpr (sizeof(T) == 2) {
        const bf16x8 ov = __builtin_bit_cast(bf16x8, raw), zv = __builtin_bit_cast(bf16x8, zraw);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            o[e] = (float)ov[e];
            z[e] = (float)zv[e];
        }
    } else {
        o[0] = raw.x; o[1] = raw.y; o[2] = raw.z; o[3] = raw.w;
        z[0] = zraw.x; z[1] = zraw.y; z[2] = zraw.z; z[3] = zraw.w;
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) ss += o[e] * o[e];
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
    const float rstd = 1.f / sqrtf(ss * (1.f / D) + p.geps);
    float y[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) y[e] = o[e] * rstd * p.gw[li * VE + e] * silu_f32(z[e]);
    if constexpr (sizeof(T) == 2) {
        bf16x8 yb;
#pragma unroll
        for (int e = 0; e < VE; ++e) yb[e] = (bf16)y[e];
        *reinterpret_cast<float4*>(ob) = __builtin_bit_cast(float4, yb);
    } else {
        *reinterpret_cast<float4*>(ob) = make_float4(y[0], y[1], y[2], y[3]);
    }
}

// ---------------------------------------------------------------------------
// Sequence tables from a device-resident cu_seqlens (one wave).  Per group of
// up to 64 sequences: sequence ends clamped to [0, T] and made non-decreasing
// (a running maximum, so every length is >= 0 and every index stays inside the
// buffers whatever the input holds), chunk offsets by a prefix sum over the
// lanes, state rows, and the state scan's bins: m = min(sequences, bins_cap)
// bins filled with the sequences longest first in boustrophedon order (round
// r of m sequences goes to bins 0 .. m-1, the next round back from m-1), so
// that every bin's position in order[] has a closed form.  The next group's
// sequence ends are loaded while a group is processed.  The ranks compare each
// lane's chunk count with all others, read back from LDS four at a time (all
// lanes the same address: a broadcast), rather than by one cross-lane shuffle
// per sequence.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void build_tables_kernel(const int32_t* __restrict__ cu, int num_seqs, int T,
                                                         int has_in, int has_out, int bins_cap, SeqTable* tabs) {
    static_assert(MAX_SEQS_PER_LAUNCH == 64, "one lane a sequence");
    __shared__ __attribute__((aligned(16))) int nc_lds[64];
    const int lane = threadIdx.x;
    int chunk_base = 0, prev_end = 0;
    int raw = lane < min(MAX_SEQS_PER_LAUNCH, num_seqs) ? cu[lane + 1] : 0;
    for (int s0 = 0; s0 < num_seqs; s0 += MAX_SEQS_PER_LAUNCH) {
        const int ns = min(MAX_SEQS_PER_LAUNCH, num_seqs - s0);
        SeqTable* tb = tabs + s0 / MAX_SEQS_PER_LAUNCH;
        int end = lane < ns ? min(max(raw, 0), T) : 0;
        {
            const int s1 = s0 + MAX_SEQS_PER_LAUNCH;  // the next group's ends, in flight meanwhile
            raw = s1 + lane < num_seqs ? cu[s1 + lane + 1] : 0;
        }
        end = max(end, prev_end);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {  // inclusive running maximum
            const int o = __shfl_up(end, off, 64);
            if (lane >= off) end = max(end, o);
        }
        const int up = __shfl_up(end, 1, 64);
        const int start = lane == 0 ? prev_end : up;
        const int len = lane < ns ? end - start : 0;
        const int nc = (len + CHUNK - 1) / CHUNK;
        int incl = nc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {  // inclusive prefix sum of chunk counts
            const int o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        const int total = __shfl(incl, ns - 1, 64);
        const int last_end = __shfl(end, ns - 1, 64);
        nc_lds[lane] = nc;  // zero past ns
        __syncthreads();
        int rank = 0;  // stable, longest first
#pragma unroll
        for (int j4 = 0; j4 < 16; ++j4) {
            const int4 v = reinterpret_cast<const int4*>(nc_lds)[j4];
            const int vj[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * j4 + e;
                rank += (j < ns && (vj[e] > nc || (vj[e] == nc && j < lane))) ? 1 : 0;
            }
        }
        __syncthreads();  // all reads done before the next group overwrites nc_lds
        const int m = min(ns, max(bins_cap, 1));
        const int rounds = ns / m, rem = ns % m;  // whole rounds, sequences of the last one
        // first position of bin b in order[]: rounds + 1 sequences for the bins
        // the last round reaches (the first rem, or the last rem when that round
        // runs backwards), rounds for the others
        auto bin_first = [&](int b) {
            return b * rounds + ((rounds & 1) ? max(0, b - (m - rem)) : min(b, rem));
        };
        if (lane < ns) {
            tb->cu[lane] = start;
            tb->choff[lane] = chunk_base + incl - nc;
            tb->s_in[lane] = has_in ? s0 + lane : -1;
            tb->s_out[lane] = has_out ? s0 + lane : -1;
            const int r = rank / m, q = rank % m;
            const int b = (r & 1) ? m - 1 - q : q;
            tb->order[bin_first(b) + r] = lane;
        }
        if (lane < m) tb->bin_first[lane] = bin_first(lane);
        if (lane == 0) {
            tb->bin_first[m] = ns;
            tb->n_bins = m;
            tb->ct = 0;
            tb->cu[ns] = last_end;
            tb->choff[ns] = chunk_base + total;
            tb->num_seqs = ns;
            tb->seq_base = s0;
            tb->chunk_begin = chunk_base;
            tb->n_chunks = total;
        }
        chunk_base += total;
        prev_end = last_end;
    }
}

hipError_t launch_build_tables(const int32_t* cu_dev, int num_seqs, int T, int has_in, int has_out, int bins_cap,
                               SeqTable* tabs, hipStream_t stream) {
    if (num_seqs > 0)
        hipLaunchKernelGGL(build_tables_kernel, dim3(1), dim3(64), 0, stream, cu_dev, num_seqs, T, has_in, has_out,
                           bins_cap, tabs);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Pipeline launcher: the four stages in stream order.
// ---------------------------------------------------------------------------
static inline int pad8(int x) { return (x + 7) & ~7; }

// Compute units of the current device (cached per device), a multiple of 8 on
// this chip (eight XCDs).
int cu_count() {
    static std::atomic<int> cached[64];  // zero-initialised; concurrent callers store the same value
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cached[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        c = pad8(n);
        cached[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

template <typename T, int D>
hipError_t launch_chunk_pipeline(const ChunkParams& p, hipStream_t stream, hipEvent_t const* events) {
    const int work_ch = p.tab.n_chunks * p.H_v;
    const int grid_ch = pad8(work_ch);
    const int groups = p.tab.n_bins * p.H_v;  // (bin, value head) pairs of the state scan
    // Column tiles per state-scan workgroup, as the bins were packed for (fp32:
    // one); a step's W and K stream serves 2 or 4 tiles.
    const int ct = sizeof(T) != 2 ? 1 : p.tab.ct == 4 ? 4 : p.tab.ct == 2 ? 2 : 1;
    // With events, each kernel is launched with hipExtLaunchKernelGGL, whose
    // start/stop events are stamped by the kernel's own dispatch (kernel time
    // only, no launch gaps).
    auto launch = [&](int k, auto kernel, int grid, int block, int padded, const ChunkParams& kp) {
        if (events)
            hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, stream, events[2 * k], events[2 * k + 1], 0, kp,
                                  padded);
        else
            hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, stream, kp, padded);
    };
    // The state scan's L2 prefetch pays when its W / K / U stream no longer
    // fits in the 256 MB Infinity Cache next to the layer's other tensors: on
    // above 128 MiB of stream (level 1), and in the A form the output waves'
    // lines too above 256 MiB (level 2).
    ChunkParams pl = p;
    const size_t stage_stream = (size_t)work_ch * StateStage<T, D>::BYTES;
    pl.l2_prefetch = stage_stream > (size_t(256) << 20) ? 2 : stage_stream > (size_t(128) << 20) ? 1 : 0;
    // The form of the chunk's operands the state scan reads (decided by the
    // host from the call's sequence count; fp32 always W and U).
    const bool af = sizeof(T) == 2 && p.aform;
    pl.write_af = af ? 1 : 0;
    // chunk_prep keeps the query rows (Qc) where the state scan reads them: one
    // column tile a workgroup, or the front end's normalised rows.
    pl.Qc = (p.fa || ct == 1) ? p.Qc : nullptr;
    // chunk_prep: with few items a slot, as many workgroups as fit on the chip at
    // once (four per CU), each looping over its items and prefetching the next
    // one (T = 4096, two items a slot: 36 against 38 us with one workgroup an
    // item); with many, one workgroup an item, which the dispatcher staggers
    // (packed 8-sequence batch, 16 items a slot: 199 against 208 us).
    const int prep_slots = 4 * cu_count();
    const int prep_grid = work_ch > 8 * prep_slots ? grid_ch : std::min(grid_ch, prep_slots);
    // bf16: chunk_output_o's work runs inside the state scan (output waves), so
    // the chunk-start states and U - W S never leave the chip; the gated
    // read-out is then a row pass over the output.  fp32 keeps the separate
    // output kernel (a stage with the query rows would not fit in LDS twice).
    constexpr bool FO = sizeof(T) == 2;
    auto run = [&](auto dev) {
        constexpr bool DEV = decltype(dev)::value;
        if (work_ch > 0) {
            if (!af || p.keep_wu)
                launch(0, chunk_prep_kernel<T, D, DEV, true>, prep_grid, 256, grid_ch, pl);
            else
                launch(0, chunk_prep_kernel<T, D, DEV, false>, prep_grid, 256, grid_ch, pl);
        }
        // grids: whole groups of workgroups on each XCD
        auto state = [&](auto ctc, auto afc) {
            constexpr int CT = decltype(ctc)::value;
            constexpr bool AF = decltype(afc)::value;
            const int grid = pad8(groups) * (D / 16 / CT);
            launch(1, chunk_state_h_kernel<T, D, DEV, CT, FO, AF>, grid, 64 * StateStage<T, D, CT, FO, AF>::WAVES, grid,
                   pl);
        };
        auto state_ct = [&](auto afc) {
            if (ct == 4)
                state(std::integral_constant<int, 4>{}, afc);
            else if (ct == 2)
                state(std::integral_constant<int, 2>{}, afc);
            else
                state(std::integral_constant<int, 1>{}, afc);
        };
        if (groups > 0) {
            if constexpr (sizeof(T) == 2) {
                if (af)
                    state_ct(std::true_type{});
                else
                    state_ct(std::false_type{});
            } else {
                state(std::integral_constant<int, 1>{}, std::false_type{});
            }
        }
        if (work_ch > 0) {
            if constexpr (!FO) {
                if (p.gz)
                    launch(2, chunk_output_o_kernel<T, D, true, DEV>, grid_ch, 256, grid_ch, pl);
                else
                    launch(2, chunk_output_o_kernel<T, D, false, DEV>, grid_ch, 256, grid_ch, pl);
            } else if (p.gz) {
                constexpr int RPB = 256 / (D * (int)sizeof(T) / 16);
                const int64_t rows = (int64_t)(DEV ? p.T : p.tab.cu[p.tab.num_seqs] - p.tab.cu[0]) * p.H_v;
                const int grid = (int)((rows + RPB - 1) / RPB);
                auto gate_kernel = chunk_gate_kernel<T, D, DEV>;
                if (grid > 0 && events)
                    hipExtLaunchKernelGGL(gate_kernel, dim3(grid), dim3(256), 0, stream, events[4], events[5], 0, pl);
                else if (grid > 0)
                    hipLaunchKernelGGL(gate_kernel, dim3(grid), dim3(256), 0, stream, pl);
                else if (events) {
                    (void)hipEventRecord(events[4], stream);
                    (void)hipEventRecord(events[5], stream);
                }
            } else if (events) {  // no third kernel: its two events mark the same point
                (void)hipEventRecord(events[4], stream);
                (void)hipEventRecord(events[5], stream);
            }
        }
    };
    if (p.dtab)
        run(std::true_type{});
    else
        run(std::false_type{});
    return hipGetLastError();
}

template hipError_t launch_chunk_pipeline<bf16, 128>(const ChunkParams&, hipStream_t, hipEvent_t const*);
template hipError_t launch_chunk_pipeline<bf16, 64>(const ChunkParams&, hipStream_t, hipEvent_t const*);
template hipError_t launch_chunk_pipeline<float, 128>(const ChunkParams&, hipStream_t, hipEvent_t const*);
template hipError_t launch_chunk_pipeline<float, 64>(const ChunkParams&, hipStream_t, hipEvent_t const*);

}  // namespace gdn
