// Launch parameters shared by the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;

// Sequences handled by one launch of the chunk pipeline.  A packed batch with
// more sequences is processed in several launches over disjoint sequence
// ranges (sequences are independent, so this is exact).
constexpr int MAX_SEQS_PER_LAUNCH = 64;

// Per-launch sequence table, passed by value in the kernel arguments so that
// no host->device copy (and no host synchronisation) is needed per call.
struct SeqTable {
    int32_t num_seqs;     // sequences in this launch
    int32_t seq_base;     // global index of the first one (indexes the state arrays)
    int32_t chunk_begin;  // global index of its first chunk
    int32_t n_chunks;     // chunks in this launch
    int32_t cu[MAX_SEQS_PER_LAUNCH + 1];     // global token offsets
    int32_t choff[MAX_SEQS_PER_LAUNCH + 1];  // global chunk offsets, choff[num_seqs] = chunk_begin + n_chunks
    int32_t s_in[MAX_SEQS_PER_LAUNCH];       // row of the initial-state array a sequence starts from, -1: zeros
    int32_t s_out[MAX_SEQS_PER_LAUNCH];      // row of the final-state array it ends in, -1: none
    int32_t order[MAX_SEQS_PER_LAUNCH];      // sequences of each state-scan bin, bin by bin (see bin_first)
    // State-scan bins: a workgroup of the scan walks the sequences of one bin
    // (order[bin_first[b]] .. order[bin_first[b + 1] - 1]) one after another for
    // its value head and column tiles.  ct: column tiles per scan workgroup the
    // bins were packed for (0: the launcher chooses, one sequence per bin).
    int32_t n_bins;
    int32_t ct;
    int32_t bin_first[MAX_SEQS_PER_LAUNCH + 1];
};

struct ChunkParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* s0;  // may be null
    void* out;
    float* sfinal;  // may be null
    // workspace regions
    float* gates;  // per (chunk, value head): [4][64] fp32 rows gc, kf = gamma_l / gamma, beta, beta gamma
    void* A;       // per (chunk, value head): A row-major, only under keep_A
    void* Af;      // per (chunk, value head): the six A fragments the state scan multiplies B Y by
    void* W;       // per (chunk, value head): W = A B Gamma K, only under keep_wu
    void* Ut;      // per (chunk, value head): U = A B V, only under keep_wu
    void* Kc;      // per (chunk, key head): the chunk's key rows for the state scan
    void* Ht;
    void* Xt;
    void* Pf;   // per (chunk, value head): P as the output's B operands (bf16; null: P not formed)
    void* Qc;   // per (chunk, key head): the query rows as the output waves' operand fragments (bf16; else null)
    int32_t H_q, H_v, G;
    float scale;
    int32_t keep_A;  // nonzero: chunk_prep also writes A to the workspace
    int32_t keep_wu;  // nonzero: chunk_prep also forms W and U and writes them to the workspace
    int32_t write_af;  // nonzero: chunk_prep forming W and U also writes A's fragments (set by the launcher)
    int32_t aform;     // nonzero (bf16): the state scan forms X from A and the raw rows instead of W and U
    int32_t keep_hx;  // nonzero: the state scan writes Ht, Xt even where the output is formed on chip
    int32_t T;       // tokens of the whole batch (bounds the gated read-out's rows on the device-table path)
    int32_t l2_prefetch;  // chunk_state_h's L2 prefetch: 0 off, 1 the stage lines, 2 also the output waves' (launcher)
    // optional read-out epilogue out = rmsnorm(o) * gw * silu(gz) (gz null: none)
    const void* gz;
    const float* gw;
    float geps;
    // optional front end (fa null: none): q, k are raw and L2-normalised in the
    // kernels; g, beta come from fa, fb (dtype [T, H_v]) with A_log, dt_bias [H_v]
    const void* fa;
    const void* fb;
    const float* A_log;
    const float* dt_bias;
    SeqTable tab;
    // Device-resident copy of the table (built from a device cu_seqlens by
    // build_tables_kernel); when set, the kernels read it instead of tab, and
    // tab.num_seqs / tab.n_chunks only bound the grids.
    const SeqTable* dtab;
};

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* slot;  // state row of each sequence (null: row n); < 0 or >= pool: padding
    int32_t pool;         // rows in the state array
    const float* g;       // plain step: per (n, h) log gate
    const float* beta;    // plain step: per (n, h) beta
    const void* a;        // fused step: per (n, h) gate input, dtype of q
    const void* b;        // fused step: per (n, h) beta input, dtype of q
    const float* A_log;   // fused step: per value head
    const float* dt_bias; // fused step: per value head
    float* state;
    void* out;
    const void* gz;  // optional read-out epilogue (fused step only), as in ChunkParams
    const float* gw;
    float geps;
    int32_t N, H_q, H_v, G;
    float scale;
};

// Causal conv1d + SiLU (gdn_conv.hip).  Prefill: x, y [T, C]; s_in, s_out
// [num_seqs, K-1, C] (either may be null).  Step: x, y [N, C]; s_out is the
// history, updated in place.  w [C, K] fp32 (oldest tap first), b [C] or null.
struct ConvParams {
    const void* x;
    void* y;
    const float* w;
    const float* b;
    const void* s_in;
    void* s_out;
    int32_t C;
    int32_t q0;    // prefill: first quarter-chunk of this launch
    const int32_t* slot;  // step: history row of each sequence (null: row n); < 0 or >= pool: padding
    int32_t pool;
    SeqTable tab;  // prefill only
};

// Pool row maintenance (gdn_pool.hip): for each listed entry i, row dst[i] of
// the pool receives row src[i] (src null: zeros); entries with a row outside
// [0, pool) are skipped.
struct PoolRowsParams {
    char* base;
    const int32_t* src;
    const int32_t* dst;
    int32_t pool;
    int32_t i0;    // first entry of this launch
    size_t row16;  // row size in 16-byte units
};

// Kernel launchers (defined in the .hip translation units).  T is float or
// __bf16, D is d_k = d_v.  `events` is null or six events: start and stop of
// each of the three chunk kernels.
template <typename T, int D>
hipError_t launch_chunk_pipeline(const ChunkParams& p, hipStream_t stream, hipEvent_t const* events);

template <typename T, int D, bool FUSED>
hipError_t launch_recurrent_step(const DecodeParams& p, hipStream_t stream);

// Sequence tables from a device cu_seqlens (gdn_chunk.hip): one SeqTable per
// group of up to MAX_SEQS_PER_LAUNCH sequences, boundaries clamped to [0, T]
// and made non-decreasing so that no kernel can index out of bounds.
// bins_cap: state-scan bins a launch group may use (at most one sequence a bin)
hipError_t launch_build_tables(const int32_t* cu_dev, int num_seqs, int T, int has_in, int has_out, int bins_cap,
                               SeqTable* tabs, hipStream_t stream);

template <typename T, int K>
hipError_t launch_conv_prefill(const ConvParams& p, hipStream_t stream);
template <typename T, int K>
hipError_t launch_conv_step(const ConvParams& p, int N, hipStream_t stream);

hipError_t launch_pool_rows(PoolRowsParams p, int32_t n, hipStream_t stream);

// Records e as this thread's last HIP error (named by gdn_strerror) and returns
// GDN_ELAUNCH (gdn_api.cpp).
int hip_fail(hipError_t e);
// Compute units of the current device (a multiple of 8).
int cu_count();

}  // namespace gdn
