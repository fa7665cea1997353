/*
 * gdn.h — Gated DeltaNet forward pass on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libgdn.so.  Two operations:
 *
 *   gdn_chunk_fwd       chunk-wise parallel prefill over packed variable-length
 *                       sequences (chunk size C = 64), with optional initial
 *                       states and returned final states;
 *   gdn_recurrent_step  one recurrent decode step for a batch of fp32 states,
 *                       updated in place.
 *
 * Notation (row vectors): q_t, k_t in R^{1 x d_k}, v_t in R^{1 x d_v},
 * S in R^{d_k x d_v}.  The recurrence both calls compute is the Gated DeltaNet
 * rule of "实验三：GDN Prefill 前向优化" (section "GLA, DeltaNet 与 Gated
 * DeltaNet"):
 *
 *     Sbar_t = alpha_t S_{t-1},   S_t = Sbar_t + beta_t k_t^T (v_t - k_t Sbar_t),
 *     o_t    = scale * q_t S_t        (the read sees the updated state)
 *
 * with alpha_t = exp(g_t); g is the per-token log decay (raw_g on that page,
 * section "输入输出定义"), never a cumulative sum.  `scale` is the 1/sqrt(d_k)
 * factor of the chunk output formula (section "计算过程描述"); callers pass it
 * explicitly so prefill and decode agree.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless the name ends in _host.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous on that stream; the library never synchronises and never
 *     allocates or frees memory: all buffers are owned by the caller.
 *   - Layouts are row-major with the last dimension contiguous:
 *       q, k   [T, H_q, d_k]          v, out [T, H_v, d_v]
 *       g, beta [T, H_v]  (always fp32)
 *       states  [N, H_v, d_k, d_v]  (always fp32, d_v contiguous)
 *     Value head h reads query/key head floor(h / (H_v / H_q)) (GVA grouping,
 *     section "输入输出定义" of the same page).
 *   - q, k, v and out share one element type, `dtype`.
 *   - Every device pointer must be 16-byte aligned.
 *   - Arguments are validated before any work is queued; on any error nothing
 *     is written and a negative status is returned.  There is no fallback path.
 *   - Supported shapes: d_k == d_v in {64, 128}; H_v a multiple of H_q.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_dtype {
    GDN_F32 = 0,  /* IEEE binary32 */
    GDN_BF16 = 1, /* bfloat16, round-to-nearest-even on output */
} gdn_dtype;

enum {
    GDN_OK = 0,
    GDN_EINVAL = -1,       /* NULL / inconsistent arguments, bad cu_seqlens */
    GDN_EUNSUPPORTED = -2, /* d_k != d_v, d not in {64,128}, H_v % H_q != 0, misaligned pointer */
    GDN_EWORKSPACE = -3,   /* workspace NULL or smaller than gdn_chunk_fwd_workspace_size() */
    GDN_ELAUNCH = -4,      /* a HIP launch failed; gdn_strerror() names the HIP error */
};

/* The HIP runtime's stream handle, declared here as the runtime declares it so
 * that callers need not include the HIP headers to use this one. */
typedef struct ihipStream_t *hipStream_t;

/* Chunk length of the prefill (fixed; section "Chunk-wise Parallel"). */
#define GDN_CHUNK 64

/*
 * Workspace of gdn_chunk_fwd.  One region per intermediate of the chunk form
 * (section "计算过程描述": g^cumsum, A, W, U, the chunk-start states, U - W S)
 * and per operand block the state scan reads, each starting on a 256-byte
 * boundary.  The intermediates stay in the workspace after the call and may be
 * read back for inspection; chunks are numbered in sequence order, each
 * sequence's chunks starting at its own first token, so chunk c of sequence n
 * has global index chunk_offset(n) + c where chunk_offset(n) = sum_{m<n}
 * ceil(L_m / 64).  Positions beyond a tail chunk's valid length hold zeros.
 *
 * The state scan forms X = U - W S in one of two ways (gdn_chunk_fwd_form
 * tells which for a call; gdn_chunk_fwd_ex can force either):
 *   W form: chunk_prep writes W and U, and the scan reads them;
 *   A form: chunk_prep writes A's fragments (Af) instead, and the scan forms
 *           X = A B (V - Gamma K S) from them and the raw K and V rows, since
 *           U - W S = A B V - A B Gamma K S.
 * W and U are written in the W form, or with GDN_FWD_KEEP_WU; Af only in the A
 * form; A only with GDN_FWD_KEEP_A.  Unwritten regions are left untouched.
 *
 * W, U, Af, Ht and Xt are kept in the order in which the MFMA units consume
 * them ("fragment order", 8 values per lane of a 64-lane wave; for an index i
 * let i = 32 s + 16 h + 4 a + b with a, b in 0..3):
 *   W   element (pos, k):  ((pos/16 * (d_k/32) + s(k)) * 64 + 16 a(k) + pos%16) * 8 + 4 h(k) + b(k)
 *   U   element (pos, j):  ((j/16 * 2 + pos/32) * 64 + 16 ((pos%16)/4) + j%16) * 8 + 4 ((pos/16)%2) + pos%4
 *   Af  element (i, j), j <= i: fragment f of (row tile i/16, K-step j/32) in
 *       the order (0,0), (1,0), (2,0), (2,1), (3,0), (3,1): (f * 64 + 16 a(j) + i%16) * 8 + 4 h(j) + b(j)
 * "perm32" means: within every block of 32 consecutive indices, index
 * 16 h + 4 a + b is stored at offset 8 a + 4 h + b.
 *
 *   gates fp32 [n_chunks][H_v][4][64]        per position: the inclusive in-chunk cumsum of g
 *                                            (gc), gamma_l / gamma (kf: the decay of a key to
 *                                            the chunk end; the state update is
 *                                            S <- gamma_l S + Kc^T Diag(kf) X), beta, and
 *                                            beta gamma; all zero past the valid length
 *   A   dtype [n_chunks][H_v][64][64]        (I + StrictLower(B Gamma K K^T Gamma^-1))^-1,
 *                                            written only under GDN_FWD_KEEP_A (gdn_chunk_fwd_ex)
 *   W   dtype [n_chunks][H_v][64 * d_k]      A B Gamma K, fragment order
 *   U   utype [n_chunks][H_v][64 * d_v]      A B V, fragment order; utype is IEEE binary16
 *                                            for bf16 inputs (the same two bytes, three more
 *                                            mantissa bits; W, U and X are formed from binary16
 *                                            operands, so |beta v|, the entries of A and of U
 *                                            must stay below 65504), fp32 for fp32 inputs
 *   Kc  dtype [n_chunks][H_q][64][d_k]       the chunk's key rows (L2-normalised with
 *                                            gdn_chunk_fwd_fused), the 16-byte pieces of row
 *                                            r permuted: piece i stored at i ^ p(r), where
 *                                            with P = d_k * sizeof(dtype) / 16 pieces a row
 *                                            p(r) = 2 (r mod P/2) for bf16 and
 *                                            4 ((r / 4) mod P/4) for fp32
 *   Ht  dtype [n_chunks][H_v][d_v * d_k]     (state at chunk start)^T, element (j, k) at
 *                                            ((j/16 * (d_k/32) + k/32) * 64 + 16 ((k%32)/8) + j%16) * 8 + k%8
 *   Xt  dtype [n_chunks][H_v][d_v * 64]      (U - W S)^T, element (j, pos) at the same place
 *                                            with d_k -> 64 and k -> perm32(pos)
 *   P   bf16  [n_chunks][H_v][6][64][8]      (bf16 only; empty for fp32) P[i][j] =
 *                                            (q_i . k_j) exp(gc_i - gc_j) for j <= i < valid
 *                                            length, else 0, as six fragments f = (query
 *                                            tile t, key step s) = (0,0), (1,0), (2,0), (2,1),
 *                                            (3,0), (3,1): lane 16 a + r, slot 4 h + b holds
 *                                            P[16 t + r][32 s + 16 h + 4 a + b]
 *   Qc  bf16  [n_chunks][H_q][4][d_k/32][64][8] (bf16 only; written when the state scan
 *                                            takes one 16-column tile a workgroup, and by
 *                                            gdn_chunk_fwd_fused) the chunk's query rows
 *                                            (L2-normalised with the front end), zero
 *                                            past the valid length, as fragments (w, s): lane
 *                                            16 a + r, slot 4 h + b holds
 *                                            q[16 w + r][32 s + 16 h + 4 a + b]
 *   Af  utype [n_chunks][H_v][6][64][8]      A's fragments (above), A form only; rows past
 *                                            the valid length are unit rows
 * For bf16 the chunk-start states and U - W S never leave the chip (the output
 * is formed inside the state scan): Ht and Xt are written only under
 * GDN_FWD_KEEP_HX (gdn_chunk_fwd_ex).
 */
typedef struct gdn_workspace_layout {
    int64_t n_chunks;
    size_t off_gates, off_A, off_Af, off_W, off_U, off_Kc, off_Ht, off_Xt, off_P, off_Qc; /* byte offsets
                                                        (the regions lie in the order of the table above) */
    size_t total_bytes;
} gdn_workspace_layout;

/*
 * Host-only.  Validates the batch description and fills `layout`.
 * cu_seqlens_host: HOST int32 [num_seqs + 1], 0 = c[0] <= c[1] <= ... <= c[num_seqs] = T.
 * Returns GDN_OK or GDN_EINVAL / GDN_EUNSUPPORTED.
 */
int gdn_chunk_fwd_workspace_layout(int32_t T, int32_t num_seqs, const int32_t *cu_seqlens_host, int32_t H_q,
                                   int32_t H_v, int32_t d_k, int32_t d_v, gdn_dtype dtype,
                                   gdn_workspace_layout *layout);

/* Host-only.  Bytes of workspace gdn_chunk_fwd needs for the batch described by
 * cu_seqlens_host (T = cu_seqlens_host[num_seqs]; may be NULL when num_seqs == 0),
 * or 0 if the arguments are invalid (an empty batch needs 0 bytes too;
 * gdn_chunk_fwd_workspace_layout tells the two cases apart). */
size_t gdn_chunk_fwd_workspace_size(const int32_t *cu_seqlens_host, int32_t num_seqs, int32_t H_q, int32_t H_v,
                                    int32_t d_k, int32_t d_v, gdn_dtype dtype);

/*
 * Host-only (it asks the HIP runtime for the current device's compute-unit
 * count).  Which form of the chunk operands the state scan of gdn_chunk_fwd
 * (and gdn_chunk_fwd_dev) reads for a call of T tokens in num_seqs sequences:
 * 0 = W and U (X = U - W S), 1 = A and the raw K, V rows (X = A B (V - Gamma
 * K S)).  Both give the chunk form's results; they differ in rounding and in
 * which workspace regions are written.  Always 0 for GDN_F32.  Returns
 * GDN_EINVAL / GDN_EUNSUPPORTED for invalid arguments.
 */
int gdn_chunk_fwd_form(int32_t T, int32_t num_seqs, int32_t H_v, int32_t d, gdn_dtype dtype);

/*
 * Chunk-wise prefill ("实验三：GDN Prefill 前向优化", sections "计算过程描述" and
 * "输入输出定义").  For every sequence n (tokens c[n] .. c[n+1]-1) and value
 * head h, starting from initial_state[n, h] (zeros if initial_state == NULL),
 * computes per chunk of <= 64 tokens
 *     A = (I + StrictLower(B Gamma K K^T Gamma^-1))^-1,  U = A B V,  W = A B Gamma K,
 *     S_next = gamma_l S + gamma_l K^T Gamma^-1 (U - W S),
 *     O      = scale [Gamma Q S + Gamma Lower(Q K^T) Gamma^-1 (U - W S)],
 * Gamma = Diag(exp(in-chunk inclusive cumsum of g)), B = Diag(beta), gamma_l the
 * last valid token's entry; this equals the token recurrence above.
 *
 *   q, k      dtype [T, H_q, d_k]      v dtype [T, H_v, d_v]
 *   g, beta   fp32  [T, H_v]           g = ln(alpha) per token
 *   cu_seqlens_host  HOST int32 [num_seqs + 1] (see above); sequences may be empty
 *   initial_state  fp32 [num_seqs, H_v, d_k, d_v] or NULL
 *   out       dtype [T, H_v, d_v]      (written for every token)
 *   final_state fp32 [num_seqs, H_v, d_k, d_v] or NULL; may equal initial_state
 *             (read fully before written).  Other overlaps are undefined.
 *   workspace  device buffer of >= gdn_chunk_fwd_workspace_size() bytes; its
 *             contents on return are documented in gdn_workspace_layout.
 * num_seqs == 0 or T == 0 is a no-op returning GDN_OK.
 */
int gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
                  const int32_t *cu_seqlens_host, int32_t num_seqs, const float *initial_state, void *out,
                  float *final_state, int32_t T, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, float scale,
                  gdn_dtype dtype, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Optional read-out epilogue of gdn_chunk_fwd_ex and gdn_recurrent_step_fused:
 * the head-wise gated RMSNorm that follows the GDN read-out ("Qwen3.5-397B-A17B"
 * trace page, Decode-GDN node 8, output_rmsnorm_silu_gate; node 18 of the
 * prefill graph):
 *     out[t, h, :] = o / sqrt(mean_j o_j^2 + eps) * weight * silu(z[t, h, :]),
 *     silu(x) = x * sigmoid(x),
 * over the d_v channels of one value head, norm before gate, computed on the
 * fp32 read-out o and rounded once to the output dtype.
 *   z       dtype [T or N, H_v, d_v], 16-byte aligned
 *   weight  fp32 [d_v] (multiplies directly), 16-byte aligned
 *   eps     the model's norm epsilon (> 0)
 */
typedef struct gdn_output_gate {
    const void *z;
    const float *weight;
    float eps;
} gdn_output_gate;

/* Flags of gdn_chunk_fwd_ex. */
#define GDN_FWD_KEEP_A 1u  /* also write A to its workspace region (otherwise that region is left untouched) */
#define GDN_FWD_KEEP_HX 2u /* also write Ht and Xt (bf16 forms the output on chip and leaves them untouched) */
#define GDN_FWD_SCAN_CT1 4u  /* bf16: the state scan takes 1 / 2 / 4 sixteen-column tiles of d_v a */
#define GDN_FWD_SCAN_CT2 8u  /* workgroup, with as many bins of sequences as fit on the chip at that */
#define GDN_FWD_SCAN_CT4 16u /* width, instead of the width the host's cost model picks (at most one) */
#define GDN_FWD_KEEP_WU 32u  /* also write W and U where the state scan does not read them (A form) */
#define GDN_FWD_FORM_W 64u   /* bf16: the state scan reads W and U, whatever the batch */
#define GDN_FWD_FORM_A 128u  /* bf16: the state scan reads A and the raw rows, whatever the batch */

/*
 * gdn_chunk_fwd with options, for inspection, profiling and benchmarks.  Same
 * arguments and results as gdn_chunk_fwd, plus:
 *   flags  0 or a combination of the GDN_FWD_ bits above.  A is an
 *          intermediate nothing downstream reads back in row-major form (W and
 *          U, or A's fragments, are formed from it on chip), so gdn_chunk_fwd
 *          does not spend the HBM write on it; GDN_FWD_KEEP_A writes it for
 *          inspection, GDN_FWD_KEEP_WU likewise W and U in the A form.  A
 *          GDN_FWD_SCAN_CT bit fixes the state scan's work split, a
 *          GDN_FWD_FORM bit the operands it reads (gdn_chunk_fwd_form; for
 *          tests of every split and form: within a form the results are
 *          bitwise the same for any split, and the two forms agree to rounding);
 *          both are ignored for fp32, which always scans one tile a workgroup
 *          from W and U.  Unknown bits, more than one GDN_FWD_SCAN_CT bit or
 *          both GDN_FWD_FORM bits: GDN_EINVAL.
 *   gate   NULL, or the read-out epilogue above applied to `out`.
 *   stage_events  NULL or an array of six hipEvent_t created by the caller:
 *          the start and stop events of the three kernels (chunk_prep: gate
 *          cumsum, A, then W and U or A's fragments; chunk_state_h: the serial
 *          state scan, with the output for bf16; chunk_output_o for fp32, the
 *          gated read-out for bf16) of the first launch (a launch covers up to 64
 *          sequences; larger batches take several).  They are stamped by the
 *          kernels' own dispatches, so event 2k+1 minus event 2k is the
 *          execution time of kernel k without launch gaps.
 */
int gdn_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *g, const float *beta,
                     const int32_t *cu_seqlens_host, int32_t num_seqs, const float *initial_state, void *out,
                     float *final_state, int32_t T, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, float scale,
                     gdn_dtype dtype, void *workspace, size_t workspace_bytes, hipStream_t stream, uint32_t flags,
                     const gdn_output_gate *gate, void *const *stage_events);

/*
 * gdn_chunk_fwd with cu_seqlens in DEVICE memory, for callers that capture the
 * prefill in a graph and replay it with new sequence boundaries (the trace
 * page's serving path keeps its sequence offsets on the device).  A small
 * kernel builds the per-launch sequence tables in the workspace from
 * cu_seqlens_dev; the grids are sized from T and num_seqs alone, so nothing in
 * the call depends on the boundaries' values.
 *   cu_seqlens_dev  DEVICE int32 [num_seqs + 1], 4-byte aligned, read by the
 *           kernels on the stream.  It should satisfy gdn_chunk_fwd's rules
 *           (0 = c[0] <= ... <= c[num_seqs] = T); it cannot be checked on the
 *           host.  Values that break them are clamped into [0, T] and made
 *           non-decreasing before use (no access leaves the buffers), with
 *           unspecified results; tokens past the last boundary are not written.
 *   workspace  >= gdn_chunk_fwd_dev_workspace_size(T, num_seqs, ...) bytes (the
 *           intermediates for the chunk-count bound T/64 + num_seqs, then the
 *           tables).
 *   gate    NULL, or the read-out epilogue (gdn_output_gate).
 * Other arguments and errors as gdn_chunk_fwd.
 */
size_t gdn_chunk_fwd_dev_workspace_size(int32_t T, int32_t num_seqs, int32_t H_q, int32_t H_v, int32_t d_k,
                                        int32_t d_v, gdn_dtype dtype);
int gdn_chunk_fwd_dev(const void *q, const void *k, const void *v, const float *g, const float *beta,
                      const int32_t *cu_seqlens_dev, int32_t num_seqs, const float *initial_state, void *out,
                      float *final_state, int32_t T, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, float scale,
                      gdn_dtype dtype, void *workspace, size_t workspace_bytes, const gdn_output_gate *gate,
                      hipStream_t stream);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and results, with the workspace taken from a static device
 * array of GDN_SCRATCH_BYTES that the library holds on each GPU it runs on
 * (placed when its code object is loaded; kept until the process ends).  The
 * first call on a device looks up that device's copy (no allocation); the call
 * allocates nothing.  Arguments, results and errors as gdn_chunk_fwd, except:
 *   - a batch whose workspace (gdn_chunk_fwd_workspace_size) exceeds
 *     GDN_SCRATCH_BYTES returns GDN_EWORKSPACE before any HIP call (256 MiB:
 *     one 4096-token sequence at H_v = 32, d = 128, bf16 needs 193 MiB);
 *   - the workspace contents after the call are those of gdn_chunk_fwd, in the
 *     library's array, and are overwritten by the next call.
 * All calls on one GPU share its array: calls that overlap in time on one GPU
 * (on different streams, or from several host threads without ordering) race
 * and give undefined results.  Calls in stream order on one stream are safe:
 * every region a call reads is written earlier in the same call, so nothing
 * left by a previous call needs clearing.
 */
#define GDN_SCRATCH_BYTES (256u << 20)
int gdn_chunk_fwd_scratch(const void *q, const void *k, const void *v, const float *g, const float *beta,
                          const int32_t *cu_seqlens_host, int32_t num_seqs, const float *initial_state, void *out,
                          float *final_state, int32_t T, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v,
                          float scale, gdn_dtype dtype, hipStream_t stream);

/*
 * One recurrent decode step ("Qwen3.5-397B-A17B" trace page, Decode-GDN node 7,
 * gdn_packed_recurrent_qk_norm_gating_state_update — its decay, delta update and
 * read; the Q/K normalisation and gate transform of that node are not part of
 * this call: q, k arrive normalised and g, beta arrive final).  For every
 * sequence n and value head h, with alpha = exp(g[n,h]):
 *     S = alpha S;  delta = beta (v - k S);  S = S + k^T delta;  o = scale * q S
 * computed in fp32 in one pass over S (read once, written once).
 *
 *   q, k   dtype [N, H_q, d_k]    v dtype [N, H_v, d_v]
 *   g, beta fp32 [N, H_v]
 *   state  fp32 [N, H_v, d_k, d_v], updated IN PLACE
 *   out    dtype [N, H_v, d_v]
 * N == 0 is a no-op returning GDN_OK.
 */
int gdn_recurrent_step(const void *q, const void *k, const void *v, const float *g, const float *beta, float *state,
                       void *out, int32_t N, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, float scale,
                       gdn_dtype dtype, hipStream_t stream);

/*
 * One recurrent decode step with its front end fused in ("Qwen3.5-397B-A17B"
 * trace page, Decode-GDN node 7, gdn_packed_recurrent_qk_norm_gating_state_update,
 * all four steps).  Takes the raw per-token inputs of that node; for every
 * sequence n and value head h (query/key head h / (H_v / H_q)):
 *     k_bar = k / sqrt(sum_j k_j^2 + 1e-6),   q_bar = scale * q / sqrt(sum_j q_j^2 + 1e-6)
 *     g = -exp(A_log[h]) * softplus(a[n,h] + dt_bias[h]),   alpha = exp(g)
 *         (softplus(x) = ln(1 + e^x), evaluated without overflow for any x)
 *     beta = sigmoid(b[n,h]) rounded to `dtype` (the bf16 rounding the page keeps)
 *     S = alpha S;  delta = beta (v - k_bar S);  S = S + k_bar^T delta;  o = q_bar S
 * in fp32, one pass over S.  The model's query scale is 1 / sqrt(d_k).
 *
 *   q, k     dtype [N, H_q, d_k]   (not normalised)    v dtype [N, H_v, d_v]
 *   a, b     dtype [N, H_v]        A_log, dt_bias fp32 [H_v]
 *   state    fp32 [N, H_v, d_k, d_v], updated IN PLACE
 *   out      dtype [N, H_v, d_v]
 *   gate     NULL, or the read-out epilogue (gdn_output_gate) applied to out:
 *            the whole of nodes 7 and 8 in one pass.
 * q, k, v, state, out 16-byte aligned; a, b, A_log, dt_bias aligned to their
 * element size.  Errors as gdn_recurrent_step.  N == 0 is a no-op returning GDN_OK.
 */
int gdn_recurrent_step_fused(const void *q, const void *k, const void *v, const void *a, const void *b,
                             const float *A_log, const float *dt_bias, float *state, void *out, int32_t N,
                             int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, float scale, gdn_dtype dtype,
                             const gdn_output_gate *gate, hipStream_t stream);

/*
 * Short causal depthwise convolution + SiLU with its input history over a
 * packed batch ("Qwen3.5-397B-A17B" trace page, Decode-GDN node 6,
 * qkvzba_unpack_causal_conv1d_silu; the window order of the "Kestrel_VLLM - 24"
 * page, section 三).  For every sequence n, token t and channel c:
 *     out[t, c] = SiLU(sum_{k=0}^{K-1} weight[c, k] * x_{t-(K-1)+k, c} + bias[c])
 * taps oldest first (weight[c, K-1] multiplies the current input); inputs
 * before a sequence's first token come from its history initial_state[n]
 * (rows oldest first) or are zero.  final_state[n] receives the sequence's
 * last K-1 raw inputs (reaching into its history when it is shorter).
 *
 *   x, out      dtype [T, C]   (out rounded to dtype; must not overlap x)
 *   weight      fp32 [C, K]    bias fp32 [C] or NULL
 *   initial_state, final_state  dtype [num_seqs, K-1, C] or NULL; may be equal
 *   cu_seqlens_host  as for gdn_chunk_fwd
 * K in {2, 3, 4}; C a multiple of 8 (bf16) or 4 (fp32); every pointer
 * 16-byte aligned.
 * num_seqs == 0 is a no-op returning GDN_OK.
 */
int gdn_conv1d_silu_fwd(const void *x, const int32_t *cu_seqlens_host, int32_t num_seqs, int32_t T, int32_t C,
                        int32_t K, const float *weight, const float *bias, const void *initial_state, void *out,
                        void *final_state, gdn_dtype dtype, hipStream_t stream);

/*
 * One decode token of the same convolution for N sequences: x, out dtype
 * [N, C]; state dtype [N, K-1, C], the history, updated IN PLACE (shifted by
 * one, x appended).  Same constraints as gdn_conv1d_silu_fwd; N == 0 is a no-op.
 */
int gdn_conv1d_silu_step(const void *x, int32_t N, int32_t C, int32_t K, const float *weight, const float *bias,
                         void *state, void *out, gdn_dtype dtype, hipStream_t stream);

/*
 * State pools for serving.  In the "Qwen3.5-397B-A17B" trace page the layer
 * reads and writes its conv and recurrent states through per-request cache
 * slots (section 1, Prefill-GDN graph: node 5 derives initial_state_mask from
 * extend_prefix_lens and feeds node 6; section 3.6.5 keeps padding slots,
 * invalid state indices and graph replays as part of the cache semantics).
 * A pool holds one row per slot: the recurrent state pool is fp32
 * [pool_size, H_v, d_k, d_v], the conv history pool dtype [pool_size, K-1, C].
 *
 * Prefill addressing (host arrays, read during the call only):
 *   slot[i]         pool row of sequence i.  In [0, pool_size): the sequence
 *                   starts from that row when has_initial[i] != 0 (it extends
 *                   a cached prefix, extend_prefix_len > 0), from zeros
 *                   otherwise, and its final state is written back to the
 *                   row.  < 0: starts from zeros, final state not kept.
 *                   >= pool_size, or a row >= 0 named twice: GDN_EINVAL.
 *   has_initial     uint8 [num_seqs], or NULL meaning all nonzero.
 *   pool_size       rows in the pool (>= 0).
 * Rows that no sequence names are left untouched.
 */
typedef struct gdn_state_slots {
    const int32_t *slot;
    const uint8_t *has_initial;
    int32_t pool_size;
} gdn_state_slots;

/*
 * gdn_chunk_fwd over a state pool: state_pool (fp32 [pool_size, H_v, d_k, d_v],
 * 16-byte aligned; may be NULL when no slot is >= 0) takes the place of
 * initial_state and final_state, addressed by `slots` as described above.
 * gate as in gdn_chunk_fwd_ex.  Other arguments, results and errors as
 * gdn_chunk_fwd; slots == NULL: GDN_EINVAL.
 */
int gdn_chunk_fwd_pooled(const void *q, const void *k, const void *v, const float *g, const float *beta,
                         const int32_t *cu_seqlens_host, int32_t num_seqs, float *state_pool,
                         const gdn_state_slots *slots, void *out, int32_t T, int32_t H_q, int32_t H_v, int32_t d_k,
                         int32_t d_v, float scale, gdn_dtype dtype, void *workspace, size_t workspace_bytes,
                         const gdn_output_gate *gate, hipStream_t stream);

/*
 * gdn_conv1d_silu_fwd over a history pool: state_pool dtype [pool_size, K-1, C]
 * (16-byte aligned) takes the place of initial_state and final_state,
 * addressed by `slots`.  Otherwise as gdn_conv1d_silu_fwd.
 */
int gdn_conv1d_silu_fwd_pooled(const void *x, const int32_t *cu_seqlens_host, int32_t num_seqs, int32_t T, int32_t C,
                               int32_t K, const float *weight, const float *bias, void *state_pool,
                               const gdn_state_slots *slots, void *out, gdn_dtype dtype, hipStream_t stream);

/*
 * Decode steps over a state pool.  slot: DEVICE int32 [N] (4-byte aligned),
 * the pool row of each sequence, read by the kernel (so a captured graph can
 * replay with new slots).  A slot outside [0, pool_size) marks padding: that
 * sequence's output row is written as zeros and no pool row is read or
 * written.  Two sequences naming one row race (undefined result): rows must
 * be distinct.  Otherwise as gdn_recurrent_step_fused / gdn_conv1d_silu_step,
 * with state_pool (fp32 [pool_size, H_v, d_k, d_v], resp. dtype
 * [pool_size, K-1, C]) updated in place.  slot == NULL with N > 0:
 * GDN_EINVAL.
 */
int gdn_recurrent_step_fused_pooled(const void *q, const void *k, const void *v, const void *a, const void *b,
                                    const float *A_log, const float *dt_bias, float *state_pool, const int32_t *slot,
                                    int32_t pool_size, void *out, int32_t N, int32_t H_q, int32_t H_v, int32_t d_k,
                                    int32_t d_v, float scale, gdn_dtype dtype, const gdn_output_gate *gate,
                                    hipStream_t stream);

int gdn_conv1d_silu_step_pooled(const void *x, int32_t N, int32_t C, int32_t K, const float *weight,
                                const float *bias, void *state_pool, const int32_t *slot, int32_t pool_size,
                                void *out, gdn_dtype dtype, hipStream_t stream);

/*
 * Front end of the prefill ("Qwen3.5-397B-A17B" trace page, section 1,
 * Prefill-GDN graph: node 8 gdn_gating turns a, b into g, beta; nodes 9 and 10
 * L2-normalise q and k), done inside the chunk kernels as rows are staged:
 *     k_bar = k / sqrt(sum_j k_j^2 + 1e-6),  q_bar = q / sqrt(sum_j q_j^2 + 1e-6)
 *             (each rounded to dtype, as the normalisation nodes write them)
 *     g     = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])   (as in
 *             gdn_recurrent_step_fused)
 *     beta  = sigmoid(b[t,h]) rounded to dtype
 * then the chunk form of gdn_chunk_fwd on (q_bar, k_bar, v, g, beta); the output
 * scale is the `scale` argument (the model's 1 / sqrt(d_k)).
 *   a, b      dtype [T, H_v], aligned to their element size
 *   A_log, dt_bias  fp32 [H_v], 4-byte aligned
 */
typedef struct gdn_front_end {
    const void *a;
    const void *b;
    const float *A_log;
    const float *dt_bias;
} gdn_front_end;

/*
 * Chunk-wise prefill from the raw per-token inputs: q, k not normalised, and
 * the gdn_front_end inputs in place of g and beta.  Other arguments as
 * gdn_chunk_fwd, plus
 *   slots   NULL: initial_state / final_state as in gdn_chunk_fwd.  Non-NULL:
 *           initial_state is a state pool addressed by slots (see
 *           gdn_state_slots) and final_state must be NULL or the same pointer.
 *   gate    NULL, or the read-out epilogue (gdn_output_gate) applied to out.
 * front == NULL: GDN_EINVAL.  The workspace is gdn_chunk_fwd's.
 */
int gdn_chunk_fwd_fused(const void *q, const void *k, const void *v, const gdn_front_end *front,
                        const int32_t *cu_seqlens_host, int32_t num_seqs, float *initial_state, void *out,
                        float *final_state, const gdn_state_slots *slots, int32_t T, int32_t H_q, int32_t H_v,
                        int32_t d_k, int32_t d_v, float scale, gdn_dtype dtype, void *workspace,
                        size_t workspace_bytes, const gdn_output_gate *gate, hipStream_t stream);

/*
 * Pool row maintenance (the "Kestrel_VLLM - 24" page, section 五, resets its
 * single state mirror for a new sequence and leaves branch cloning for
 * speculative decoding to later; here both work on any pool).  The pool is
 * [pool_size][row_bytes], 16-byte aligned, row_bytes a multiple of 16 (a
 * recurrent state row is H_v*d_k*d_v*4 bytes, a conv history row
 * (K-1)*C*sizeof(dtype)).  rows, src_rows, dst_rows: DEVICE int32 [n].
 *   gdn_state_rows_zero   row rows[i] := 0
 *   gdn_state_rows_copy   row dst_rows[i] := row src_rows[i]
 * Entries naming a row outside [0, pool_size) are skipped.  Within one call
 * a destination row must not also be a source row or appear twice (race);
 * one source may feed many destinations (cloning one state into several
 * branches).  n == 0 is a no-op.
 */
int gdn_state_rows_zero(void *pool, int32_t pool_size, size_t row_bytes, const int32_t *rows, int32_t n,
                        hipStream_t stream);
int gdn_state_rows_copy(void *pool, int32_t pool_size, size_t row_bytes, const int32_t *src_rows,
                        const int32_t *dst_rows, int32_t n, hipStream_t stream);

/*
 * Measurement aid (not part of the GDN computation): dst[0 .. bytes) :=
 * src[0 .. bytes) with 16-byte vector accesses over the whole chip, a plain
 * read-once / write-once stream.  Its bandwidth, 2 * bytes / time, is the
 * achievable HBM figure the library's kernels are compared with, and a copy of
 * known size calibrates HBM byte counters.  Device buffers, 16-byte aligned,
 * bytes a multiple of 16, not overlapping (GDN_EINVAL), asynchronous on
 * `stream`.  bytes == 0 is a no-op.
 */
int gdn_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

/* Text naming a status code.  For GDN_ELAUNCH it also names the last HIP error
 * this thread saw inside the library (the text is then thread-local and valid
 * until the next call into the library from this thread); otherwise, and for
 * codes it does not know, a static string. */
const char *gdn_strerror(int status);

/* Static string naming a status code (gdn_strerror without the HIP error). */
const char *gdn_status_string(int status);

/* Text of the last HIP error seen by this thread inside the library ("" if none). */
const char *gdn_last_hip_error(void);

/* Library version, e.g. "0.1.0". */
const char *gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
