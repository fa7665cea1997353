// Host side of libgdn.so: argument validation, workspace layout, launch
// grouping.  Every check runs before any HIP call, so a rejected call writes
// nothing and never touches the device (all-or-nothing entry points).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <string>
#include <vector>

#include "gdn.h"
#include "gdn_params.h"

namespace {

thread_local std::string g_last_hip_error;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t elem_size(gdn_dtype dt) { return dt == GDN_BF16 ? 2 : 4; }

int check_shapes(int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, gdn_dtype dtype) {
    if (H_q <= 0 || H_v <= 0 || d_k <= 0 || d_v <= 0) return GDN_EINVAL;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_EUNSUPPORTED;
    if (d_k != d_v || (d_k != 64 && d_k != 128)) return GDN_EUNSUPPORTED;
    if (H_v % H_q != 0) return GDN_EUNSUPPORTED;
    return GDN_OK;
}

// Read-out epilogue arguments: z and weight present and 16-byte aligned, eps > 0.
int check_gate(const gdn_output_gate* gate, bool need_z) {
    if (!(gate->eps > 0.f) || !(gate->eps < INFINITY)) return GDN_EINVAL;
    if (need_z && (!gate->z || !gate->weight)) return GDN_EINVAL;
    if ((gate->z && !aligned16(gate->z)) || (gate->weight && !aligned16(gate->weight))) return GDN_EUNSUPPORTED;
    return GDN_OK;
}

// Validates cu_seqlens and counts chunks (each sequence chunked from its own start).
int check_seqlens(int32_t T, int32_t num_seqs, const int32_t* cu, int64_t* n_chunks) {
    if (T < 0 || num_seqs < 0) return GDN_EINVAL;
    if (num_seqs == 0) {
        if (T != 0) return GDN_EINVAL;
        *n_chunks = 0;
        return GDN_OK;
    }
    if (!cu) return GDN_EINVAL;
    if (cu[0] != 0 || cu[num_seqs] != T) return GDN_EINVAL;
    int64_t nc = 0;
    for (int32_t i = 0; i < num_seqs; ++i) {
        const int64_t len = (int64_t)cu[i + 1] - cu[i];
        if (len < 0) return GDN_EINVAL;
        nc += (len + GDN_CHUNK - 1) / GDN_CHUNK;
    }
    if (nc > (int64_t)INT32_MAX / 1024) return GDN_EUNSUPPORTED;
    *n_chunks = nc;
    return GDN_OK;
}

// Pool addressing of a prefill: row indices inside the pool, no duplicate
// kept rows (two sequences writing one row would race).
int check_slots(const gdn_state_slots* sl, int32_t num_seqs, const void* pool) {
    if (!sl || sl->pool_size < 0) return GDN_EINVAL;
    if (num_seqs == 0) return GDN_OK;
    if (!sl->slot) return GDN_EINVAL;
    std::vector<int32_t> kept;
    kept.reserve(num_seqs);
    for (int32_t i = 0; i < num_seqs; ++i) {
        const int32_t r = sl->slot[i];
        if (r >= sl->pool_size) return GDN_EINVAL;
        if (r >= 0) kept.push_back(r);
    }
    if (!kept.empty() && !pool) return GDN_EINVAL;
    std::sort(kept.begin(), kept.end());
    if (std::adjacent_find(kept.begin(), kept.end()) != kept.end()) return GDN_EINVAL;
    return GDN_OK;
}

// Fills the launch table of sequences s0 .. s0+ns-1 (chunk offsets from
// chunk_base) with their state rows: pool rows from `slots`, else row i of the
// initial/final arrays when present, -1 for none.  Returns the next chunk base.
int32_t fill_table(gdn::SeqTable& tab, const int32_t* cu, int32_t s0, int32_t ns, int32_t chunk_base,
                   const gdn_state_slots* slots, bool have_in, bool have_out) {
    tab.num_seqs = ns;
    tab.seq_base = s0;
    tab.chunk_begin = chunk_base;
    int32_t c = chunk_base;
    for (int32_t i = 0; i <= ns; ++i) {
        tab.cu[i] = cu[s0 + i];
        tab.choff[i] = c;
        if (i == ns) break;
        c += (cu[s0 + i + 1] - cu[s0 + i] + GDN_CHUNK - 1) / GDN_CHUNK;
        const int32_t gi = s0 + i;
        if (slots) {
            const int32_t r = slots->slot[gi];
            const bool resume = !slots->has_initial || slots->has_initial[gi];
            tab.s_in[i] = (r >= 0 && resume) ? r : -1;
            tab.s_out[i] = r >= 0 ? r : -1;
        } else {
            tab.s_in[i] = have_in ? gi : -1;
            tab.s_out[i] = have_out ? gi : -1;
        }
    }
    tab.n_chunks = c - chunk_base;
    // Longest sequences first (stable): the serial state scan then starts its
    // longest chains earliest.
    for (int32_t i = 0; i < ns; ++i) tab.order[i] = i;
    std::stable_sort(tab.order, tab.order + ns, [&](int32_t a, int32_t b) {
        return tab.choff[a + 1] - tab.choff[a] > tab.choff[b + 1] - tab.choff[b];
    });
    // one sequence a state-scan bin until pack_scan_bins says otherwise
    for (int32_t i = 0; i <= ns; ++i) tab.bin_first[i] = i;
    tab.n_bins = ns;
    tab.ct = 0;
    return c;
}

// Cost model of the state scan on MI355X (bf16, d = 128, all CUs busy), in
// units of one serial step with one column tile a workgroup (1.15 us): a step
// with 1, 2 or 4 tiles a workgroup (the MFMA and LDS work grows with the
// tiles, the W and K loads do not), and the extra cost of moving from one
// sequence of a bin to the next (final-state stores, initial-state loads).
// Measured: 4 x 16384 tokens, 1.15 / 1.47 / 2.39 us a step; 64 x 128 tokens,
// 1.5 / 2.1 / 3.1 us a sequence boundary.
constexpr double kScanStep[3] = {1.0, 1.28, 2.08};
constexpr double kScanSeq[3] = {1.3, 1.8, 2.7};

// Longest-processing-time packing of the launch's sequences (tab.order, longest
// first) into m bins, a sequence of c chunks weighing step c + seq; rewrites
// order bin by bin, heaviest bin first, and bin_first.  Returns the heaviest
// bin's weight.
double lpt_bins(gdn::SeqTable& tab, int32_t m, double step, double seq, bool write) {
    const int32_t ns = tab.num_seqs;
    std::vector<double> load(m, 0.0);
    std::vector<int32_t> bin_of(ns, 0);
    for (int32_t i = 0; i < ns; ++i) {
        const int32_t n = tab.order[i];
        const int32_t b = (int32_t)(std::min_element(load.begin(), load.end()) - load.begin());
        bin_of[i] = b;
        load[b] += step * (tab.choff[n + 1] - tab.choff[n]) + seq;
    }
    const double heaviest = *std::max_element(load.begin(), load.end());
    if (!write) return heaviest;
    std::vector<int32_t> bins(m);
    for (int32_t b = 0; b < m; ++b) bins[b] = b;
    std::stable_sort(bins.begin(), bins.end(), [&](int32_t a, int32_t b) { return load[a] > load[b]; });
    std::vector<int32_t> order(tab.order, tab.order + ns);
    int32_t k = 0;
    for (int32_t j = 0; j < m; ++j) {
        tab.bin_first[j] = k;
        for (int32_t i = 0; i < ns; ++i)
            if (bin_of[i] == bins[j]) tab.order[k++] = order[i];
    }
    tab.bin_first[m] = k;
    tab.n_bins = m;
    return heaviest;
}

// State-scan work split for a host table: the column tiles per workgroup (ct)
// and the bins of sequences a workgroup scans one after another.  A workgroup
// holds a CU (its LDS), so a launch of more workgroups than CUs runs in waves,
// each paying a workgroup's start-up and drain; instead the sequences are
// packed into as many bins as there are CUs for them (cus / workgroups a bin),
// at most one sequence a bin, and ct is the one whose heaviest bin is the
// cheapest under the cost model.
void pack_scan_bins(gdn::SeqTable& tab, int32_t H_v, int32_t d, bool bf16, int32_t cus, int32_t force_ct = 0) {
    const int32_t ns = tab.num_seqs;
    if (ns <= 0) return;
    const int32_t nt = d / 16;
    int32_t best_ci = 0, best_m = 1;
    double best = 0.0;
    for (int32_t ci = 0; ci < (bf16 ? 3 : 1); ++ci) {  // ct = 1 << ci
        if (bf16 && force_ct && (1 << ci) != force_ct) continue;
        const int64_t per_bin = (int64_t)H_v * (nt >> ci);  // workgroups a bin
        const int32_t m = (int32_t)std::max<int64_t>(1, std::min<int64_t>(ns, cus / per_bin));
        const int64_t waves = (m * per_bin + cus - 1) / cus;
        const double cost = lpt_bins(tab, m, kScanStep[ci], kScanSeq[ci], false) * (double)waves;
        if ((bf16 && force_ct) || ci == 0 || cost < best) {
            best = cost;
            best_ci = ci;
            best_m = m;
        }
    }
    lpt_bins(tab, best_m, kScanStep[best_ci], kScanSeq[best_ci], true);
    tab.ct = 1 << best_ci;
}

// The same choice for device tables, whose lengths the host does not see: the
// cost model on a launch group of equal sequences of the batch's mean length.
// Returns ct; *bins_cap is the number of bins a group of that ct may use.
// Form of the chunk operands the state scan reads (bf16; fp32 always reads W
// and U).  The scan's time is its serial chain, and the A form (X = A B (V -
// Gamma K S)) adds an exchange to every step of it, while it takes the W and U
// products and 40 % of the bytes out of chunk_prep.  W and U pay only where
// chunk_prep is cheap: the batch's tile chains (sequence, value head, 16 columns
// of d_v) fit on the chip about twice over, and the scan's W-form operand
// stream fits in the 256 MB Infinity Cache next to the layer's other tensors
// (at most 128 MiB).  Measured on MI355X (one call, binding included): one
// sequence of 4096 tokens x 32 heads 105 (W) against 108 us (A); of 8192
// tokens 227 against 205 us; of 65536 tokens 1.48 against 1.43 ms; 8
// sequences of about 3800 tokens 554 against 488 us; 256 requests of up to
// 256 tokens 952 against 844 us.  Decided from the call's token and sequence
// counts alone, so host and device boundaries take the same form.
int32_t a_form(int32_t T, int32_t num_seqs, int32_t H_v, int32_t d, gdn_dtype dtype, int32_t cus) {
    if (dtype != GDN_BF16) return 0;
    if ((int64_t)num_seqs * H_v * (d / 16) > 2 * (int64_t)cus) return 1;
    const int64_t chunks = ((int64_t)T + GDN_CHUNK - 1) / GDN_CHUNK + num_seqs;  // bound on the chunk count
    const int64_t stage = 2 * (int64_t)GDN_CHUNK * d * 2 + GDN_CHUNK * 16 * 2 + 1024 + 6 * 1024;  // W, K, U, gates, P
    return chunks * H_v * stage > (int64_t(128) << 20) ? 1 : 0;
}

int32_t dev_scan_shape(int32_t num_seqs, int32_t T, int32_t H_v, int32_t d, bool bf16, int32_t cus,
                       int32_t* bins_cap) {
    gdn::SeqTable t;
    const int32_t ns = std::min<int32_t>(gdn::MAX_SEQS_PER_LAUNCH, num_seqs);
    const int64_t len = num_seqs > 0 ? (int64_t)T / num_seqs : 0;
    const int32_t c = (int32_t)std::min<int64_t>((len + GDN_CHUNK - 1) / GDN_CHUNK, 1 << 24);
    t.num_seqs = ns;
    for (int32_t i = 0; i <= ns; ++i) t.choff[i] = i * c;
    for (int32_t i = 0; i < ns; ++i) t.order[i] = i;
    pack_scan_bins(t, H_v, d, bf16, cus);
    const int64_t per_bin = (int64_t)H_v * ((d / 16) / t.ct);
    *bins_cap = (int32_t)std::max<int64_t>(1, cus / per_bin);
    return t.ct;
}

hipError_t run_chunk(const gdn::ChunkParams& p, gdn_dtype dt, int d, hipStream_t s, hipEvent_t const* ev) {
    if (dt == GDN_BF16)
        return d == 128 ? gdn::launch_chunk_pipeline<gdn::bf16, 128>(p, s, ev)
                        : gdn::launch_chunk_pipeline<gdn::bf16, 64>(p, s, ev);
    return d == 128 ? gdn::launch_chunk_pipeline<float, 128>(p, s, ev) : gdn::launch_chunk_pipeline<float, 64>(p, s, ev);
}

template <typename T>
hipError_t run_conv(const gdn::ConvParams& p, int K, int N_step, hipStream_t s) {
    // N_step < 0: prefill; else a decode step over N_step sequences
    switch (K) {
        case 2: return N_step < 0 ? gdn::launch_conv_prefill<T, 2>(p, s) : gdn::launch_conv_step<T, 2>(p, N_step, s);
        case 3: return N_step < 0 ? gdn::launch_conv_prefill<T, 3>(p, s) : gdn::launch_conv_step<T, 3>(p, N_step, s);
        default: return N_step < 0 ? gdn::launch_conv_prefill<T, 4>(p, s) : gdn::launch_conv_step<T, 4>(p, N_step, s);
    }
}

int check_conv(int32_t C, int32_t K, gdn_dtype dtype, const float* weight, const float* bias) {
    if (C <= 0 || K <= 0 || !weight) return GDN_EINVAL;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_EUNSUPPORTED;
    if (K < 2 || K > 4) return GDN_EUNSUPPORTED;
    if (C % (int32_t)(16 / elem_size(dtype)) != 0) return GDN_EUNSUPPORTED;
    if (!aligned16(weight) || (bias && !aligned16(bias))) return GDN_EUNSUPPORTED;
    return GDN_OK;
}

template <bool FUSED>
hipError_t run_decode(const gdn::DecodeParams& p, gdn_dtype dt, int d, hipStream_t s) {
    if (dt == GDN_BF16)
        return d == 128 ? gdn::launch_recurrent_step<gdn::bf16, 128, FUSED>(p, s)
                        : gdn::launch_recurrent_step<gdn::bf16, 64, FUSED>(p, s);
    return d == 128 ? gdn::launch_recurrent_step<float, 128, FUSED>(p, s)
                    : gdn::launch_recurrent_step<float, 64, FUSED>(p, s);
}

int layout_for_chunks(int64_t nc, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, gdn_dtype dtype,
                      gdn_workspace_layout* layout);

using gdn::hip_fail;


int conv_fwd_impl(const void* x, const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t T, int32_t C, int32_t K,
                  const float* weight, const float* bias, const void* s_in, void* out, void* s_out,
                  const gdn_state_slots* slots, gdn_dtype dtype, hipStream_t stream) {
    int rc = check_conv(C, K, dtype, weight, bias);
    if (rc != GDN_OK) return rc;
    int64_t n_chunks = 0;
    rc = check_seqlens(T, num_seqs, cu_seqlens_host, &n_chunks);
    if (rc != GDN_OK) return rc;
    if (slots && (rc = check_slots(slots, num_seqs, s_in)) != GDN_OK) return rc;
    if (num_seqs == 0) return GDN_OK;
    if ((int64_t)T * C > INT32_MAX * (int64_t)16) return GDN_EUNSUPPORTED;
    if (T > 0 && (!x || !out)) return GDN_EINVAL;
    const void* ptrs[] = {x, out, s_in, s_out};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDN_EUNSUPPORTED;
    gdn::ConvParams p{};
    p.x = x; p.y = out; p.w = weight; p.b = bias; p.s_in = s_in; p.s_out = s_out; p.C = C;
    int32_t chunk_base = 0;
    for (int32_t s0 = 0; s0 < num_seqs; s0 += gdn::MAX_SEQS_PER_LAUNCH) {
        const int32_t ns = std::min<int32_t>(gdn::MAX_SEQS_PER_LAUNCH, num_seqs - s0);
        chunk_base = fill_table(p.tab, cu_seqlens_host, s0, ns, chunk_base, slots, s_in != nullptr, s_out != nullptr);
        const hipError_t e =
            dtype == GDN_BF16 ? run_conv<gdn::bf16>(p, K, -1, stream) : run_conv<float>(p, K, -1, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    return GDN_OK;
}

int conv_step_impl(const void* x, int32_t N, int32_t C, int32_t K, const float* weight, const float* bias,
                   void* pool, const int32_t* slot, int32_t pool_size, void* out, gdn_dtype dtype,
                   hipStream_t stream) {
    int rc = check_conv(C, K, dtype, weight, bias);
    if (rc != GDN_OK) return rc;
    if (N < 0 || pool_size < 0) return GDN_EINVAL;
    if (N == 0) return GDN_OK;
    if (!x || !out || (pool_size > 0 && !pool)) return GDN_EINVAL;
    const void* ptrs[] = {x, pool, out};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDN_EUNSUPPORTED;
    if (slot && (reinterpret_cast<uintptr_t>(slot) & 3u)) return GDN_EUNSUPPORTED;
    gdn::ConvParams p{};
    p.x = x; p.y = out; p.w = weight; p.b = bias; p.s_in = pool; p.s_out = pool; p.C = C;
    p.slot = slot; p.pool = pool_size;
    const hipError_t e = dtype == GDN_BF16 ? run_conv<gdn::bf16>(p, K, N, stream) : run_conv<float>(p, K, N, stream);
    if (e != hipSuccess) return hip_fail(e);
    return GDN_OK;
}

int chunk_fwd_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                   const int32_t* cu_seqlens_host, int32_t num_seqs, const float* initial_state, void* out,
                   float* final_state, const gdn_state_slots* slots, int32_t T, int32_t H_q, int32_t H_v, int32_t d_k,
                   int32_t d_v, float scale, gdn_dtype dtype, void* workspace, size_t workspace_bytes,
                   hipStream_t stream,
                   uint32_t flags, const gdn_output_gate* gate, void* const* stage_events,
                   const gdn_front_end* front = nullptr) {
    constexpr uint32_t kScanCt = GDN_FWD_SCAN_CT1 | GDN_FWD_SCAN_CT2 | GDN_FWD_SCAN_CT4;
    constexpr uint32_t kForm = GDN_FWD_FORM_W | GDN_FWD_FORM_A;
    if (flags & ~(uint32_t)(GDN_FWD_KEEP_A | GDN_FWD_KEEP_HX | GDN_FWD_KEEP_WU | kScanCt | kForm)) return GDN_EINVAL;
    const uint32_t ctf = flags & kScanCt;
    if (ctf & (ctf - 1)) return GDN_EINVAL;  // more than one tile width
    if ((flags & kForm) == kForm) return GDN_EINVAL;  // both forms
    const int32_t force_ct = ctf == GDN_FWD_SCAN_CT1 ? 1 : ctf == GDN_FWD_SCAN_CT2 ? 2 : ctf == GDN_FWD_SCAN_CT4 ? 4 : 0;
    if (gate) {
        const int grc = check_gate(gate, T > 0);
        if (grc != GDN_OK) return grc;
    }
    gdn_workspace_layout L;
    int rc = gdn_chunk_fwd_workspace_layout(T, num_seqs, cu_seqlens_host, H_q, H_v, d_k, d_v, dtype, &L);
    if (rc != GDN_OK) return rc;
    if (slots && (rc = check_slots(slots, num_seqs, initial_state)) != GDN_OK) return rc;
    if (num_seqs == 0) return GDN_OK;
    // Pointers: tensors with T > 0 rows must be present; all must be 16-byte aligned.
    if (T > 0 && (!q || !k || !v || !out)) return GDN_EINVAL;
    if (front) {
        if (g || beta) return GDN_EINVAL;
        if (T > 0 && (!front->a || !front->b || !front->A_log || !front->dt_bias)) return GDN_EINVAL;
        const size_t es = elem_size(dtype);
        if ((reinterpret_cast<uintptr_t>(front->a) % es) || (reinterpret_cast<uintptr_t>(front->b) % es) ||
            (reinterpret_cast<uintptr_t>(front->A_log) & 3u) || (reinterpret_cast<uintptr_t>(front->dt_bias) & 3u))
            return GDN_EUNSUPPORTED;
    } else if (T > 0 && (!g || !beta)) {
        return GDN_EINVAL;
    }
    const void* ptrs[] = {q, k, v, g, beta, out, initial_state, final_state, workspace};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDN_EUNSUPPORTED;
    if (!(scale == scale)) return GDN_EINVAL;  // NaN
    if (L.n_chunks > 0 && (!workspace || workspace_bytes < L.total_bytes)) return GDN_EWORKSPACE;

    char* ws = static_cast<char*>(workspace);
    gdn::ChunkParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.s0 = initial_state; p.out = out; p.sfinal = final_state;
    p.gates = reinterpret_cast<float*>(ws + L.off_gates);
    p.A = ws + L.off_A; p.Af = ws + L.off_Af; p.W = ws + L.off_W; p.Ut = ws + L.off_U;
    p.Kc = ws + L.off_Kc;
    p.Ht = ws + L.off_Ht; p.Xt = ws + L.off_Xt;
    p.Pf = dtype == GDN_BF16 ? ws + L.off_P : nullptr;
    p.Qc = dtype == GDN_BF16 ? ws + L.off_Qc : nullptr;
    p.H_q = H_q; p.H_v = H_v; p.G = H_v / H_q; p.scale = scale;
    p.keep_A = (flags & GDN_FWD_KEEP_A) ? 1 : 0;
    p.keep_wu = (flags & GDN_FWD_KEEP_WU) ? 1 : 0;
    p.aform = (flags & GDN_FWD_FORM_A) ? 1 : (flags & GDN_FWD_FORM_W) ? 0 : a_form(T, num_seqs, H_v, d_k, dtype, gdn::cu_count());
    p.keep_hx = (flags & GDN_FWD_KEEP_HX) ? 1 : 0;
    p.T = T;
    p.gz = gate ? gate->z : nullptr;
    p.gw = gate ? gate->weight : nullptr;
    p.geps = gate ? gate->eps : 0.f;
    p.fa = front ? front->a : nullptr;
    p.fb = front ? front->b : nullptr;
    p.A_log = front ? front->A_log : nullptr;
    p.dt_bias = front ? front->dt_bias : nullptr;

    // Launch groups of up to MAX_SEQS_PER_LAUNCH sequences, each with its table in the kernel arguments.
    int32_t chunk_base = 0;
    for (int32_t s0 = 0; s0 < num_seqs; s0 += gdn::MAX_SEQS_PER_LAUNCH) {
        const int32_t ns = std::min<int32_t>(gdn::MAX_SEQS_PER_LAUNCH, num_seqs - s0);
        chunk_base = fill_table(p.tab, cu_seqlens_host, s0, ns, chunk_base, slots, initial_state != nullptr,
                                final_state != nullptr);
        pack_scan_bins(p.tab, H_v, d_k, dtype == GDN_BF16, gdn::cu_count(), force_ct);
        hipEvent_t const* ev = (s0 == 0 && stage_events) ? reinterpret_cast<hipEvent_t const*>(stage_events) : nullptr;
        const hipError_t e = run_chunk(p, dtype, d_k, stream, ev);
        if (e != hipSuccess) return hip_fail(e);
    }
    return GDN_OK;
}

int step_fused_impl(const void* q, const void* k, const void* v, const void* a, const void* b, const float* A_log,
                    const float* dt_bias, float* state, const int32_t* slot, int32_t pool_size, void* out, int32_t N,
                    int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, float scale, gdn_dtype dtype,
                    const gdn_output_gate* gate, hipStream_t stream) {
    int rc = check_shapes(H_q, H_v, d_k, d_v, dtype);
    if (rc != GDN_OK) return rc;
    if (N < 0 || pool_size < 0) return GDN_EINVAL;
    if (N == 0) return GDN_OK;
    if ((int64_t)N * H_v > INT32_MAX) return GDN_EUNSUPPORTED;
    if (!q || !k || !v || !a || !b || !A_log || !dt_bias || !out || (pool_size > 0 && !state)) return GDN_EINVAL;
    const void* ptrs[] = {q, k, v, state, out};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDN_EUNSUPPORTED;
    if (slot && (reinterpret_cast<uintptr_t>(slot) & 3u)) return GDN_EUNSUPPORTED;
    // per-head scalars: natural alignment of their element type
    const size_t es = elem_size(dtype);
    if ((reinterpret_cast<uintptr_t>(a) % es) || (reinterpret_cast<uintptr_t>(b) % es) ||
        (reinterpret_cast<uintptr_t>(A_log) & 3u) || (reinterpret_cast<uintptr_t>(dt_bias) & 3u))
        return GDN_EUNSUPPORTED;
    if (!(scale == scale)) return GDN_EINVAL;
    if (gate) {
        const int grc = check_gate(gate, true);
        if (grc != GDN_OK) return grc;
    }
    gdn::DecodeParams p{};
    p.q = q; p.k = k; p.v = v; p.a = a; p.b = b; p.A_log = A_log; p.dt_bias = dt_bias;
    p.gz = gate ? gate->z : nullptr;
    p.gw = gate ? gate->weight : nullptr;
    p.geps = gate ? gate->eps : 0.f;
    p.state = state; p.out = out;
    p.slot = slot; p.pool = pool_size;
    p.N = N; p.H_q = H_q; p.H_v = H_v; p.G = H_v / H_q; p.scale = scale;
    const hipError_t e = run_decode<true>(p, dtype, d_k, stream);
    if (e != hipSuccess) return hip_fail(e);
    return GDN_OK;
}

}  // namespace

int gdn::hip_fail(hipError_t e) {
    g_last_hip_error = hipGetErrorString(e);
    return GDN_ELAUNCH;
}

extern "C" {

const char* gdn_version(void) { return "0.1.0"; }

int gdn_conv1d_silu_fwd(const void* x, const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t T, int32_t C,
                        int32_t K, const float* weight, const float* bias, const void* initial_state, void* out,
                        void* final_state, gdn_dtype dtype, hipStream_t stream) {
    return conv_fwd_impl(x, cu_seqlens_host, num_seqs, T, C, K, weight, bias, initial_state, out, final_state, nullptr,
                         dtype, stream);
}

int gdn_conv1d_silu_fwd_pooled(const void* x, const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t T, int32_t C,
                               int32_t K, const float* weight, const float* bias, void* state_pool,
                               const gdn_state_slots* slots, void* out, gdn_dtype dtype, hipStream_t stream) {
    if (!slots) return GDN_EINVAL;
    return conv_fwd_impl(x, cu_seqlens_host, num_seqs, T, C, K, weight, bias, state_pool, out, state_pool, slots,
                         dtype, stream);
}

int gdn_conv1d_silu_step(const void* x, int32_t N, int32_t C, int32_t K, const float* weight, const float* bias,
                         void* state, void* out, gdn_dtype dtype, hipStream_t stream) {
    if (!state && N > 0) return GDN_EINVAL;
    return conv_step_impl(x, N, C, K, weight, bias, state, nullptr, N, out, dtype, stream);
}

int gdn_conv1d_silu_step_pooled(const void* x, int32_t N, int32_t C, int32_t K, const float* weight,
                                const float* bias, void* state_pool, const int32_t* slot, int32_t pool_size, void* out,
                                gdn_dtype dtype, hipStream_t stream) {
    if (!slot && N > 0) return GDN_EINVAL;
    return conv_step_impl(x, N, C, K, weight, bias, state_pool, slot, pool_size, out, dtype, stream);
}

const char* gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_EINVAL: return "invalid argument";
        case GDN_EUNSUPPORTED: return "unsupported shape, dtype or alignment";
        case GDN_EWORKSPACE: return "workspace missing or too small";
        case GDN_ELAUNCH: return "HIP launch failed";
        default: return "unknown status";
    }
}

const char* gdn_last_hip_error(void) { return g_last_hip_error.c_str(); }

const char* gdn_strerror(int status) {
    if (status != GDN_ELAUNCH || g_last_hip_error.empty()) return gdn_status_string(status);
    thread_local std::string text;
    text = std::string(gdn_status_string(status)) + ": " + g_last_hip_error;
    return text.c_str();
}

int gdn_chunk_fwd_workspace_layout(int32_t T, int32_t num_seqs, const int32_t* cu_seqlens_host, int32_t H_q,
                                   int32_t H_v, int32_t d_k, int32_t d_v, gdn_dtype dtype,
                                   gdn_workspace_layout* layout) {
    if (!layout) return GDN_EINVAL;
    int rc = check_shapes(H_q, H_v, d_k, d_v, dtype);
    if (rc != GDN_OK) return rc;
    int64_t nc = 0;
    rc = check_seqlens(T, num_seqs, cu_seqlens_host, &nc);
    if (rc != GDN_OK) return rc;
    return layout_for_chunks(nc, H_q, H_v, d_k, d_v, dtype, layout);
}

}  // extern "C"

namespace {

// Region offsets for n_chunks chunks (sizes are per chunk and value head).
int layout_for_chunks(int64_t nc, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, gdn_dtype dtype,
                      gdn_workspace_layout* layout) {
    const size_t es = elem_size(dtype);
    const size_t C = GDN_CHUNK;
    const size_t chv = (size_t)nc * (size_t)H_v;
    const size_t chq = (size_t)nc * (size_t)H_q;
    size_t off = 0;
    gdn_workspace_layout L;
    L.n_chunks = nc;
    L.off_gates = off; off = align_up(off + chv * 4 * C * sizeof(float));
    L.off_A = off;  off = align_up(off + chv * C * C * es);
    L.off_W = off;  off = align_up(off + chv * C * (size_t)d_k * es);
    L.off_U = off; off = align_up(off + chv * (size_t)d_v * C * es);
    L.off_Kc = off; off = align_up(off + chq * C * (size_t)d_k * es);
    L.off_Ht = off; off = align_up(off + chv * (size_t)d_v * (size_t)d_k * es);
    L.off_Xt = off; off = align_up(off + chv * (size_t)d_v * C * es);
    // P (bf16 only: the output is formed inside the state scan): six 1 KiB fragments
    L.off_P = off; off = align_up(off + (dtype == GDN_BF16 ? chv * 6 * 64 * 8 * es : 0));
    // Qc (bf16 only): the query rows (normalised by the front end) as the state
    // scan's output waves' operand fragments, one copy per key head
    L.off_Qc = off; off = align_up(off + (dtype == GDN_BF16 ? chq * C * (size_t)d_k * es : 0));
    // A's six MFMA fragments (64 lanes x 8 values, in the two-byte product type
    // for bf16 inputs, fp32 for fp32)
    L.off_Af = off; off = align_up(off + chv * 6 * 64 * 8 * es);
    L.total_bytes = off;
    *layout = L;
    return GDN_OK;
}

// Chunk-count bound for a device cu_seqlens: sum_i ceil(len_i / 64) <= T / 64 + num_seqs.
int64_t chunk_bound(int32_t T, int32_t num_seqs) { return ((int64_t)T + GDN_CHUNK - 1) / GDN_CHUNK + num_seqs; }

// Workspace of the device-table path: the regions for the chunk bound, then one
// sequence table per launch group.
int dev_layout(int32_t T, int32_t num_seqs, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, gdn_dtype dtype,
               gdn_workspace_layout* L, size_t* tab_off, size_t* total) {
    int rc = check_shapes(H_q, H_v, d_k, d_v, dtype);
    if (rc != GDN_OK) return rc;
    if (T < 0 || num_seqs < 0) return GDN_EINVAL;
    const int64_t nb = chunk_bound(T, num_seqs);
    if (nb > (int64_t)INT32_MAX / 1024) return GDN_EUNSUPPORTED;
    rc = layout_for_chunks(nb, H_q, H_v, d_k, d_v, dtype, L);
    if (rc != GDN_OK) return rc;
    const int64_t groups = ((int64_t)num_seqs + gdn::MAX_SEQS_PER_LAUNCH - 1) / gdn::MAX_SEQS_PER_LAUNCH;
    *tab_off = L->total_bytes;
    *total = align_up(L->total_bytes + (size_t)groups * sizeof(gdn::SeqTable));
    return GDN_OK;
}

}  // namespace

extern "C" {

size_t gdn_chunk_fwd_workspace_size(const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t H_q, int32_t H_v,
                                    int32_t d_k, int32_t d_v, gdn_dtype dtype) {
    if (num_seqs < 0 || (num_seqs > 0 && !cu_seqlens_host)) return 0;
    const int32_t T = num_seqs > 0 ? cu_seqlens_host[num_seqs] : 0;
    gdn_workspace_layout L;
    if (gdn_chunk_fwd_workspace_layout(T, num_seqs, cu_seqlens_host, H_q, H_v, d_k, d_v, dtype, &L) != GDN_OK)
        return 0;
    return L.total_bytes;
}

int gdn_chunk_fwd_form(int32_t T, int32_t num_seqs, int32_t H_v, int32_t d, gdn_dtype dtype) {
    if (T < 0 || num_seqs < 0 || H_v <= 0 || (d != 64 && d != 128)) return GDN_EINVAL;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_EUNSUPPORTED;
    return a_form(T, num_seqs, H_v, d, dtype, gdn::cu_count());
}

int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  const int32_t* cu_seqlens_host, int32_t num_seqs, const float* initial_state, void* out,
                  float* final_state, int32_t T, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, float scale,
                  gdn_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return gdn_chunk_fwd_ex(q, k, v, g, beta, cu_seqlens_host, num_seqs, initial_state, out, final_state, T, H_q, H_v,
                            d_k, d_v, scale, dtype, workspace, workspace_bytes, stream, 0u, nullptr, nullptr);
}

int gdn_chunk_fwd_ex(const void* q, const void* k, const void* v, const float* g, const float* beta,
                     const int32_t* cu_seqlens_host, int32_t num_seqs, const float* initial_state, void* out,
                     float* final_state, int32_t T, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, float scale,
                     gdn_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream, uint32_t flags,
                     const gdn_output_gate* gate, void* const* stage_events) {
    return chunk_fwd_impl(q, k, v, g, beta, cu_seqlens_host, num_seqs, initial_state, out, final_state, nullptr, T,
                          H_q, H_v, d_k, d_v, scale, dtype, workspace, workspace_bytes, stream, flags, gate,
                          stage_events);
}

int gdn_chunk_fwd_pooled(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const int32_t* cu_seqlens_host, int32_t num_seqs, float* state_pool,
                         const gdn_state_slots* slots, void* out, int32_t T, int32_t H_q, int32_t H_v, int32_t d_k,
                         int32_t d_v, float scale, gdn_dtype dtype, void* workspace, size_t workspace_bytes,
                         const gdn_output_gate* gate, hipStream_t stream) {
    if (!slots) return GDN_EINVAL;
    return chunk_fwd_impl(q, k, v, g, beta, cu_seqlens_host, num_seqs, state_pool, out, state_pool, slots, T, H_q,
                          H_v, d_k, d_v, scale, dtype, workspace, workspace_bytes, stream, 0u, gate, nullptr);
}

size_t gdn_chunk_fwd_dev_workspace_size(int32_t T, int32_t num_seqs, int32_t H_q, int32_t H_v, int32_t d_k,
                                        int32_t d_v, gdn_dtype dtype) {
    gdn_workspace_layout L;
    size_t tab_off = 0, total = 0;
    if (dev_layout(T, num_seqs, H_q, H_v, d_k, d_v, dtype, &L, &tab_off, &total) != GDN_OK) return 0;
    return total;
}

int gdn_chunk_fwd_dev(const void* q, const void* k, const void* v, const float* g, const float* beta,
                      const int32_t* cu_seqlens_dev, int32_t num_seqs, const float* initial_state, void* out,
                      float* final_state, int32_t T, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, float scale,
                      gdn_dtype dtype, void* workspace, size_t workspace_bytes, const gdn_output_gate* gate,
                      hipStream_t stream) {
    if (gate) {
        const int grc = check_gate(gate, T > 0);
        if (grc != GDN_OK) return grc;
    }
    gdn_workspace_layout L;
    size_t tab_off = 0, total = 0;
    int rc = dev_layout(T, num_seqs, H_q, H_v, d_k, d_v, dtype, &L, &tab_off, &total);
    if (rc != GDN_OK) return rc;
    if (num_seqs == 0) return GDN_OK;
    // T == 0 still runs: every sequence is empty and its final state is its
    // initial state (or zero), as in gdn_chunk_fwd.
    if (!cu_seqlens_dev || (T > 0 && (!q || !k || !v || !g || !beta || !out))) return GDN_EINVAL;
    const void* ptrs[] = {q, k, v, g, beta, out, initial_state, final_state, workspace};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDN_EUNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(cu_seqlens_dev) & 3u) return GDN_EUNSUPPORTED;
    if (!(scale == scale)) return GDN_EINVAL;
    if (!workspace || workspace_bytes < total) return GDN_EWORKSPACE;

    char* ws = static_cast<char*>(workspace);
    gdn::SeqTable* tabs = reinterpret_cast<gdn::SeqTable*>(ws + tab_off);
    int32_t bins_cap = 1;
    const int32_t ct = dev_scan_shape(num_seqs, T, H_v, d_k, dtype == GDN_BF16, gdn::cu_count(), &bins_cap);
    hipError_t e = gdn::launch_build_tables(cu_seqlens_dev, num_seqs, T, initial_state != nullptr,
                                            final_state != nullptr, bins_cap, tabs, stream);
    if (e != hipSuccess) return hip_fail(e);
    gdn::ChunkParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.s0 = initial_state; p.out = out; p.sfinal = final_state;
    p.gates = reinterpret_cast<float*>(ws + L.off_gates);
    p.A = ws + L.off_A; p.Af = ws + L.off_Af; p.W = ws + L.off_W; p.Ut = ws + L.off_U;
    p.Kc = ws + L.off_Kc;
    p.Ht = ws + L.off_Ht; p.Xt = ws + L.off_Xt;
    p.Pf = dtype == GDN_BF16 ? ws + L.off_P : nullptr;
    p.Qc = dtype == GDN_BF16 ? ws + L.off_Qc : nullptr;
    p.H_q = H_q; p.H_v = H_v; p.G = H_v / H_q; p.scale = scale;
    p.T = T;
    p.aform = a_form(T, num_seqs, H_v, d_k, dtype, gdn::cu_count());
    p.gz = gate ? gate->z : nullptr;
    p.gw = gate ? gate->weight : nullptr;
    p.geps = gate ? gate->eps : 0.f;
    // Per launch group: the host table carries only the grid bounds (sequence
    // count, a chunk-count bound); the kernels read the device table.
    const int64_t nb = chunk_bound(T, num_seqs);
    for (int32_t s0 = 0; s0 < num_seqs; s0 += gdn::MAX_SEQS_PER_LAUNCH) {
        const int32_t ns = std::min<int32_t>(gdn::MAX_SEQS_PER_LAUNCH, num_seqs - s0);
        p.tab.num_seqs = ns;
        p.tab.n_bins = std::min(ns, bins_cap);  // as build_tables computes it
        p.tab.ct = ct;
        p.tab.n_chunks = (int32_t)std::min<int64_t>(nb, ((int64_t)T + GDN_CHUNK - 1) / GDN_CHUNK + ns);
        p.dtab = tabs + s0 / gdn::MAX_SEQS_PER_LAUNCH;
        e = run_chunk(p, dtype, d_k, stream, nullptr);
        if (e != hipSuccess) return hip_fail(e);
    }
    return GDN_OK;
}

int gdn_chunk_fwd_fused(const void* q, const void* k, const void* v, const gdn_front_end* front,
                        const int32_t* cu_seqlens_host, int32_t num_seqs, float* initial_state, void* out,
                        float* final_state, const gdn_state_slots* slots, int32_t T, int32_t H_q, int32_t H_v,
                        int32_t d_k, int32_t d_v, float scale, gdn_dtype dtype, void* workspace,
                        size_t workspace_bytes, const gdn_output_gate* gate, hipStream_t stream) {
    if (!front) return GDN_EINVAL;
    if (slots) {  // initial_state is the pool; final_state NULL or the same pool
        if (final_state && final_state != initial_state) return GDN_EINVAL;
        final_state = initial_state;
    }
    return chunk_fwd_impl(q, k, v, nullptr, nullptr, cu_seqlens_host, num_seqs, initial_state, out, final_state,
                          slots, T, H_q, H_v, d_k, d_v, scale, dtype, workspace, workspace_bytes, stream, 0u, gate,
                          nullptr, front);
}

int gdn_recurrent_step(const void* q, const void* k, const void* v, const float* g, const float* beta, float* state,
                       void* out, int32_t N, int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, float scale,
                       gdn_dtype dtype, hipStream_t stream) {
    int rc = check_shapes(H_q, H_v, d_k, d_v, dtype);
    if (rc != GDN_OK) return rc;
    if (N < 0) return GDN_EINVAL;
    if (N == 0) return GDN_OK;
    if ((int64_t)N * H_v > INT32_MAX) return GDN_EUNSUPPORTED;
    if (!q || !k || !v || !g || !beta || !state || !out) return GDN_EINVAL;
    const void* ptrs[] = {q, k, v, g, beta, state, out};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return GDN_EUNSUPPORTED;
    if (!(scale == scale)) return GDN_EINVAL;
    gdn::DecodeParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.state = state; p.out = out;
    p.slot = nullptr; p.pool = N;
    p.N = N; p.H_q = H_q; p.H_v = H_v; p.G = H_v / H_q; p.scale = scale;
    const hipError_t e = run_decode<false>(p, dtype, d_k, stream);
    if (e != hipSuccess) return hip_fail(e);
    return GDN_OK;
}

int gdn_recurrent_step_fused(const void* q, const void* k, const void* v, const void* a, const void* b,
                             const float* A_log, const float* dt_bias, float* state, void* out, int32_t N,
                             int32_t H_q, int32_t H_v, int32_t d_k, int32_t d_v, float scale, gdn_dtype dtype,
                             const gdn_output_gate* gate, hipStream_t stream) {
    if (!state && N > 0) return GDN_EINVAL;
    return step_fused_impl(q, k, v, a, b, A_log, dt_bias, state, nullptr, N, out, N, H_q, H_v, d_k, d_v, scale, dtype,
                           gate, stream);
}

int gdn_recurrent_step_fused_pooled(const void* q, const void* k, const void* v, const void* a, const void* b,
                                    const float* A_log, const float* dt_bias, float* state_pool, const int32_t* slot,
                                    int32_t pool_size, void* out, int32_t N, int32_t H_q, int32_t H_v, int32_t d_k,
                                    int32_t d_v, float scale, gdn_dtype dtype, const gdn_output_gate* gate,
                                    hipStream_t stream) {
    if (!slot && N > 0) return GDN_EINVAL;
    return step_fused_impl(q, k, v, a, b, A_log, dt_bias, state_pool, slot, pool_size, out, N, H_q, H_v, d_k, d_v,
                           scale, dtype, gate, stream);
}

int gdn_state_rows_zero(void* pool, int32_t pool_size, size_t row_bytes, const int32_t* rows, int32_t n,
                        hipStream_t stream) {
    return gdn_state_rows_copy(pool, pool_size, row_bytes, nullptr, rows, n, stream);
}

int gdn_state_rows_copy(void* pool, int32_t pool_size, size_t row_bytes, const int32_t* src_rows,
                        const int32_t* dst_rows, int32_t n, hipStream_t stream) {
    if (n < 0 || pool_size < 0 || row_bytes == 0) return GDN_EINVAL;
    if (row_bytes % 16 != 0) return GDN_EUNSUPPORTED;
    if (n == 0 || pool_size == 0) return GDN_OK;
    if (!pool || !dst_rows) return GDN_EINVAL;
    if (!aligned16(pool) || (reinterpret_cast<uintptr_t>(dst_rows) & 3u) ||
        (reinterpret_cast<uintptr_t>(src_rows) & 3u))
        return GDN_EUNSUPPORTED;
    if (row_bytes > SIZE_MAX / (size_t)pool_size) return GDN_EINVAL;
    gdn::PoolRowsParams p{};
    p.base = static_cast<char*>(pool);
    p.src = src_rows;
    p.dst = dst_rows;
    p.pool = pool_size;
    p.row16 = row_bytes / 16;
    const hipError_t e = gdn::launch_pool_rows(p, n, stream);
    if (e != hipSuccess) return hip_fail(e);
    return GDN_OK;
}

}  // extern "C"
