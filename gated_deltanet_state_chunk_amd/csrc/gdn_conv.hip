// Short causal depthwise convolution + SiLU with its input history, for gfx950.
//
// "Qwen3.5-397B-A17B" trace page, Decode-GDN node 6
// (qkvzba_unpack_causal_conv1d_silu): per channel c,
//     y_{t,c} = SiLU(sum_l w_{c,l} x_{t-l,c} + b_c)      (b = 0 without bias)
// with the taps stored oldest first (w[c][K-1] on the current input, the
// window [s_0 .. s_{K-2}, x_t] of the "Kestrel_VLLM - 24" page, section 三),
// and a per-sequence history of the K-1 previous raw inputs ([K-1][C], row 0
// the oldest) that the next call continues from.  The output keeps the
// rounding to the input dtype the trace page notes for this node.
//
// Every thread owns 16 bytes of channels (8 bf16 or 4 fp32) and a K-tap window
// over its tokens in registers: per token one coalesced 16-byte load and one
// 16-byte store, weights held in registers.  The op is bound by
// HBM bandwidth (x read once, y written once).
//   conv_prefill_kernel     one thread per (16 tokens of a sequence, channel group), all
//                           of its window's loads issued together
//   conv_final_state_kernel each sequence's last K-1 inputs, launched after it
//                           (stream order makes final_state == initial_state safe)
//   conv_step_kernel        one decode token per sequence, four sequences a thread
//                           (the taps read once for them), history updated in place
#include "gdn_device.h"
#include "gdn_params.h"

namespace gdn {

namespace {

template <typename T>
struct Vec16;  // 16 bytes of channels
template <>
struct Vec16<bf16> {
    static constexpr int N = 8;
    bf16x8 v;
};
template <>
struct Vec16<float> {
    static constexpr int N = 4;
    float4 v;
};

template <typename T>
__device__ __forceinline__ Vec16<T> ld16(const T* p) {
    Vec16<T> r;
    if constexpr (sizeof(T) == 2)
        r.v = *reinterpret_cast<const bf16x8*>(p);
    else
        r.v = *reinterpret_cast<const float4*>(p);
    return r;
}
template <typename T>
__device__ __forceinline__ void st16(T* p, const Vec16<T>& r) {
    if constexpr (sizeof(T) == 2)
        *reinterpret_cast<bf16x8*>(p) = r.v;
    else
        *reinterpret_cast<float4*>(p) = r.v;
}
template <typename T>
__device__ __forceinline__ float get(const Vec16<T>& r, int i) {
    if constexpr (sizeof(T) == 2)
        return (float)r.v[i];
    else
        return i == 0 ? r.v.x : i == 1 ? r.v.y : i == 2 ? r.v.z : r.v.w;
}
template <typename T>
__device__ __forceinline__ Vec16<T> zero16() {
    Vec16<T> r;
    if constexpr (sizeof(T) == 2)
        r.v = bf16x8{};
    else
        r.v = make_float4(0.f, 0.f, 0.f, 0.f);
    return r;
}
template <typename T>
__device__ __forceinline__ Vec16<T> from_floats(const float* f) {
    Vec16<T> r;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) r.v[i] = (bf16)f[i];
    } else {
        r.v = make_float4(f[0], f[1], f[2], f[3]);
    }
    return r;
}

__device__ __forceinline__ float silu(float a) { return silu_f32(a); }

// The weights [C][K] of a thread's V channels are K*V consecutive floats
// starting 16-byte aligned (c is a multiple of V): load them as float4s.
template <int K, int V>
__device__ __forceinline__ void load_taps(const ConvParams& p, int c, float (&wk)[K][V], float (&bc)[V]) {
    float f[K * V];
    const float4* w4 = reinterpret_cast<const float4*>(p.w + (size_t)c * K);
#pragma unroll
    for (int j = 0; j < K * V / 4; ++j) {
        const float4 t = w4[j];
        f[4 * j] = t.x; f[4 * j + 1] = t.y; f[4 * j + 2] = t.z; f[4 * j + 3] = t.w;
    }
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
        for (int k = 0; k < K; ++k) wk[k][i] = f[i * K + k];
    if (p.b) {
        const float4* b4 = reinterpret_cast<const float4*>(p.b + c);
#pragma unroll
        for (int j = 0; j < V / 4; ++j) {
            const float4 t = b4[j];
            bc[4 * j] = t.x; bc[4 * j + 1] = t.y; bc[4 * j + 2] = t.z; bc[4 * j + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) bc[i] = 0.f;
    }
}

// Sequence owning global chunk ci (largest n with choff[n] <= ci).
__device__ __forceinline__ int seq_of_chunk(const SeqTable& tab, int ci) {
    int lo = 0, hi = tab.num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tab.choff[mid] <= ci)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Input at token position p (global) of sequence n, channel group base c:
// from x inside the sequence, from its history before it (or zero).
template <typename T, int K>
__device__ __forceinline__ Vec16<T> input_at(const ConvParams& p, int n, int p_tok, int c) {
    const int s0 = p.tab.cu[n];
    if (p_tok >= s0) return ld16(reinterpret_cast<const T*>(p.x) + (size_t)p_tok * p.C + c);
    const int si = p.tab.s_in[n];
    if (si < 0) return zero16<T>();
    const int j = K - 1 + (p_tok - s0);  // history row, 0 = oldest
    return ld16(reinterpret_cast<const T*>(p.s_in) + ((size_t)si * (K - 1) + j) * p.C + c);
}

constexpr int CONV_SUB = 16;  // tokens per thread (a quarter of a chunk)

template <typename T, int K>
__global__ __launch_bounds__(256) void conv_prefill_kernel(const ConvParams p) {
    constexpr int V = Vec16<T>::N;
    constexpr int R = CONV_SUB;
    // Channel blocks vary fastest across the grid, so workgroups running together
    // cover whole rows of x (measured: 38 -> 32 us at T = 4096, C = 8192).
    const int cg = blockIdx.x * 256 + threadIdx.x;
    if (cg * V >= p.C) return;
    const int c = cg * V;
    const int qi = p.q0 + blockIdx.y;  // quarter-chunk index in this launch
    const int ci = p.tab.chunk_begin + qi / (CHUNK / R);
    const int n = seq_of_chunk(p.tab, ci);
    const int t0 = p.tab.cu[n] + (ci - p.tab.choff[n]) * CHUNK + (qi % (CHUNK / R)) * R;
    const int t1 = min(t0 + R, p.tab.cu[n + 1]);
    if (t0 >= t1) return;  // a tail chunk's unused quarters (whole workgroup)
    // All inputs of this thread's window go out at once: the K-1 before t0
    // (x or history) and the R tokens (clamped to the sequence; never stored past t1).
    Vec16<T> win[K - 1 + R];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) win[k] = input_at<T, K>(p, n, t0 - (K - 1) + k, c);
    const T* xb = reinterpret_cast<const T*>(p.x) + c;
#pragma unroll
    for (int r = 0; r < R; ++r) win[K - 1 + r] = ld16(xb + (size_t)min(t0 + r, t1 - 1) * p.C);
    float wk[K][V], bc[V];
    load_taps<K, V>(p, c, wk, bc);
    T* yb = reinterpret_cast<T*>(p.y) + c;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float y[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float a = bc[i];
#pragma unroll
            for (int k = 0; k < K; ++k) a += wk[k][i] * get(win[r + k], i);
            y[i] = silu(a);
        }
        if (t0 + r < t1) st16(yb + (size_t)(t0 + r) * p.C, from_floats<T>(y));
    }
}

template <typename T, int K>
__global__ __launch_bounds__(256) void conv_final_state_kernel(const ConvParams p) {
    constexpr int V = Vec16<T>::N;
    const int cg = blockIdx.y * 256 + threadIdx.x;
    if (cg * V >= p.C) return;
    const int c = cg * V, n = blockIdx.x;
    const int so = p.tab.s_out[n];
    if (so < 0) return;  // this sequence keeps no history (whole workgroup)
    const int end = p.tab.cu[n + 1];
    Vec16<T> last[K - 1];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) last[j] = input_at<T, K>(p, n, end - (K - 1) + j, c);
#pragma unroll
    for (int j = 0; j < K - 1; ++j)
        st16(reinterpret_cast<T*>(p.s_out) + ((size_t)so * (K - 1) + j) * p.C + c, last[j]);
}

// Decode step: each thread serves STEP_SEQS sequences for its 16 bytes of
// channels, so its taps are read once for all of them (per workgroup they are
// 32 KiB, as much as the step's own traffic for one sequence each) and the
// loads of all its sequences are in flight together.
constexpr int STEP_SEQS = 4;

template <typename T, int K>
__global__ __launch_bounds__(256) void conv_step_kernel(const ConvParams p, int N) {
    constexpr int V = Vec16<T>::N;
    const int cg = blockIdx.y * 256 + threadIdx.x;
    if (cg * V >= p.C) return;
    const int c = cg * V, n0 = blockIdx.x * STEP_SEQS;
    // window per sequence: its K-1 history rows, then its input; padding
    // (slot outside the pool) reads and writes no history, outputs zeros
    Vec16<T> win[STEP_SEQS][K];
    T* st[STEP_SEQS];
    bool live[STEP_SEQS];
#pragma unroll
    for (int j = 0; j < STEP_SEQS; ++j) {
        const int n = n0 + j;
        const int slot = n < N ? (p.slot ? p.slot[n] : n) : -1;
        live[j] = slot >= 0 && slot < p.pool;
        st[j] = reinterpret_cast<T*>(p.s_out) + (size_t)max(slot, 0) * (K - 1) * p.C + c;
        if (live[j]) {
#pragma unroll
            for (int k = 0; k < K - 1; ++k) win[j][k] = ld16(st[j] + (size_t)k * p.C);
            win[j][K - 1] = ld16(reinterpret_cast<const T*>(p.x) + (size_t)n * p.C + c);
        }
    }
    float wk[K][V], bc[V];
    load_taps<K, V>(p, c, wk, bc);
#pragma unroll
    for (int j = 0; j < STEP_SEQS; ++j) {
        const int n = n0 + j;
        if (n >= N) break;
        T* yrow = reinterpret_cast<T*>(p.y) + (size_t)n * p.C + c;
        if (!live[j]) {
            st16(yrow, zero16<T>());
            continue;
        }
        float y[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float a = bc[i];
#pragma unroll
            for (int k = 0; k < K; ++k) a += wk[k][i] * get(win[j][k], i);
            y[i] = silu(a);
        }
        st16(yrow, from_floats<T>(y));
#pragma unroll
        for (int k = 0; k < K - 1; ++k) st16(st[j] + (size_t)k * p.C, win[j][k + 1]);
    }
}

}  // namespace

template <typename T, int K>
hipError_t launch_conv_prefill(const ConvParams& p, hipStream_t stream) {
    constexpr int V = Vec16<T>::N;
    const int cblocks = (p.C / V + 255) / 256;
    const int nq = p.tab.n_chunks * (CHUNK / CONV_SUB);
    for (int q0 = 0; q0 < nq; q0 += 65535) {  // grid y is limited to 65535
        ConvParams pq = p;
        pq.q0 = q0;
        hipLaunchKernelGGL((conv_prefill_kernel<T, K>), dim3(cblocks, min(65535, nq - q0)), dim3(256), 0, stream,
                           pq);
    }
    if (p.s_out && p.tab.num_seqs > 0)  // rows with s_out < 0 return at once
        hipLaunchKernelGGL((conv_final_state_kernel<T, K>), dim3(p.tab.num_seqs, cblocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int K>
hipError_t launch_conv_step(const ConvParams& p, int N, hipStream_t stream) {
    constexpr int V = Vec16<T>::N;
    const int cblocks = (p.C / V + 255) / 256;
    if (N > 0)
        hipLaunchKernelGGL((conv_step_kernel<T, K>), dim3((N + STEP_SEQS - 1) / STEP_SEQS, cblocks), dim3(256), 0, stream,
                           p, N);
    return hipGetLastError();
}

#define GDN_CONV_INST(T, K)                                                   \
    template hipError_t launch_conv_prefill<T, K>(const ConvParams&, hipStream_t); \
    template hipError_t launch_conv_step<T, K>(const ConvParams&, int, hipStream_t);
GDN_CONV_INST(bf16, 2)
GDN_CONV_INST(bf16, 3)
GDN_CONV_INST(bf16, 4)
GDN_CONV_INST(float, 2)
GDN_CONV_INST(float, 3)
GDN_CONV_INST(float, 4)
#undef GDN_CONV_INST

}  // namespace gdn
