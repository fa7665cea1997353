// Recurrent Gated DeltaNet decode step for gfx950.
//
// The update of one (sequence, value head) state S (d_k x d_v, fp32) for one
// token ("实验三：GDN Prefill 前向优化", section "GLA, DeltaNet 与 Gated DeltaNet";
// "Qwen3.5-397B-A17B" trace page, Decode-GDN node 7, its decay / delta / read
// steps):
//     Sbar = alpha S,  delta = beta (v - k Sbar),  S' = Sbar + k^T delta,  o = scale q S'.
// It is computed in ONE pass over S: k Sbar = alpha (k S) and
// q S' = alpha (q S) + (q . k) delta, so both column reductions k S and q S are
// taken from the values read once, and S' is written once.  The pass is bound
// by HBM bandwidth (64 KiB read + 64 KiB written per head at d = 128).
//
// The fused variant takes the raw inputs of that node instead (its first two
// steps): k_bar = k / sqrt(sum k^2 + 1e-6), q_bar = scale q / sqrt(sum q^2 +
// 1e-6), g = -exp(A_log) softplus(a + dt_bias) (softplus(x) = ln(1 + e^x) in
// an overflow-free form, front_gate), beta = sigmoid(b)
// rounded to the input dtype (bf16 keeps that rounding, as the trace page
// notes).  The two sums of squares ride along with the column reductions, and
// the norms are applied as scalars afterwards, so the state is still read
// and written once.
//
// One 256-thread workgroup per (sequence, value head).  Thread t owns a 16-byte
// column group cg = t % (d/4) of rows rg + RG*m (RG = 1024/d row groups), so
// each wave reads whole contiguous rows with 128-bit loads; the updated state
// goes back with non-temporal 128-bit stores.  Column sums are
// reduced across row groups with lane shuffles inside a wave and through LDS
// across the four waves.
#include "gdn_device.h"
#include "gdn_params.h"

namespace gdn {

template <typename T, int D, bool FUSED>
__global__ __launch_bounds__(256) void recurrent_step_kernel(const DecodeParams p) {
    constexpr int CPR = D / 4;      // float4 column groups per row
    constexpr int RG = 256 / CPR;   // row groups
    constexpr int RPT = D / RG;     // rows per thread
    constexpr int RGW = 64 / CPR;   // row groups per wave
    constexpr int NV = FUSED ? 11 : 9;  // reduced values: k S (4), q S (4), q . k [, k . k, q . q]
    const int nh = blockIdx.x;
    const int n = nh / p.H_v, h = nh % p.H_v;
    const int hq = h / p.G;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int cg = tid % CPR, rg = tid / CPR;

    __shared__ float s_red[4][CPR][NV];

    // State row of this sequence; padding (negative or out-of-pool slot) reads
    // and writes no state and yields a zero output row.
    const int slot = p.slot ? p.slot[n] : n;
    if (slot < 0 || slot >= p.pool) {
        if (tid < D / 4) store4(reinterpret_cast<T*>(p.out) + (size_t)nh * D + 4 * tid, 0.f, 0.f, 0.f, 0.f);
        return;  // whole workgroup
    }
    const size_t sidx = ((size_t)slot * p.H_v + h) * D * D;
    float4* Sp = reinterpret_cast<float4*>(p.state + sidx);
    const T* qp = reinterpret_cast<const T*>(p.q) + ((size_t)n * p.H_q + hq) * D;
    const T* kp = reinterpret_cast<const T*>(p.k) + ((size_t)n * p.H_q + hq) * D;
    const T* vp = reinterpret_cast<const T*>(p.v) + (size_t)nh * D;
    float alpha, beta;
    if constexpr (FUSED) {
        alpha = expf(front_gate(to_f32<T>(reinterpret_cast<const T*>(p.a)[nh]), p.A_log[h], p.dt_bias[h]));
        beta = front_beta<T>(to_f32<T>(reinterpret_cast<const T*>(p.b)[nh]));  // rounded to the input dtype (RNE)
    } else {
        alpha = __expf(p.g[nh]);
        beta = p.beta[nh];
    }

    float4 s[RPT];
    float kr[RPT], qr[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) s[m] = Sp[(rg + RG * m) * CPR + cg];
    // The q / k elements go out after the state rows (issuing them first, or
    // interleaved, measured 5 % slower: 182 against 173 us for 256 x 32 heads),
    // and for the plain bf16 step as one 4-byte word per lane spread by lane
    // shuffles rather than 2 x RPT two-byte loads per thread (173 -> 164 us; the
    // fused step, which waits for its gate inputs first, measured 164 -> 171 us
    // with the shuffles and keeps the element loads).
    if constexpr (sizeof(T) == 2 && !FUSED) {
        constexpr int NW = D / 2;  // 4-byte words of q (and k)
        const int wl = lane % NW;
        const unsigned kw = reinterpret_cast<const unsigned*>(kp)[wl];
        const unsigned qw = reinterpret_cast<const unsigned*>(qp)[wl];
        const int sh = (rg & 1) ? 16 : 0;  // RG is even: every row of this thread has rg's parity
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int src = (rg + RG * m) >> 1;
            const unsigned ku = (unsigned)__shfl((int)kw, src, 64), qu = (unsigned)__shfl((int)qw, src, 64);
            kr[m] = __uint_as_float((ku >> sh) << 16);
            qr[m] = __uint_as_float((qu >> sh) << 16);
        }
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int row = rg + RG * m;
            kr[m] = to_f32<T>(kp[row]);
            qr[m] = to_f32<T>(qp[row]);
        }
    }
    float red[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) red[e] = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        red[0] += kr[m] * s[m].x;
        red[1] += kr[m] * s[m].y;
        red[2] += kr[m] * s[m].z;
        red[3] += kr[m] * s[m].w;
        red[4] += qr[m] * s[m].x;
        red[5] += qr[m] * s[m].y;
        red[6] += qr[m] * s[m].z;
        red[7] += qr[m] * s[m].w;
        red[8] += qr[m] * kr[m];
        if constexpr (FUSED) {
            red[9] += kr[m] * kr[m];
            red[10] += qr[m] * qr[m];
        }
    }
    // Row groups inside a wave differ in the lane bits above log2(CPR).
#pragma unroll
    for (int msk = CPR; msk < 64; msk <<= 1)
#pragma unroll
        for (int e = 0; e < NV; ++e) red[e] += wave_shfl_xor(red[e], msk);
    if (lane < CPR) {
#pragma unroll
        for (int e = 0; e < NV; ++e) s_red[w][lane][e] = red[e];
    }
    lds_sync();
#pragma unroll
    for (int e = 0; e < NV; ++e) red[e] = s_red[0][cg][e] + s_red[1][cg][e] + s_red[2][cg][e] + s_red[3][cg][e];
    (void)RGW;

    float vv[4];
    load4(vp + 4 * cg, vv[0], vv[1], vv[2], vv[3]);
    // Norm factors (1 and scale for the plain step, whose q, k arrive normalised).
    float rk = 1.f, rq = p.scale;
    if constexpr (FUSED) {
        rk = 1.f / sqrtf(red[9] + 1e-6f);
        rq = p.scale / sqrtf(red[10] + 1e-6f);
    }
    float dl[4], o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        dl[c] = beta * (vv[c] - alpha * rk * red[c]);
        o[c] = rq * (alpha * red[4 + c] + rk * red[8] * dl[c]);
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int row = rg + RG * m;
        float4 t = s[m];
        const float kn = rk * kr[m];
        t.x = alpha * t.x + kn * dl[0];
        t.y = alpha * t.y + kn * dl[1];
        t.z = alpha * t.z + kn * dl[2];
        t.w = alpha * t.w + kn * dl[3];
        // non-temporal: the state is not touched again by this step, and keeping
        // it out of the caches measurably raises the read/write stream rate
        __builtin_nontemporal_store(f32x4{t.x, t.y, t.z, t.w}, reinterpret_cast<f32x4*>(&Sp[row * CPR + cg]));
    }
    if constexpr (FUSED) {
        if (p.gz) {
            // Gated read-out (trace page, Decode-GDN node 8): every group of CPR
            // consecutive lanes holds the head's d_v outputs, 4 per lane.
            float ssq = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
#pragma unroll
            for (int msk = 1; msk < CPR; msk <<= 1) ssq += wave_shfl_xor(ssq, msk);
            const float rstd = 1.f / sqrtf(ssq * (1.f / D) + p.geps);
            float zv[4];
            load4(reinterpret_cast<const T*>(p.gz) + (size_t)nh * D + 4 * cg, zv[0], zv[1], zv[2], zv[3]);
            const float4 wv = *reinterpret_cast<const float4*>(p.gw + 4 * cg);
            const float wf[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = o[c] * rstd * wf[c] * silu_f32(zv[c]);
        }
    }
    if (rg == 0) store4(reinterpret_cast<T*>(p.out) + (size_t)nh * D + 4 * cg, o[0], o[1], o[2], o[3]);
}

template <typename T, int D, bool FUSED>
hipError_t launch_recurrent_step(const DecodeParams& p, hipStream_t stream) {
    const int nwg = p.N * p.H_v;
    if (nwg > 0) hipLaunchKernelGGL((recurrent_step_kernel<T, D, FUSED>), dim3(nwg), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template hipError_t launch_recurrent_step<bf16, 128, false>(const DecodeParams&, hipStream_t);
template hipError_t launch_recurrent_step<bf16, 64, false>(const DecodeParams&, hipStream_t);
template hipError_t launch_recurrent_step<float, 128, false>(const DecodeParams&, hipStream_t);
template hipError_t launch_recurrent_step<float, 64, false>(const DecodeParams&, hipStream_t);
template hipError_t launch_recurrent_step<bf16, 128, true>(const DecodeParams&, hipStream_t);
template hipError_t launch_recurrent_step<bf16, 64, true>(const DecodeParams&, hipStream_t);
template hipError_t launch_recurrent_step<float, 128, true>(const DecodeParams&, hipStream_t);
template hipError_t launch_recurrent_step<float, 64, true>(const DecodeParams&, hipStream_t);

}  // namespace gdn
