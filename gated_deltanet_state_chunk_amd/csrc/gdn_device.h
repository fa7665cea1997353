// Device helpers shared by the gfx950 kernels: MFMA fragments, element
// conversion, layout permutation and XCD-aware work mapping.
//
// MFMA conventions (gfx950, wave64).  A 16x16 output tile D = A B + C is held
// as f32x4 per lane: lane l holds column (l & 15), rows 4*(l >> 4) + {0..3}.
// An operand fragment covers 16 rows (A) or 16 columns (B) by 32 contraction
// indices and holds 8 values per lane: lane l serves row/column (l & 15) and
// slots j = 0..7 of lane group a = (l >> 4).  Which contraction index a slot
// stands for is a free choice as long as A and B agree; two conventions are
// used:
//   * "contiguous": slot j of group a is index 8a + j (both operands loaded
//     from memory with 16-byte loads);
//   * "perm32": slot j = 4h + b of group a is index 16h + 4a + b, so that two
//     vertically stacked D tiles (rows 0..15 and 16..31) ARE a B fragment
//     without any data movement.  Operands stored in memory with the perm32
//     layout (index 16h + 4a + b at offset 8a + 4h + b) load with one 16-byte
//     access per fragment.
// For bf16 one fragment feeds one v_mfma_f32_16x16x32_bf16; for fp32 it feeds
// eight v_mfma_f32_16x16x4_f32, instruction j consuming slot j of every lane
// (group a supplies contraction row a), which is the same pairing.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int CHUNK = 64;

// 8-value operand fragment of element type T.
template <typename T>
struct Frag;
template <>
struct Frag<bf16> {
    bf16x8 v;
};
template <>
struct Frag<f16> {
    f16x8 v;
};
template <>
struct Frag<float> {
    float v[8];
};

// Element type of chunk_prep's W and U products and of the stored U: fp16 for
// bf16 inputs (the same two bytes as bf16 and the same MFMA rate, with three
// more mantissa bits for values well inside its range), fp32 for fp32 inputs.
template <typename T>
using ProdT = std::conditional_t<sizeof(T) == 2, f16, float>;

__device__ __forceinline__ f32x4 mma(const Frag<bf16>& a, const Frag<bf16>& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<f16>& a, const Frag<f16>& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---- element conversion --------------------------------------------------
template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }
template <>
__device__ __forceinline__ float to_f32<f16>(f16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // round to nearest even
template <>
__device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }  // round to nearest even

// ---- fragment loads ------------------------------------------------------
// 8 consecutive elements at p (16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ void load8(Frag<bf16>& f, const bf16* p) { f.v = *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void load8(Frag<float>& f, const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// Same, but the 8 values are zero when `valid` is false (no memory access).
template <typename T>
__device__ __forceinline__ void load8_masked(Frag<T>& f, const T* p, bool valid) {
    if (valid) {
        load8(f, p);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) f.v[j] = from_f32<T>(0.f);
    }
}

// Set slot j of a fragment from an fp32 value.
template <typename T>
__device__ __forceinline__ void frag_set(Frag<T>& f, int j, float x) {
    f.v[j] = from_f32<T>(x);
}
template <typename T>
__device__ __forceinline__ float frag_get(const Frag<T>& f, int j) {
    return to_f32<T>(f.v[j]);
}

// Two stacked D tiles (rows 0..15 -> lo, rows 16..31 -> hi) as a perm32 B fragment,
// each value multiplied by s.
template <typename T>
__device__ __forceinline__ Frag<T> pack_perm32(const f32x4& lo, const f32x4& hi, float s) {
    Frag<T> f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f.v[b] = from_f32<T>(lo[b] * s);
        f.v[4 + b] = from_f32<T>(hi[b] * s);
    }
    return f;
}

// Four fp32 values times s, rounded to T (vector conversion: packed cvt for bf16).
__device__ __forceinline__ bf16x4 cvt4_bf16(const f32x4& v, float s) {
    return __builtin_convertvector(v * s, bf16x4);
}

// ---- stores of 4 consecutive values --------------------------------------
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
    bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
// Two groups of four values to 8 consecutive elements (one 16-byte store for bf16).
__device__ __forceinline__ void store8(bf16* p, const f32x4& lo, const f32x4& hi) {
    const bf16x4 a = __builtin_convertvector(lo, bf16x4), b = __builtin_convertvector(hi, bf16x4);
    *reinterpret_cast<bf16x8*>(p) = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void store8(f16* p, const f32x4& lo, const f32x4& hi) {
    const f16x4 a = __builtin_convertvector(lo, f16x4), b = __builtin_convertvector(hi, f16x4);
    *reinterpret_cast<f16x8*>(p) = f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void store8(float* p, const f32x4& lo, const f32x4& hi) {
    *reinterpret_cast<float4*>(p) = make_float4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(hi[0], hi[1], hi[2], hi[3]);
}
__device__ __forceinline__ void load4(const bf16* p, float& a, float& b, float& c, float& d) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    a = (float)v[0]; b = (float)v[1]; c = (float)v[2]; d = (float)v[3];
}
__device__ __forceinline__ void load4(const float* p, float& a, float& b, float& c, float& d) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    a = v.x; b = v.y; c = v.z; d = v.w;
}

// Four raw elements (kept unconverted so that a prefetch does not force a wait).
template <typename T>
struct Raw4;
template <>
struct Raw4<bf16> {
    bf16x4 v;
};
template <>
struct Raw4<f16> {
    f16x4 v;
};
template <>
struct Raw4<float> {
    float4 v;
};
__device__ __forceinline__ void load_raw4(Raw4<bf16>& r, const bf16* p) { r.v = *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ void load_raw4(Raw4<float>& r, const float* p) { r.v = *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ f32x4 raw4_to_f32(const Raw4<bf16>& r) {
    return f32x4{(float)r.v[0], (float)r.v[1], (float)r.v[2], (float)r.v[3]};
}
__device__ __forceinline__ f32x4 raw4_to_f32(const Raw4<f16>& r) {
    return f32x4{(float)r.v[0], (float)r.v[1], (float)r.v[2], (float)r.v[3]};
}
__device__ __forceinline__ f32x4 raw4_to_f32(const Raw4<float>& r) { return f32x4{r.v.x, r.v.y, r.v.z, r.v.w}; }

// perm32 storage offset of logical index i.
__host__ __device__ __forceinline__ int perm32(int i) {
    const int blk = i & ~31, r = i & 31;
    const int h = r >> 4, a = (r >> 2) & 3, b = r & 3;
    return blk + 8 * a + 4 * h + b;
}

// ---- XCD-aware work mapping ----------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i % 8).  Mapping workgroup i to work item (i % 8) * per + i / 8 hands
// each XCD one contiguous run of work items, so neighbouring items (the value
// heads sharing a key head, consecutive chunks of a sequence) share that XCD's
// L2.  `padded` is the grid size, a multiple of 8.
__device__ __forceinline__ int xcd_remap(int i, int padded) { return (i & 7) * (padded >> 3) + (i >> 3); }

// ---- workgroup barrier ---------------------------------------------------
// s_waitcnt lgkmcnt(0): this wave's LDS operations have completed.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Workgroup barrier that publishes this wave's LDS writes.  The release fence
// of __syncthreads() emits no LDS wait when only LDS ordering is at stake (the
// compiler takes LDS operations of all waves to be performed in one global
// order); on gfx950, with direct-to-LDS loads streaming into the same LDS, a
// ds_write issued before s_barrier was observed to be missed by another wave's
// ds_read issued after it.  Every barrier here therefore waits explicitly.
__device__ __forceinline__ void lds_sync() {
    wait_lgkmcnt0();
    __syncthreads();
}

// ---- wave helpers --------------------------------------------------------
__device__ __forceinline__ float wave_shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// Sum of x over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the same lane of the four
// 16-lane rows), every one of them receiving the same bits.  gfx950's lane
// swaps are VALU instructions: v_permlane16_swap exchanges the odd rows of its
// first operand with the even rows of its second, v_permlane32_swap the upper
// half of the first with the lower half of the second, so with both operands
// equal the two results add to the pairwise sums.  A shuffle (ds_bpermute)
// would travel through the LDS unit and queue behind the LDS traffic of a busy
// workgroup.
__device__ __forceinline__ float sum_over_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---- transposed LDS reads (gfx950 ds_read_b64_tr_b16) ----------------------
// Rows r0 .. r0+3 of column c0 + (lane % 16) of a row-major bf16 matrix in LDS
// (row stride RS elements; r0 uniform within each group of 16 lanes, c0 a
// multiple of 16, 8-byte aligned addresses).  In one ds_read_b64_tr_b16, lane j
// of a 16-lane group supplies the address of 4 elements (8 bytes) and lane i
// receives element i % 4 of the chunks of lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12,
// in that order (layout checked on the device); so lane j points at row
// r0 + j/4, columns c0 + 4 (j % 4) .. + 3, and lane i gets column c0 + i.
template <int RS>
__device__ __forceinline__ bf16x4 lds_col4(const bf16* base, int r0, int c0, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int j = lane & 15;
    const bf16* a = base + (r0 + (j >> 2)) * RS + c0 + 4 * (j & 3);
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)a);
    return __builtin_bit_cast(bf16x4, r);
}

// ---- row L2 normalisation of staged rows ---------------------------------
// A D-element row held as 16-byte pieces by D / (16 / sizeof(T)) consecutive
// lanes (aligned groups inside one wave): each lane returns its piece times
// 1 / sqrt(sum over the row of x^2 + 1e-6), rounded to T, and that factor in
// rnorm.  All lanes of the wave must take part (the sum is reduced with lane
// shuffles).
template <typename T, int D>
__device__ __forceinline__ float4 l2norm_piece(float4 raw, float& rnorm) {
    constexpr int VEC = 16 / (int)sizeof(T);
    constexpr int LPR = D / VEC;  // lanes per row
    static_assert(LPR <= 64 && (LPR & (LPR - 1)) == 0, "row must fit a power-of-two lane group");
    if constexpr (sizeof(T) == 2) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, raw);
        float x[8];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = (float)v[i];
            ss += x[i] * x[i];
        }
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
        const float r = 1.f / sqrtf(ss + 1e-6f);
        rnorm = r;
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (bf16)(x[i] * r);
        return __builtin_bit_cast(float4, o);
    } else {
        float ss = raw.x * raw.x + raw.y * raw.y + raw.z * raw.z + raw.w * raw.w;
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
        const float r = 1.f / sqrtf(ss + 1e-6f);
        rnorm = r;
        return make_float4(raw.x * r, raw.y * r, raw.z * r, raw.w * r);
    }
}
template <typename T, int D>
__device__ __forceinline__ float4 l2norm_piece(float4 raw) {
    float r;
    return l2norm_piece<T, D>(raw, r);
}

// ---- SiLU ------------------------------------------------------------------
// x * sigmoid(x) with the hardware reciprocal (v_rcp_f32, about 1 ulp) rather
// than an IEEE division sequence, which dominated the VALU time where SiLU is
// applied per element (the convolution, the gated read-out).
__device__ __forceinline__ float silu_f32(float x) { return x * __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// ---- gate transform of the front end ---------------------------------------
// g = -exp(A_log) softplus(a + dt_bias), with softplus(x) = ln(1 + e^x) taken
// as max(x, 0) + ln(1 + e^-|x|): the exponential never overflows, and where |x|
// is large the correction term drops below rounding of its own accord (above
// x = 17 it is under half an fp32 ulp of x; below x = -88 e^x underflows).
__device__ __forceinline__ float front_gate(float a, float A_log, float dt_bias) {
    const float x = a + dt_bias;
    return -expf(A_log) * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))));
}
// beta = sigmoid(b) rounded to T (the activation dtype the gating hands on).
template <typename T>
__device__ __forceinline__ float front_beta(float b) {
    return to_f32<T>(from_f32<T>(1.f / (1.f + expf(-b))));
}

}  // namespace gdn
