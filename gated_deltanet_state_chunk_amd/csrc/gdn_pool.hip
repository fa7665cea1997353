// Row maintenance of state pools for serving: reset rows to zero (a new
// sequence reusing a slot) and copy rows (cloning a sequence's state into
// another slot, e.g. for a speculative branch).  The "Qwen3.5-397B-A17B"
// trace page (section 3.6.5) asks that padding slots, invalid state indices
// and slot reuse keep their cache semantics; the "Kestrel_VLLM - 24" page (section 五, the
// state mirror) keeps a reset of its single state for slot reuse and leaves branch
// cloning for speculative decoding to a later stage.  A pool is
// [rows][row_bytes]; the recurrent state pool and the conv history pool are
// both maintained with this one kernel.
//
// One workgroup column per listed row, 16-byte vector loads and stores
// (HBM bound: a row is read once and written once, or only written).
#include "gdn_device.h"
#include "gdn_params.h"

namespace gdn {

namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void pool_rows_kernel(const PoolRowsParams p) {
    const int i = p.i0 + blockIdx.y;
    const int dst = p.dst[i];
    if (dst < 0 || dst >= p.pool) return;  // skipped entry (whole workgroup)
    int src = -1;
    if (p.src) {
        src = p.src[i];
        if (src < 0 || src >= p.pool) return;
    }
    u32x4v* d = reinterpret_cast<u32x4v*>(p.base) + (size_t)dst * p.row16;
    const u32x4v* s = src >= 0 ? reinterpret_cast<const u32x4v*>(p.base) + (size_t)src * p.row16 : nullptr;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < p.row16; e += stride)
        d[e] = s ? s[e] : u32x4v{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_pool_rows(PoolRowsParams p, int32_t n, hipStream_t stream) {
    const size_t per_row = (p.row16 + 255) / 256;
    const unsigned gx = (unsigned)(per_row < 512 ? per_row : 512);
    for (int32_t i0 = 0; i0 < n; i0 += 65535) {
        p.i0 = i0;
        const unsigned gy = (unsigned)(n - i0 < 65535 ? n - i0 : 65535);
        hipLaunchKernelGGL(pool_rows_kernel, dim3(gx, gy), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace gdn
