// gdn_chunk_fwd without a workspace argument, for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The workspace is a file-scope device array of
// GDN_SCRATCH_BYTES, one copy per GPU, held from the first use of this code
// object on that GPU until the process ends.
//
// In host code `scratch` names a host-side shadow, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_params.h"

namespace {

static __device__ __align__(256) char scratch[GDN_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up
hipError_t g_scratch_err[kMaxDevices];  // the lookup's error on that device (hipSuccess: none yet)

// Device address of this device's copy of the array, or null with *err set
// (no device, or the lookup failed; a failed lookup is not retried).  No
// allocation: the array was placed when the code object was loaded.
void* scratch_for_current_device(hipError_t* err) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = e != hipSuccess ? e : hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev] && g_scratch_err[dev] == hipSuccess) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e == hipSuccess && ptr)
            g_scratch_ptr[dev] = ptr;
        else
            g_scratch_err[dev] = e != hipSuccess ? e : hipErrorInvalidSymbol;
    }
    *err = g_scratch_err[dev];
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int gdn_chunk_fwd_scratch(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                     const int32_t* cu_seqlens_host, int32_t num_seqs, const float* initial_state,
                                     void* out, float* final_state, int32_t T, int32_t H_q, int32_t H_v, int32_t d_k,
                                     int32_t d_v, float scale, gdn_dtype dtype, hipStream_t stream) {
    // Batch description first (host only): an invalid batch or one whose
    // intermediates exceed the array is refused before any HIP call.
    gdn_workspace_layout L;
    const int rc = gdn_chunk_fwd_workspace_layout(T, num_seqs, cu_seqlens_host, H_q, H_v, d_k, d_v, dtype, &L);
    if (rc != GDN_OK) return rc;
    if (L.total_bytes > (size_t)GDN_SCRATCH_BYTES) return GDN_EWORKSPACE;
    if (num_seqs == 0) return GDN_OK;
    hipError_t err = hipSuccess;
    void* ws = scratch_for_current_device(&err);
    if (!ws) return gdn::hip_fail(err != hipSuccess ? err : hipErrorInvalidSymbol);
    // Every region the pipeline reads is written earlier in the same call, so
    // nothing left by a previous call needs clearing.
    return gdn_chunk_fwd(q, k, v, g, beta, cu_seqlens_host, num_seqs, initial_state, out, final_state, T, H_q, H_v,
                         d_k, d_v, scale, dtype, ws, (size_t)GDN_SCRATCH_BYTES, stream);
}
