// kda_chunk_fwd_noalloc: kda_chunk_fwd for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The workspace kda_chunk_fwd takes from
// its caller comes instead from a file-scope device array; the call
// allocates nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/kda.h"

// The packed-batch order, or the sequence-parallel path's transitions, local
// final states and incoming states: at most 3 x 256 states of 64 KiB, since
// that path never runs more than 256 segment chains.  Every GPU the library
// runs on holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

// Per-device address of `scratch` (its host-side name is only a stand-in,
// never a device address): looked up once per device, with that device
// current, on the device's first call.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, int in_dtype,
                                     const float* log_alpha, const float* beta, const float* S0,
                                     const int32_t* cu_seqlens, int32_t n_seqs, int64_t T,
                                     int32_t H, int32_t dk, int32_t dv, float* o, float* S_T,
                                     hipStream_t stream) {
    // The workspace kda_chunk_fwd would take (0 for invalid sizes, which
    // kda_chunk_fwd then reports).  It never exceeds the array, but a larger
    // size is refused rather than written past its end.
    const size_t need =
        kda_chunk_fwd_workspace_bytes(n_seqs, T, H, dk, dv, cu_seqlens != nullptr ? 1 : 0);
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_TOO_LARGE;
    void* ws = nullptr;
    if (need > 0 && scratch_address(&ws) != hipSuccess) return KDA_ERR_HIP;
    return kda_chunk_fwd(q, k, v, in_dtype, log_alpha, beta, S0, cu_seqlens, n_seqs, T, H, dk, dv, o,
                         S_T, ws, ws ? (size_t)KDA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
