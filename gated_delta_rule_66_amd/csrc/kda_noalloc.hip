// kda_chunk_fwd_noalloc: the prefill for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Its workspace (the segment transitions, local states
// and a redirected final state) lives in `scratch`, a device array of fixed
// size that every GPU the library runs on holds until the process ends.
//
// `scratch` is a device symbol: in host code its name stands for a host-side
// shadow, not a device address.  Its address on a device is taken once per
// device with hipGetSymbolAddress, with that device current, on the first
// call there, and only that address is handed to the kernels.
#include "kda.h"
#include "kda_internal.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace kda {

constexpr size_t kNoallocScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
static_assert(kNoallocScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the device address of `scratch` on the current device
kda_status device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace
}  // namespace kda

extern "C" kda_status kda_chunk_fwd_noalloc(int B, int T, int H, int K, int V, kda_dtype dt,
                                           const void* q, const void* k, const void* v,
                                           const void* g, const void* beta,
                                           const float* initial_state,
                                           void* o, float* final_state,
                                           const kda_plan* plan,
                                           hipStream_t stream) {
    using namespace kda;
    // every host check and the plan choice first: errors return before the
    // scratch address is taken
    kda_status s = chunk_fwd_bounded(B, T, H, K, V, dt, q, k, v, g, beta, initial_state, o, final_state, plan,
                                     nullptr, kNoallocScratchBytes, false, stream);
    if (s != KDA_OK) return s;
    void* ws = nullptr;
    // nothing to evaluate (at most a state copy): no workspace
    if ((long)B * H > 0 && T > 0) {
        s = device_scratch(&ws);
        if (s != KDA_OK) return s;
    }
    return chunk_fwd_bounded(B, T, H, K, V, dt, q, k, v, g, beta, initial_state, o, final_state, plan, ws,
                             ws ? kNoallocScratchBytes : 0, true, stream);
}
