// The consumer side of the readiness words: a one-wave kernel that waits on a
// device word, so that work enqueued after it on the same stream starts only
// once a producer running on another stream has published its stores.  On the
// pages ("Fused QKV Projection + Norm + RoPE + Head Exchange" on
// docs.flashinfer.ai/api/comm.html) a single small workgroup, launched on a
// separate stream, does this acquire, and the caller's stream then waits for
// that stream; this kernel is the one-GPU version of it.  The wait is bounded:
// after spin_limit polls it gives up, counts a timeout and returns, so the
// kernel always exits.
#include "qkvx_internal.h"

namespace qkvx {
namespace {

__global__ __launch_bounds__(64) void wait_word_kernel(const unsigned long long* word,
                                                       unsigned long long expected,
                                                       int spin_limit, int* timeouts) {
    if (threadIdx.x != 0) return;
    for (int n = 0;; ++n) {
        const unsigned long long v =
            __hip_atomic_load(word, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        if (v >= expected) return;
        if (n >= spin_limit) {
            __hip_atomic_fetch_add(timeouts, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        __builtin_amdgcn_s_sleep(8);
    }
}

}  // namespace

hipError_t launch_wait_word(const unsigned long long* word, unsigned long long expected,
                            int spin_limit, int* timeouts, hipStream_t stream) {
    hipLaunchKernelGGL(wait_word_kernel, dim3(1), dim3(64), 0, stream, word, expected,
                       spin_limit, timeouts);
    return hipGetLastError();
}

}  // namespace qkvx
