// hg_noalloc.hip — hgemm_splitk for callers that cannot allocate device
// memory or pass a workspace (code under stream capture, tight serving
// loops, harnesses that forbid allocation): the fp32 partial products live in
// one static device array of this library instead of a caller's workspace.
#include "hgemm.h"

#include <atomic>

#include <hip/hip_runtime.h>

namespace {

// The partials of one call: at most HG_NOALLOC_SCRATCH_BYTES, one array per
// GPU the library runs on, held until the process ends.
__device__ __align__(256) unsigned char scratch[HG_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on each device (the host-side name is a
// stand-in and must never reach a kernel), looked up once per device.
std::atomic<void *> g_scratch[64];

// The current device's address of `scratch`; nullptr with *err set when the
// lookup fails.
void *scratch_ptr(hipError_t *err)
{
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess)
        return nullptr;
    if (dev < 0 || dev >= 64) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || p == nullptr) {
            if (*err == hipSuccess)
                *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" int hgemm_splitk_noalloc(int64_t M, int64_t N, int64_t K, float alpha, const void *A,
                                    int64_t lda, const void *B, int64_t ldb, float beta, void *C,
                                    int64_t ldc, int out_dtype, int splits, void *stream)
{
    hipError_t e = hipSuccess;
    void *ws = scratch_ptr(&e);
    if (ws == nullptr)
        return HG_ERR_HIP_BASE + (int)e;
    // hgemm_splitk validates every argument in order; the only difference is
    // where its partials go.  A problem whose partials exceed the array is
    // reported as such instead of as a short workspace.
    const int st = hgemm_splitk(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, out_dtype, splits, ws,
                                (int64_t)HG_NOALLOC_SCRATCH_BYTES, stream);
    return st == -15 ? HG_ERR_SCRATCH_LIMIT : st;
}
