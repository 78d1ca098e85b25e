// glu_dual_gemv_backward without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The backward needs scratch beyond its inputs and outputs: the bf16 gate and
// up gradients, the zero-padded operand copies of the matrix-core path and the
// fp32 partial sums of dhidden.  Here that scratch is one file-scope device
// array of kScratchBytes.  The code object holds it, so every GPU the library
// runs on keeps its own copy, at its own address, until the process ends.  In
// host code the array's name stands for a host-side shadow, not for device
// memory: the device address of the current GPU's copy is looked up once per
// device with hipGetSymbolAddress and only that address is passed on.  Every
// call on one GPU shares that GPU's copy and leaves the last call's contents
// in it; calls that overlap on one GPU (different streams, or a graph and an
// eager call in flight together) race on it.  No kernel needs any part of it
// cleared first: each launch writes every scratch element it later reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/glu_gemv.h"
#include "glu_backward.h"

namespace {

constexpr int64_t kScratchBytes = (int64_t)48 << 20;  // 48 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of each GPU's copy, once looked up

// The current device's copy of the scratch array (looked up on its first use on that device).
glu_status scratch_on_current_device(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return glu::launch_failed(e);
    if (dev < 0 || dev >= kMaxDevices) return glu::launch_failed(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return glu::launch_failed(e != hipSuccess ? e : hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GLU_OK;
}

}  // namespace

extern "C" {

glu_status glu_dual_gemv_backward_noalloc(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                                          const uint16_t* dout, uint16_t* dhidden, uint16_t* dgate_w,
                                          uint16_t* dup_w, int64_t M, int64_t N, int64_t K, void* stream)
{
    int64_t need = 0;
    glu_status st = glu::backward_workspace(M, N, K, &need);
    if (st != GLU_OK) return st;
    // every argument check of glu_dual_gemv_backward, before any HIP call
    st = glu::backward_entry(hidden, gate_w, up_w, dout, dhidden, dgate_w, dup_w, M, N, K, nullptr, 0, stream, true);
    if (st != GLU_OK) return st;
    if (need > kScratchBytes) return GLU_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_on_current_device(&ws);
        if (st != GLU_OK) return st;
    }
    return glu::backward_entry(hidden, gate_w, up_w, dout, dhidden, dgate_w, dup_w, M, N, K, ws, kScratchBytes,
                               stream, false);
}

}  // extern "C"
