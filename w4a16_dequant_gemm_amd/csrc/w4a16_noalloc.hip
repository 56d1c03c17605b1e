// w4a16_noalloc.hip -- w4a16_gemm_noalloc: the fused product for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  The kernels' scratch (cross-
// workgroup counters and fp32 partial tiles) lives in a file-scope device
// array of fixed size instead of a caller-supplied workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/w4a16.h"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr size_t kScratchBytes = W4A16_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes > kCounterBytes, "the scratch holds the counter area");
constexpr int kMaxDevices = 64;

// One copy per GPU the library runs on, held until the process ends.  In
// host code this name is only a stand-in for the symbol: its device address
// comes from hipGetSymbolAddress (below) and is the only form ever passed to
// a kernel or a copy.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Zero-fills the counter area: the kernels return every counter to zero at the
// end of each call, so this is needed once per device (device memory of a
// loaded code object starts zeroed as well; this does not rely on it).
__global__ __launch_bounds__(256) void clear_counters_kernel(uint4* p, int n16) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n16) p[i] = uint4{0u, 0u, 0u, 0u};
}

// The device address of this device's scratch array, looked up (and its
// counters cleared, on `stream`) on the first call on the device.
w4a16_status_t scratch_for_current_device(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W4A16_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W4A16_ERR_HIP;
        const int n16 = (int)(kCounterBytes / 16);
        hipLaunchKernelGGL(clear_counters_kernel, dim3((n16 + 255) / 256), dim3(256), 0, stream,
                           (uint4*)p, n16);
        if (hipGetLastError() != hipSuccess) return W4A16_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return W4A16_OK;
}

}  // namespace

}  // namespace w4a16

using namespace w4a16;

extern "C" w4a16_status_t w4a16_gemm_noalloc(const void* X, const void* packed,
                                             size_t packed_bytes, void* Y, int64_t M, int64_t N,
                                             int64_t K, int group_size, uint32_t flags,
                                             const w4a16_epilogue_t* epilogue, void* stream) {
    GemmCall c;
    const w4a16_status_t st =
        prepare_gemm(X, packed, packed_bytes, Y, M, N, K, group_size, flags, epilogue, &c);
    if (st != W4A16_OK) return st;
    if (c.plan.workspace > kScratchBytes) return W4A16_ERR_WORKSPACE;
    void* ws = nullptr;
    if (c.plan.workspace > 0) {
        const w4a16_status_t s2 = scratch_for_current_device((hipStream_t)stream, &ws);
        if (s2 != W4A16_OK) return s2;
    }
    return run_gemm(c, X, packed, Y, M, ws, (hipStream_t)stream);
}
