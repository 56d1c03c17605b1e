// mx_api.cpp -- the extern "C" entry points declared in include/mxfp4.h:
// host-side validation (always before any HIP call), the kernel plan and the
// launches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/mxfp4.h"
#include "mx_internal.h"

namespace mxfp4 {

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr uint32_t kPlanBits = MXFP4_PLAN_MASK | (0xFFu << W4A16_PLAN_PARAM_SHIFT);

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

w4a16_status_t from_hip(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP; }

constexpr int kDefaultCUs = 256;
constexpr int kMaxDevices = 64;

// Compute units of the current device, read once per device.
int num_cus() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCUs;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = kDefaultCUs;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

w4a16_status_t check_kn(int64_t K, int64_t N) {
    if (K < 1 || N < 1 || K >= kMaxDim || N >= kMaxDim) return W4A16_ERR_INVALID_ARG;
    if ((double)K * (double)N >= (double)((int64_t)1 << 40)) return W4A16_ERR_INVALID_ARG;
    if (K % kKAlign != 0 || N % kNAlign != 0) return W4A16_ERR_UNSUPPORTED;
    return W4A16_OK;
}

}  // namespace

PlanMX make_plan_mx(int64_t M, int64_t N, int64_t K, uint32_t flags, int cus) {
    PlanMX p{};
    const uint32_t hint = flags & MXFP4_PLAN_MASK;
    const int param = (int)((flags >> W4A16_PLAN_PARAM_SHIFT) & 0xFFu);
    const int64_t NT = N / kTileCols;
    const int64_t KS = K / kStepK;
    const bool stream = hint == MXFP4_PLAN_TILED    ? false
                        : hint == MXFP4_PLAN_STREAM ? M <= kMxStreamMaxRows
                                                    : M <= kMxStreamDefaultRows;
    if (stream) {
        p.variant = MX_STREAM;
        p.rt = M <= 32 ? 1 : 2;
        // parts of K per tile.  M <= 8: the most parts whose workgroups are
        // all resident at two per CU (measured, us per call: 8192 x 28672,
        // 896 tiles, 4 parts 28.7 vs 29.2 with 8; 8192 x 8192, 256 tiles, 8
        // parts 11.2 vs 17.1 with 4; 28672 x 8192 31.4 vs 53.4).  M > 8: 2
        // parts (36.8 us at M = 16 on 8192 x 28672 against 39.6 with 4),
        // more while fewer than 3/4 of the CUs would get a workgroup (8192 x
        // 8192: M = 16 13.0 with 8 vs 34.8 with 2, M = 32 18.8 vs 47.2).
        int kp = 2;
        if (M <= 8) {
            for (int c = 8; c >= 2; c /= 2)
                if (NT * c / kMxWaves <= 2 * (int64_t)cus && KS >= c) {
                    kp = c;
                    break;
                }
        } else {
            while (kp < 8 && NT * kp / kMxWaves < (int64_t)cus * 3 / 4 && KS >= 2 * kp) kp *= 2;
        }
        p.kp = (param == 2 || param == 4 || param == 8) && KS >= param ? param : kp;
        // block-diagonal 16x16x128 form, measured on the 8192 x 28672 layer
        // (us per call, same box): M = 1 28.9 vs 30.1, M = 2 28.8 vs 30.0,
        // M = 4 30.5 vs 30.8, but M = 8 34.6 vs 31.5
        p.bd = M <= 4 && M * K <= kMxBlockDiagMaxXBytes;
        const int ctw = kMxWaves / p.kp;
        p.grid = (int)(NT / ctw);
        p.lds = (size_t)(p.kp - 1) * ctw * p.rt * 16 * 64 * 4;   // enough for either form
    } else {
        p.variant = MX_TILED;
        p.cfg = (hint == MXFP4_PLAN_TILED && param >= 1 && param <= 4) ? param - 1
                : M <= 128                                              ? 1
                : M <= 512                                              ? 2
                                                                        : 3;
        const int64_t bm = p.cfg == 1 ? 128 : 256;
        const int64_t bn = (p.cfg == 0 || p.cfg == 3) ? 256 : 128;
        p.rt = p.cfg == 1 ? 2 : 4;
        p.nbm = (int)((M + bm - 1) / bm);
        p.nbn = (int)((N + bn - 1) / bn);
        p.grid = p.nbm * p.nbn;
        p.lds = (size_t)2 * bm * (p.cfg == 3 ? 2 * kStepK + 16 : kMxRowBytes);
    }
    return p;
}

}  // namespace mxfp4

using namespace mxfp4;

extern "C" {

size_t mxfp4_packed_bytes(int64_t K, int64_t N) {
    if (check_kn(K, N) != W4A16_OK) return 0;
    return make_layout_mx(K, N).total;
}

w4a16_status_t mxfp4_repack(const uint32_t* qweight, const uint8_t* ws, int64_t K, int64_t N,
                            void* packed, size_t packed_bytes, void* stream) {
    const w4a16_status_t st = check_kn(K, N);
    if (st != W4A16_OK) return st;
    if (!qweight || !ws || !packed || !aligned16(qweight) || !aligned16(ws) || !aligned16(packed))
        return W4A16_ERR_INVALID_ARG;
    const LayoutMX L = make_layout_mx(K, N);
    if (packed_bytes < L.total) return W4A16_ERR_INVALID_ARG;
    return from_hip(launch_mx_repack(qweight, ws, L, packed, (hipStream_t)stream));
}

w4a16_status_t mxfp4_quantize_rows(const void* X, uint8_t* xq, uint8_t* xs, int64_t M, int64_t K,
                                   uint32_t flags, void* stream) {
    if (flags & ~MXFP4_BF16) return W4A16_ERR_INVALID_ARG;
    if (M < 1 || M >= kMaxDim || K < 1 || K >= kMaxDim) return W4A16_ERR_INVALID_ARG;
    if (K % kKAlign != 0) return W4A16_ERR_UNSUPPORTED;
    if (!X || !xq || !xs || !aligned16(X) || !aligned16(xq) || !aligned16(xs))
        return W4A16_ERR_INVALID_ARG;
    return from_hip(launch_mx_quantize_rows(X, (flags & MXFP4_BF16) != 0, xq, xs, M, K,
                                            (hipStream_t)stream));
}

w4a16_status_t mxfp4_gemm(const uint8_t* xq, const uint8_t* xs, const void* packed,
                          size_t packed_bytes, void* Y, int64_t M, int64_t N, int64_t K,
                          uint32_t flags, void* stream) {
    if (flags & ~(MXFP4_BF16 | kPlanBits)) return W4A16_ERR_INVALID_ARG;
    if (M < 1 || M >= kMaxDim) return W4A16_ERR_INVALID_ARG;
    const w4a16_status_t st = check_kn(K, N);
    if (st != W4A16_OK) return st;
    if (!xq || !xs || !packed || !Y || !aligned16(xq) || !aligned16(xs) || !aligned16(packed) ||
        !aligned16(Y))
        return W4A16_ERR_INVALID_ARG;
    const LayoutMX L = make_layout_mx(K, N);
    if (packed_bytes < L.total) return W4A16_ERR_INVALID_ARG;
    const PlanMX plan = make_plan_mx(M, N, K, flags, num_cus());
    hipStream_t s = (hipStream_t)stream;
    const hipError_t e = (flags & MXFP4_BF16) ? launch_mx_gemm_bf16(xq, xs, packed, Y, M, L, plan, s)
                                              : launch_mx_gemm_f16(xq, xs, packed, Y, M, L, plan, s);
    return from_hip(e);
}

}  // extern "C"
