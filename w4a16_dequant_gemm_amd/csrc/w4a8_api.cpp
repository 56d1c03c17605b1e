// w4a8_api.cpp -- the extern "C" entry points declared in include/w4a8.h:
// host-side validation (always before any HIP call), the kernel plan and the
// launches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/w4a8.h"
#include "w4a8_internal.h"

namespace w4a8 {

namespace {

constexpr int kDefaultCUs = 256;
constexpr int kMaxDevices = 64;
constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr uint32_t kPlanBits = W4A8_PLAN_MASK | (0xFFu << W4A16_PLAN_PARAM_SHIFT);

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

w4a16_status_t from_hip(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP; }

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

// K, N, G checks shared by every entry point.
w4a16_status_t check_kng(int64_t K, int64_t N, int group_size) {
    if (K < 1 || N < 1 || K >= kMaxDim || N >= kMaxDim) return W4A16_ERR_INVALID_ARG;
    if (group_size < 1 || K % group_size != 0) return W4A16_ERR_INVALID_ARG;
    if ((double)K * (double)N >= (double)((int64_t)1 << 40)) return W4A16_ERR_INVALID_ARG;
    if (group_size != 32 && group_size != 64 && group_size != 128) return W4A16_ERR_UNSUPPORTED;
    if (K % kKAlign != 0 || K > kMaxK || N % kNAlign != 0) return W4A16_ERR_UNSUPPORTED;
    return W4A16_OK;
}

}  // namespace

PlanW8 make_plan_w8(int64_t M, int64_t N, int64_t K, uint32_t flags, int cus) {
    PlanW8 p{};
    const uint32_t hint = flags & W4A8_PLAN_MASK;
    const int param = (int)((flags >> W4A16_PLAN_PARAM_SHIFT) & 0xFFu);
    const int64_t NT = N / kTileCols;
    const int64_t KC = K / kChunkK;
    const bool stream_ok = M <= kStreamMaxRows;
    const bool stream = hint == W4A8_PLAN_TILED    ? false
                        : hint == W4A8_PLAN_STREAM ? stream_ok
                                                   : M <= kStreamDefaultRows;
    if (stream) {
        p.variant = W8_STREAM;
        p.rt = M <= 32 ? 1 : 2;
        if ((param == 2 || param == 4 || param == 8) && KC >= param) {
            p.kp = param;
        } else {
            // M <= 8: the most parts whose workgroups are all resident at
            // two per CU.  Measured (us per call, same box): 8192 x 28672
            // (896 tiles) M = 1 28.3 with 4 parts (448 workgroups) vs 29.1-30.6
            // with 8, M = 4 29.6 vs 31.4; 8192 x 8192 (256 tiles) 11.5 with 8
            // vs 17.6 with 4.  M > 8: 4 parts (measured fastest on the
            // 8192 x 28672 layer), more while fewer than 3/4 of the CUs would
            // get a workgroup (8192 x 8192: M = 16 13.8 with 8 vs 20.3 with
            // 4, M = 32 18.9 vs 27.6).
            p.kp = 2;
            if (M > 8) {
                p.kp = KC >= 4 ? 4 : 2;
                while (p.kp < 8 && NT * p.kp / kW8Waves < (int64_t)cus * 3 / 4 && KC >= 2 * p.kp)
                    p.kp *= 2;
            } else {
                for (int kp = 8; kp >= 2; kp /= 2)
                    if (NT * kp / kW8Waves <= 2 * (int64_t)cus && KC >= kp) {
                        p.kp = kp;
                        break;
                    }
            }
        }
        // block-diagonal 16x16x64 form, measured on the 8192 x 28672 layer
        // (us per call, same box): M = 1 30.7 vs 34.1, M = 4 33.4 vs 36.4, but
        // M = 8 38.4 vs 37.0
        p.bd = M <= 4;
        const int ctw = kW8Waves / p.kp;
        p.grid = (int)(NT / ctw);
        p.lds = (size_t)(p.kp - 1) * ctw * p.rt * (p.bd ? 4 : 16) * 64 * 4;
    } else {
        p.variant = W8_TILED;
        // tile shapes: 0 = 256 x 256 (4 x 2 tiles per wave), 1 = 128 x 128 (2 x 1),
        // 2 = 256 x 128 (4 x 1), 3 = 256 x 256 with two chunks per LDS stage,
        // 4 = 3 with the int8 weights made once per workgroup in LDS (measured
        // 4-7% slower than 3, not chosen by default); W4A16_PLAN_PARAM(1 + shape)
        // forces one
        // (measured on the 8192 x 28672 layer: 128 x 128 is fastest up to M = 128,
        // 256 x 128 up to 512, 256 x 256 beyond)
        // (256 x 256 with two chunks per LDS stage: half the barriers, 3-11%
        // faster than one chunk per stage at M = 1024..4096)
        p.cfg = (hint == W4A8_PLAN_TILED && param >= 1 && param <= 5) ? param - 1
                : M <= 128                                            ? 1
                : M <= 512                                            ? 2
                                                                      : 3;
        const int64_t bm = p.cfg == 1 ? 128 : 256;
        const int64_t bn = (p.cfg == 0 || p.cfg == 3 || p.cfg == 4) ? 256 : 128;
        p.rt = p.cfg == 1 ? 2 : 4;
        p.nbm = (int)((M + bm - 1) / bm);
        p.nbn = (int)((N + bn - 1) / bn);
        p.grid = p.nbm * p.nbn;
        // two LDS slots of bm rows: 64 bytes of X per chunk (+16), or two chunks (cfg 3)
        p.lds = (size_t)2 * bm * (p.cfg >= 3 ? 2 * kChunkK + 16 : kTiledRowBytes);
        if (p.cfg == 4) p.lds += (size_t)2 * (bn / kTileCols) * 2 * 2 * 1024;   // B operands
    }
    return p;
}

}  // namespace w4a8

using namespace w4a8;

extern "C" {

size_t w4a8_packed_bytes(int64_t K, int64_t N, int group_size) {
    if (check_kng(K, N, group_size) != W4A16_OK) return 0;
    return make_layout_w8(K, N, group_size).total;
}

w4a16_status_t w4a8_repack(const uint32_t* qweight, const uint8_t* s8, const uint8_t* a,
                           const float* sw, int64_t K, int64_t N, int group_size, void* packed,
                           size_t packed_bytes, void* stream) {
    const w4a16_status_t st = check_kng(K, N, group_size);
    if (st != W4A16_OK) return st;
    if (!qweight || !s8 || !a || !sw || !packed) return W4A16_ERR_INVALID_ARG;
    if (!aligned16(qweight) || !aligned16(s8) || !aligned16(a) || !aligned16(sw) ||
        !aligned16(packed))
        return W4A16_ERR_INVALID_ARG;
    const LayoutW8 L = make_layout_w8(K, N, group_size);
    if (packed_bytes < L.total) return W4A16_ERR_INVALID_ARG;
    return from_hip(launch_w8_repack(qweight, s8, a, sw, L, packed, (hipStream_t)stream));
}

w4a16_status_t w4a8_dequant(const void* packed, size_t packed_bytes, int8_t* W_out, int64_t K,
                            int64_t N, int group_size, void* stream) {
    const w4a16_status_t st = check_kng(K, N, group_size);
    if (st != W4A16_OK) return st;
    if (!packed || !W_out || !aligned16(packed) || !aligned16(W_out)) return W4A16_ERR_INVALID_ARG;
    const LayoutW8 L = make_layout_w8(K, N, group_size);
    if (packed_bytes < L.total) return W4A16_ERR_INVALID_ARG;
    return from_hip(launch_w8_dequant(packed, L, W_out, (hipStream_t)stream));
}

w4a16_status_t w4a8_quantize_rows(const void* X, int8_t* xq, float* sx, int64_t M, int64_t K,
                                  uint32_t flags, void* stream) {
    if (flags & ~W4A8_X_BF16) return W4A16_ERR_INVALID_ARG;
    if (M < 1 || M >= kMaxDim || K < 1 || K >= kMaxDim) return W4A16_ERR_INVALID_ARG;
    if (K % kKAlign != 0 || K > kMaxK) return W4A16_ERR_UNSUPPORTED;
    if (!X || !xq || !sx || !aligned16(X) || !aligned16(xq) || !aligned16(sx))
        return W4A16_ERR_INVALID_ARG;
    return from_hip(launch_w8_quantize_rows(X, (flags & W4A8_X_BF16) != 0, xq, sx, M, K,
                                            (hipStream_t)stream));
}

w4a16_status_t w4a8_gemm(const int8_t* xq, const float* sx, const void* packed,
                         size_t packed_bytes, void* Y, int64_t M, int64_t N, int64_t K,
                         int group_size, uint32_t flags, void* stream) {
    if (flags & ~(W4A8_OUT_MASK | kPlanBits)) return W4A16_ERR_INVALID_ARG;
    const uint32_t out = flags & W4A8_OUT_MASK;
    if (out == 3u) return W4A16_ERR_INVALID_ARG;
    if (M < 1 || M >= kMaxDim) return W4A16_ERR_INVALID_ARG;
    const w4a16_status_t st = check_kng(K, N, group_size);
    if (st != W4A16_OK) return st;
    if (!xq || !packed || !Y || !aligned16(xq) || !aligned16(packed) || !aligned16(Y))
        return W4A16_ERR_INVALID_ARG;
    if (out != W4A8_OUT_I32 && (!sx || !aligned16(sx))) return W4A16_ERR_INVALID_ARG;
    if (sx && !aligned16(sx)) return W4A16_ERR_INVALID_ARG;
    const LayoutW8 L = make_layout_w8(K, N, group_size);
    if (packed_bytes < L.total) return W4A16_ERR_INVALID_ARG;
    const PlanW8 plan = make_plan_w8(M, N, K, flags, num_cus());
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (out == W4A8_OUT_FP16)
        e = launch_w8_gemm_f16(xq, sx, packed, Y, M, L, plan, s);
    else if (out == W4A8_OUT_BF16)
        e = launch_w8_gemm_bf16(xq, sx, packed, Y, M, L, plan, s);
    else
        e = launch_w8_gemm_i32(xq, sx, packed, Y, M, L, plan, s);
    return from_hip(e);
}

}  // extern "C"
