// mx_prep.hip -- the MXFP4 repack (canonical codes and block scales -> blob)
// and the per-row MX quantisation of activations to E4M3 with E8M0 block
// scales.
//
// Repack: page "量化开销对比" (laojiahuo2003.github.io), section 6.4 -- the
// weights and their scales are reordered once, offline, into the order the
// matrix instruction consumes them.  Quantisation: same page, section 3 (an
// E8M0 scale per block of 32) and section 4 (the scale taken at run time).
#include <hip/hip_runtime.h>

#include "mx_internal.h"

namespace mxfp4 {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void mx_repack_words(const uint32_t* __restrict__ qweight, uint32_t* __restrict__ out,
                                int64_t N, int64_t KS, int64_t nwords) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nwords) return;
    const int u = (int)(idx & 3);
    const int lane = (int)((idx >> 2) & 63);
    const int64_t chunk = idx >> 8;
    const int64_t s = chunk % KS;
    const int64_t t = chunk / KS;
    const int64_t col = t * kTileCols + (lane & 31);
    const int64_t row = 8 * s + 4 * (lane >> 5) + u;
    out[idx] = qweight[row * N + col];
}

// A scale of 0xFF (the E8M0 NaN) is flagged in the trailer, which is written
// before this kernel runs.
__global__ void mx_repack_scales(const uint8_t* __restrict__ ws, uint8_t* __restrict__ out,
                                 int64_t N, int64_t KQ, int64_t nbytes, uint32_t* __restrict__ trailer) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nbytes) return;
    const int u = (int)(idx & 3);
    const int lane = (int)((idx >> 2) & 63);
    const int64_t quad = idx >> 8;
    const int64_t q = quad % KQ;
    const int64_t t = quad / KQ;
    const int64_t block = 2 * (4 * q + u) + (lane >> 5);
    const uint8_t v = ws[block * N + t * kTileCols + (lane & 31)];
    out[idx] = v;
    if (v == 0xFFu) atomicOr(trailer + 2, kTrailerFlagNanScale);
}

__global__ void mx_init_trailer(uint32_t* __restrict__ trailer) {
    trailer[0] = kTrailerMagic;
    trailer[1] = MXFP4_LAYOUT_VERSION;
    trailer[2] = 0u;
    trailer[3] = 32u;
}

// The E4M3 code nearest to v (finite), ties to the even code, magnitudes of
// 448 and above saturating to 448 (0x7E).  Scaling by powers of two is exact,
// so each case is one round-half-even to an integer: the subnormal range in
// steps of 2^-9 (its top, 8 steps, is the smallest normal, code 0x08), a
// normal binade 2^e in steps of 2^(e-3).
__device__ __forceinline__ uint32_t to_e4m3(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {
        code = (uint32_t)rintf(a * 512.0f);
    } else {
        const int e = (int)((__float_as_uint(a) >> 23) & 255u) - 127;   // -6 .. 8
        code = (uint32_t)(8 * (e + 6)) + (uint32_t)rintf(ldexpf(a, 3 - e));
        code = min(code, 0x7Eu);
    }
    return sign | code;
}

template <bool BF16>
__device__ __forceinline__ float x_at(const u32x4& v, int i) {
    const uint32_t w = v[i >> 1];
    const uint32_t h = (i & 1) ? (w >> 16) : (w & 0xFFFFu);
    if (BF16) return __uint_as_float(h << 16);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

constexpr int kQuantThreads = 256;

// Thread t of a workgroup converts 8 elements (16 bytes of X); 4 threads make
// a block of 32 and share its largest magnitude through lane shuffles.
template <bool BF16>
__global__ __launch_bounds__(kQuantThreads) void mx_quantize_rows(
    const uint16_t* __restrict__ X, uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
    int64_t M, int64_t K) {
    const int64_t piece = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;   // 8 elements
    const bool live = piece < K / 8;
    for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (live) v = __builtin_nontemporal_load((const u32x4*)(X + row * K) + piece);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x_at<BF16>(v, i)));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
        const int ef = (int)((__float_as_uint(amax) >> 23) & 255u);
        const int E = ef == 0 ? -127 : max(ef - 127 - 8, -127);   // floor(log2 amax) - 8
        if (!live) continue;
        if ((threadIdx.x & 3) == 0) xs[row * (K / 32) + piece / 4] = (uint8_t)(E + 127);
        uint32_t out[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            out[i >> 2] |= to_e4m3(ldexpf(x_at<BF16>(v, i), -E)) << (8 * (i & 3));
        ((uint2*)(xq + row * K))[piece] = make_uint2(out[0], out[1]);
    }
}

int blocks_for(int64_t n, int threads) { return (int)((n + threads - 1) / threads); }

}  // namespace

hipError_t launch_mx_repack(const uint32_t* qweight, const uint8_t* ws, const LayoutMX& L,
                            void* packed, hipStream_t stream) {
    uint8_t* base = (uint8_t*)packed;
    const int64_t nwords = (int64_t)(L.w_bytes / 4);
    mx_repack_words<<<blocks_for(nwords, 256), 256, 0, stream>>>(qweight, (uint32_t*)base, L.N,
                                                                 L.KS, nwords);
    uint32_t* trailer = (uint32_t*)(base + L.t_off);
    mx_init_trailer<<<1, 1, 0, stream>>>(trailer);
    const int64_t nsc = (int64_t)L.s_bytes;
    mx_repack_scales<<<blocks_for(nsc, 256), 256, 0, stream>>>(ws, base + L.s_off, L.N, L.KQ, nsc,
                                                               trailer);
    return hipGetLastError();
}

hipError_t launch_mx_quantize_rows(const void* X, bool bf16, uint8_t* xq, uint8_t* xs, int64_t M,
                                   int64_t K, hipStream_t stream) {
    const dim3 grid((unsigned)blocks_for(K / 8, kQuantThreads), (unsigned)(M < 65535 ? M : 65535));
    if (bf16)
        mx_quantize_rows<true><<<grid, kQuantThreads, 0, stream>>>((const uint16_t*)X, xq, xs, M,
                                                                   K);
    else
        mx_quantize_rows<false><<<grid, kQuantThreads, 0, stream>>>((const uint16_t*)X, xq, xs, M,
                                                                    K);
    return hipGetLastError();
}

}  // namespace mxfp4
