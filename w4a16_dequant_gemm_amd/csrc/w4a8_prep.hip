// w4a8_prep.hip -- the W4A8 repack (canonical tensors -> blob), the
// materialising dequant used for bit-exact checks, and the dynamic per-row
// int8 quantisation of activations.
//
// Repack: page "量化开销对比" (laojiahuo2003.github.io), section 6.4 -- the
// weights and their group constants are reordered once, offline, into the
// order the kernels consume.  Quantisation: same page, section 4 (per-token
// scale from the row's largest magnitude, taken at run time).  These kernels
// favour simple indexing over speed, except the row quantisation, which runs
// per token and reads X once per pass with 16-byte loads.
#include <hip/hip_runtime.h>

#include "w4a8_device.h"
#include "w4a8_internal.h"

namespace w4a8 {

namespace {

// Canonical word (code i at nibble i) -> repacked word (code i at nibble 2i
// for i < 4, 2(i-4)+1 for i >= 4).
__device__ __forceinline__ uint32_t to_repacked(uint32_t w) {
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int pos = i < 4 ? 2 * i : 2 * (i - 4) + 1;
        out |= ((w >> (4 * i)) & 0xFu) << (4 * pos);
    }
    return out;
}

// Word idx of region W -> its column and the first of its eight k.
struct WordAt {
    int64_t col, k0, t;
    int lane;
};

__device__ __forceinline__ WordAt word_at(int64_t idx, int64_t KC) {
    const int j = (int)(idx & 3);
    const int lane = (int)((idx >> 2) & 63);
    const int64_t chunk = idx >> 8;
    const int64_t c = chunk % KC;
    WordAt p;
    p.t = chunk / KC;
    p.lane = lane;
    p.col = p.t * kTileCols + (lane & 31);
    p.k0 = kChunkK * c + 32 * (j >> 1) + 16 * (lane >> 5) + 8 * (j & 1);
    return p;
}

__global__ void w8_repack_words(const uint32_t* __restrict__ qweight, uint32_t* __restrict__ out,
                                int64_t N, int64_t KC, int64_t nwords) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nwords) return;
    const WordAt p = word_at(idx, KC);
    out[idx] = to_repacked(qweight[(p.k0 / 8) * N + p.col]);
}

__global__ void w8_init_trailer(uint32_t* __restrict__ trailer, uint32_t group_size) {
    trailer[0] = kTrailerMagic;
    trailer[1] = kLayoutVersion;
    trailer[2] = 0u;
    trailer[3] = group_size;
}

__global__ void w8_repack_meta(const uint8_t* __restrict__ s8, const uint8_t* __restrict__ a,
                               const float* __restrict__ sw, uint16_t* __restrict__ meta,
                               float* __restrict__ colscale, uint32_t* __restrict__ trailer,
                               int64_t N, int64_t NG) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= NG * N) return;
    const int64_t g = idx / N;
    const int64_t n = idx % N;
    const uint32_t s = s8[idx];
    const uint32_t o = a[idx];
    meta[((n / kTileCols) * NG + g) * kTileCols + (n % kTileCols)] = (uint16_t)(s | (o << 8));
    if (s > 16u || o + 15u * s > 255u) atomicOr(&trailer[2], kW8FlagOverflow);
    if (g == 0) colscale[n] = sw[n];
}

__global__ void w8_dequant_words(const uint32_t* __restrict__ words,
                                 const uint16_t* __restrict__ meta, int8_t* __restrict__ W,
                                 int64_t N, int64_t KC, int64_t NG, int64_t G, int64_t nwords) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nwords) return;
    const WordAt p = word_at(idx, KC);
    const int64_t g = p.k0 / G;
    const GroupW8 gp = group_w8(meta[(p.t * NG + g) * kTileCols + (p.lane & 31)]);
    uint32_t lo, hi;
    word_to_i8(words[idx], gp, lo, hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        W[(p.k0 + i) * N + p.col] = (int8_t)((lo >> (8 * i)) & 0xFFu);
        W[(p.k0 + 4 + i) * N + p.col] = (int8_t)((hi >> (8 * i)) & 0xFFu);
    }
}

constexpr int kQuantThreads = 256;

template <bool BF16>
__device__ __forceinline__ float x_at(const u32x4& v, int i) {
    const uint32_t w = v[i >> 1];
    const uint32_t h = (i & 1) ? (w >> 16) : (w & 0xFFFFu);
    if (BF16) return __uint_as_float(h << 16);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// One workgroup per row: the row's largest magnitude, then every element
// divided by sx = amax / 127 and rounded half to even, both in fp32 with IEEE
// division.
template <bool BF16>
__global__ __launch_bounds__(kQuantThreads) void w8_quantize_rows(
    const uint16_t* __restrict__ X, int8_t* __restrict__ xq, float* __restrict__ sx, int64_t K) {
    __shared__ float part[kQuantThreads / 64];
    const int64_t row = blockIdx.x;
    const u32x4* src = (const u32x4*)(X + row * K);
    const int64_t pieces = K / 8;
    float amax = 0.0f;
    for (int64_t p = threadIdx.x; p < pieces; p += kQuantThreads) {
        const u32x4 v = __builtin_nontemporal_load(src + p);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x_at<BF16>(v, i)));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = part[0];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, part[w]);
    const float s = __fdiv_rn(amax, 127.0f);
    if (threadIdx.x == 0) sx[row] = s;
    uint2* dst = (uint2*)(xq + row * K);
    for (int64_t p = threadIdx.x; p < pieces; p += kQuantThreads) {
        const u32x4 v = __builtin_nontemporal_load(src + p);
        uint32_t out[2] = {0u, 0u};
        if (s > 0.0f) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float q = rintf(__fdiv_rn(x_at<BF16>(v, i), s));
                q = fminf(fmaxf(q, -127.0f), 127.0f);
                out[i >> 2] |= ((uint32_t)(int)q & 0xFFu) << (8 * (i & 3));
            }
        }
        dst[p] = make_uint2(out[0], out[1]);
    }
}

int blocks_for(int64_t n, int threads) { return (int)((n + threads - 1) / threads); }

}  // namespace

hipError_t launch_w8_repack(const uint32_t* qweight, const uint8_t* s8, const uint8_t* a,
                            const float* sw, const LayoutW8& L, void* packed, hipStream_t stream) {
    uint8_t* base = (uint8_t*)packed;
    const int64_t nwords = (int64_t)(L.w_bytes / 4);
    uint32_t* trailer = (uint32_t*)(base + L.t_off);
    w8_repack_words<<<blocks_for(nwords, 256), 256, 0, stream>>>(qweight, (uint32_t*)base, L.N,
                                                                 L.KC, nwords);
    w8_init_trailer<<<1, 1, 0, stream>>>(trailer, (uint32_t)L.G);
    const int64_t nmeta = L.NG * L.N;
    w8_repack_meta<<<blocks_for(nmeta, 256), 256, 0, stream>>>(
        s8, a, sw, (uint16_t*)(base + L.m_off), (float*)(base + L.c_off), trailer, L.N, L.NG);
    return hipGetLastError();
}

hipError_t launch_w8_dequant(const void* packed, const LayoutW8& L, int8_t* W_out,
                             hipStream_t stream) {
    const uint8_t* base = (const uint8_t*)packed;
    const int64_t nwords = (int64_t)(L.w_bytes / 4);
    w8_dequant_words<<<blocks_for(nwords, 256), 256, 0, stream>>>(
        (const uint32_t*)base, (const uint16_t*)(base + L.m_off), W_out, L.N, L.KC, L.NG, L.G,
        nwords);
    return hipGetLastError();
}

hipError_t launch_w8_quantize_rows(const void* X, bool bf16, int8_t* xq, float* sx, int64_t M,
                                   int64_t K, hipStream_t stream) {
    if (bf16)
        w8_quantize_rows<true><<<(unsigned)M, kQuantThreads, 0, stream>>>((const uint16_t*)X, xq,
                                                                           sx, K);
    else
        w8_quantize_rows<false><<<(unsigned)M, kQuantThreads, 0, stream>>>((const uint16_t*)X, xq,
                                                                            sx, K);
    return hipGetLastError();
}

}  // namespace w4a8
