// w4a16_repack.hip -- offline repack of canonical tensors into the kernel
// order (layout version 1, see w4a16_layout.h), its exact inverse, and the
// materialising dequant used for bit-exact checks.
//
// Page "量化开销对比", section 6.4: weights, scales and zeros are reordered
// together, once, into the order the kernel reads them.  These kernels run
// outside the per-token path; they favour simple indexing over speed.
#include <hip/hip_runtime.h>

#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

// Nibble position p of a repacked word holds j = 2*(p%4) + p/4 of its eight
// consecutive reduction indices.
__device__ __forceinline__ uint32_t canonical_to_repacked(uint32_t w) {
    uint32_t out = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int j = 2 * (p & 3) + (p >> 2);
        out |= ((w >> (4 * j)) & 0xFu) << (4 * p);
    }
    return out;
}

__device__ __forceinline__ uint32_t repacked_to_canonical(uint32_t w) {
    uint32_t out = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int j = 2 * (p & 3) + (p >> 2);
        out |= ((w >> (4 * p)) & 0xFu) << (4 * j);
    }
    return out;
}

// Word index inside region W -> (column, canonical word row).
struct WordPos {
    int64_t col, row;   // canonical qweight[row][col]
};

__device__ __forceinline__ WordPos word_pos(int64_t idx, int64_t KS) {
    const int t = (int)(idx & 3);
    const int lane = (int)((idx >> 2) & 63);
    const int64_t chunk = idx >> 8;
    const int64_t ks = chunk % KS;
    const int64_t nb = chunk / KS;
    WordPos p;
    p.col = nb * kColBlock + 32 * t + (lane & 31);
    p.row = 2 * ks + (lane >> 5);
    return p;
}

__global__ void repack_words_kernel(const uint32_t* __restrict__ qweight,
                                    uint32_t* __restrict__ out, int64_t N, int64_t KS,
                                    int64_t nwords) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nwords) return;
    const WordPos p = word_pos(idx, KS);
    out[idx] = canonical_to_repacked(qweight[p.row * N + p.col]);
}

__global__ void unrepack_words_kernel(const uint32_t* __restrict__ in,
                                      uint32_t* __restrict__ qweight, int64_t N, int64_t KS,
                                      int64_t nwords) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nwords) return;
    const WordPos p = word_pos(idx, KS);
    qweight[p.row * N + p.col] = repacked_to_canonical(in[idx]);
}

__global__ void init_trailer_kernel(uint32_t* __restrict__ trailer, uint32_t group_size) {
    trailer[0] = kTrailerMagic;
    trailer[1] = 1u;   // layout version
    trailer[2] = 0u;   // feature flags, OR-ed by repack_meta_kernel
    trailer[3] = group_size;
}

// One thread per (nb, g, c32): four scales and four zeros.  For bf16 it also
// flags the blob when -z*s overflows fp32 for some column.
__global__ void repack_meta_kernel(const uint16_t* __restrict__ scales,
                                   const uint8_t* __restrict__ zeros, uint8_t* __restrict__ packed,
                                   int64_t N, int64_t NG, size_t s_off, size_t z_off,
                                   size_t t_off, int bf16, int64_t nrec32) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nrec32) return;
    const int c32 = (int)(idx & 31);
    const int64_t rec = idx >> 5;          // nb * NG + g
    const int64_t g = rec % NG;
    const int64_t nb = rec / NG;
    uint16_t* srec = (uint16_t*)(packed + s_off + rec * kScaleRecBytes) + 4 * c32;
    uint32_t zword = 0;
    bool needs_exact = false;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t col = nb * kColBlock + 32 * t + c32;
        const uint16_t sb = scales[g * N + col];
        const uint32_t z = zeros ? (uint32_t)(zeros[g * N + col] & 0xFu) : 8u;
        srec[t] = sb;
        zword |= z << (4 * t);
        if (bf16) needs_exact |= needs_exact_path(col_params<DT_BF16>(sb, z));
    }
    if (zeros) ((uint16_t*)(packed + z_off + rec * kZeroRecBytes))[c32] = (uint16_t)zword;
    if (needs_exact) atomicOr((uint32_t*)(packed + t_off) + 2, kFlagExactBf16);
}

__global__ void unrepack_meta_kernel(const uint8_t* __restrict__ packed,
                                     uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros,
                                     int64_t N, int64_t NG, size_t s_off, size_t z_off,
                                     int64_t nrec32) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nrec32) return;
    const int c32 = (int)(idx & 31);
    const int64_t rec = idx >> 5;
    const int64_t g = rec % NG;
    const int64_t nb = rec / NG;
    const uint16_t* srec = (const uint16_t*)(packed + s_off + rec * kScaleRecBytes) + 4 * c32;
    const uint32_t zword =
        zeros ? ((const uint16_t*)(packed + z_off + rec * kZeroRecBytes))[c32] : 0u;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t col = nb * kColBlock + 32 * t + c32;
        scales[g * N + col] = srec[t];
        if (zeros) zeros[g * N + col] = (uint8_t)((zword >> (4 * t)) & 0xFu);
    }
}

// Materialising dequant: one thread per repacked word, the same device
// dequantization the GEMM kernels run, eight values written to W[k][col].
template <int DT, bool SYM>
__global__ void dequant_kernel(const uint8_t* __restrict__ packed, uint16_t* __restrict__ W,
                               int64_t N, int64_t KS, int64_t NG, int GS, size_t s_off,
                               size_t z_off, int64_t nwords) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nwords) return;
    const int t = (int)(idx & 3);
    const int lane = (int)((idx >> 2) & 63);
    const int64_t chunk = idx >> 8;
    const int64_t ks = chunk % KS;
    const int64_t nb = chunk / KS;
    const int64_t g = ks / GS;
    const int64_t rec = nb * NG + g;
    const int c32 = lane & 31;
    const u32x2 sc = *(const u32x2*)(packed + s_off + rec * kScaleRecBytes + 8 * c32);
    const uint32_t zw =
        SYM ? 0u : (uint32_t)((const uint16_t*)(packed + z_off + rec * kZeroRecBytes))[c32];
    const ColParams<DT> prm = tile_params<DT, SYM>(sc, zw, t);
    const uint32_t w = ((const uint32_t*)packed)[idx];
    const u32x4 d = needs_exact_path(prm) ? dequant_word_exact(w, prm) : dequant_word(w, prm);
    const int64_t col = nb * kColBlock + 32 * t + c32;
    const int64_t k0 = kKStep * ks + 8 * (lane >> 5);
    const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int j = 0; j < 8; ++j)
        W[(k0 + j) * N + col] = (uint16_t)((j & 1) ? (dw[j >> 1] >> 16) : (dw[j >> 1] & 0xFFFFu));
}

inline unsigned blocks_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

hipError_t launch_repack(const uint32_t* qweight, const void* scales, const uint8_t* zeros,
                         const Layout& L, bool bf16, void* packed, hipStream_t stream) {
    const int64_t nwords = (int64_t)(L.w_bytes / 4);
    const int64_t nrec32 = L.NB * L.NG * 32;
    hipLaunchKernelGGL(repack_words_kernel, dim3(blocks_for(nwords, 256)), dim3(256), 0, stream,
                       qweight, (uint32_t*)packed, L.N, L.KS, nwords);
    hipLaunchKernelGGL(init_trailer_kernel, dim3(1), dim3(1), 0, stream,
                       (uint32_t*)((uint8_t*)packed + L.t_off), (uint32_t)L.G);
    hipLaunchKernelGGL(repack_meta_kernel, dim3(blocks_for(nrec32, 256)), dim3(256), 0, stream,
                       (const uint16_t*)scales, L.sym ? nullptr : zeros, (uint8_t*)packed, L.N,
                       L.NG, L.s_off, L.z_off, L.t_off, bf16 ? 1 : 0, nrec32);
    return hipGetLastError();
}

hipError_t launch_unrepack(const void* packed, const Layout& L, bool /*bf16*/, uint32_t* qweight,
                           void* scales, uint8_t* zeros, hipStream_t stream) {
    const int64_t nwords = (int64_t)(L.w_bytes / 4);
    const int64_t nrec32 = L.NB * L.NG * 32;
    hipLaunchKernelGGL(unrepack_words_kernel, dim3(blocks_for(nwords, 256)), dim3(256), 0,
                       stream, (const uint32_t*)packed, qweight, L.N, L.KS, nwords);
    hipLaunchKernelGGL(unrepack_meta_kernel, dim3(blocks_for(nrec32, 256)), dim3(256), 0, stream,
                       (const uint8_t*)packed, (uint16_t*)scales, L.sym ? nullptr : zeros, L.N,
                       L.NG, L.s_off, L.z_off, nrec32);
    return hipGetLastError();
}

hipError_t launch_dequant(const void* packed, const Layout& L, bool bf16, void* W_out,
                          hipStream_t stream) {
    const int64_t nwords = (int64_t)(L.w_bytes / 4);
    const int GS = (int)(L.G / kKStep);
    const dim3 grid(blocks_for(nwords, 256)), block(256);
    const uint8_t* p = (const uint8_t*)packed;
    uint16_t* W = (uint16_t*)W_out;
    if (bf16) {
        if (L.sym)
            hipLaunchKernelGGL((dequant_kernel<DT_BF16, true>), grid, block, 0, stream, p, W, L.N,
                               L.KS, L.NG, GS, L.s_off, L.z_off, nwords);
        else
            hipLaunchKernelGGL((dequant_kernel<DT_BF16, false>), grid, block, 0, stream, p, W,
                               L.N, L.KS, L.NG, GS, L.s_off, L.z_off, nwords);
    } else {
        if (L.sym)
            hipLaunchKernelGGL((dequant_kernel<DT_F16, true>), grid, block, 0, stream, p, W, L.N,
                               L.KS, L.NG, GS, L.s_off, L.z_off, nwords);
        else
            hipLaunchKernelGGL((dequant_kernel<DT_F16, false>), grid, block, 0, stream, p, W,
                               L.N, L.KS, L.NG, GS, L.s_off, L.z_off, nwords);
    }
    return hipGetLastError();
}

}  // namespace w4a16
