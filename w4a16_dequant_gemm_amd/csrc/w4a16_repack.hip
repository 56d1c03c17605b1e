// w4a16_repack.hip -- offline repack of canonical tensors into the kernel
// order (see w4a16_layout.h), its exact inverse, and the
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

// Word index inside region W -> (column, canonical word row): word u of lane
// l of chunk (t, c) holds column 32t + l%32 at k = 64c + 16u + 8(l/32) + j,
// i.e. canonical word row (64c + 16u + 8(l/32)) / 8.
struct WordPos {
    int64_t col, row;   // canonical qweight[row][col]
};

__device__ __forceinline__ WordPos word_pos(int64_t idx, int64_t KC) {
    const int u = (int)(idx & 3);
    const int lane = (int)((idx >> 2) & 63);
    const int64_t chunk = idx >> 8;
    const int64_t c = chunk % KC;
    const int64_t t = chunk / KC;
    WordPos p;
    p.col = t * kTileCols + (lane & 31);
    p.row = 8 * c + 2 * u + (lane >> 5);
    return p;
}

__global__ void repack_words_kernel(const uint32_t* __restrict__ qweight,
                                    uint32_t* __restrict__ out, int64_t N, int64_t KC,
                                    int64_t nwords) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nwords) return;
    const WordPos p = word_pos(idx, KC);
    out[idx] = canonical_to_repacked(qweight[p.row * N + p.col]);
}

__global__ void unrepack_words_kernel(const uint32_t* __restrict__ in,
                                      uint32_t* __restrict__ qweight, int64_t N, int64_t KC,
                                      int64_t nwords) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nwords) return;
    const WordPos p = word_pos(idx, KC);
    qweight[p.row * N + p.col] = repacked_to_canonical(in[idx]);
}

__global__ void init_trailer_kernel(uint32_t* __restrict__ trailer, uint32_t group_size) {
    trailer[0] = kTrailerMagic;
    trailer[1] = kLayoutVersion;
    trailer[2] = 0u;   // feature flags, OR-ed by repack_meta_kernel
    trailer[3] = group_size;
}

// One thread per lane entry (t, b, c32): the EPB = 256/G scales and zeros of
// body b of column 32t + c32.  For bf16 it also flags the blob when
// -(1024+z)*s overflows fp32 for some column.
__global__ void repack_meta_kernel(const uint16_t* __restrict__ scales,
                                   const uint8_t* __restrict__ zeros, uint8_t* __restrict__ packed,
                                   int64_t N, int64_t KB, int EPB, size_t s_off, size_t z_off,
                                   size_t t_off, int bf16, int64_t nent) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nent) return;
    const int c32 = (int)(idx & 31);
    const int64_t rec = idx >> 5;          // t * KB + b
    const int64_t b = rec % KB;
    const int64_t t = rec / KB;
    const int64_t col = t * kTileCols + c32;
    uint16_t* sent = (uint16_t*)(packed + s_off) + idx * EPB;
    uint32_t zword = 0;
    bool needs_exact = false;
    for (int e = 0; e < EPB; ++e) {
        const int64_t g = b * EPB + e;
        const uint16_t sb = scales[g * N + col];
        const uint32_t z = zeros ? (uint32_t)(zeros[g * N + col] & 0xFu) : 8u;
        sent[e] = sb;
        zword |= z << (4 * e);
        if (bf16) needs_exact |= needs_exact_path(col_params<DT_BF16>(sb, z));
    }
    if (zeros) {
        uint8_t* zent = packed + z_off + idx * (EPB / 2);
        for (int i = 0; i < EPB / 2; ++i) zent[i] = (uint8_t)(zword >> (8 * i));
    }
    if (needs_exact) atomicOr((uint32_t*)(packed + t_off) + 2, kFlagExactBf16);
}

__global__ void unrepack_meta_kernel(const uint8_t* __restrict__ packed,
                                     uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros,
                                     int64_t N, int64_t KB, int EPB, size_t s_off, size_t z_off,
                                     int64_t nent) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nent) return;
    const int c32 = (int)(idx & 31);
    const int64_t rec = idx >> 5;
    const int64_t b = rec % KB;
    const int64_t t = rec / KB;
    const int64_t col = t * kTileCols + c32;
    const uint16_t* sent = (const uint16_t*)(packed + s_off) + idx * EPB;
    const uint8_t* zent = packed + z_off + idx * (EPB / 2);
    for (int e = 0; e < EPB; ++e) {
        const int64_t g = b * EPB + e;
        scales[g * N + col] = sent[e];
        if (zeros) zeros[g * N + col] = (uint8_t)((zent[e >> 1] >> (4 * (e & 1))) & 0xFu);
    }
}

// Materialising dequant: one thread per repacked word, the same device
// dequantization the GEMM kernels run, eight values written to W[k][col].
template <int DT, bool SYM>
__global__ void dequant_kernel(const uint8_t* __restrict__ packed, uint16_t* __restrict__ W,
                               int64_t N, int64_t KC, int64_t KB, int G, size_t s_off,
                               size_t z_off, int64_t nwords) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nwords) return;
    const int u = (int)(idx & 3);
    const int lane = (int)((idx >> 2) & 63);
    const int64_t chunk = idx >> 8;
    const int64_t c = chunk % KC;
    const int64_t t = chunk / KC;
    const int c32 = lane & 31;
    const int64_t k0 = kChunkK * c + kKStep * u + 8 * (lane >> 5);
    const int EPB = kBodyK / G;
    const int64_t b = k0 / kBodyK;
    const int e = (int)((k0 - b * kBodyK) / G);           // group entry inside the body
    const int64_t ent = (t * KB + b) * 32 + c32;           // lane entry of record (t, b)
    const uint32_t sword = ((const uint32_t*)(packed + s_off + ent * 2 * EPB))[e >> 1];
    const uint32_t zword =
        SYM ? 0u : (uint32_t)(packed + z_off + ent * (EPB / 2))[e >> 1] << (4 * (e & ~1));
    const ColParams<DT> prm = entry_params<DT, SYM>(sword, zword, e);
    const uint32_t w = ((const uint32_t*)packed)[idx];
    const Magic mg = make_magic();
    const u32x4 d =
        needs_exact_path(prm) ? dequant_word_exact(w, prm, mg) : dequant_word(w, prm, mg);
    const int64_t col = t * kTileCols + c32;
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
    const int64_t nent = L.NT * L.KB * 32;
    hipLaunchKernelGGL(repack_words_kernel, dim3(blocks_for(nwords, 256)), dim3(256), 0, stream,
                       qweight, (uint32_t*)packed, L.N, L.KC, nwords);
    hipLaunchKernelGGL(init_trailer_kernel, dim3(1), dim3(1), 0, stream,
                       (uint32_t*)((uint8_t*)packed + L.t_off), (uint32_t)L.G);
    hipLaunchKernelGGL(repack_meta_kernel, dim3(blocks_for(nent, 256)), dim3(256), 0, stream,
                       (const uint16_t*)scales, L.sym ? nullptr : zeros, (uint8_t*)packed, L.N,
                       L.KB, (int)(kBodyK / L.G), L.s_off, L.z_off, L.t_off, bf16 ? 1 : 0, nent);
    return hipGetLastError();
}

hipError_t launch_unrepack(const void* packed, const Layout& L, bool /*bf16*/, uint32_t* qweight,
                           void* scales, uint8_t* zeros, hipStream_t stream) {
    const int64_t nwords = (int64_t)(L.w_bytes / 4);
    const int64_t nent = L.NT * L.KB * 32;
    hipLaunchKernelGGL(unrepack_words_kernel, dim3(blocks_for(nwords, 256)), dim3(256), 0,
                       stream, (const uint32_t*)packed, qweight, L.N, L.KC, nwords);
    hipLaunchKernelGGL(unrepack_meta_kernel, dim3(blocks_for(nent, 256)), dim3(256), 0, stream,
                       (const uint8_t*)packed, (uint16_t*)scales, L.sym ? nullptr : zeros, L.N,
                       L.KB, (int)(kBodyK / L.G), L.s_off, L.z_off, nent);
    return hipGetLastError();
}

hipError_t launch_dequant(const void* packed, const Layout& L, bool bf16, void* W_out,
                          hipStream_t stream) {
    const int64_t nwords = (int64_t)(L.w_bytes / 4);
    const dim3 grid(blocks_for(nwords, 256)), block(256);
    const uint8_t* p = (const uint8_t*)packed;
    uint16_t* W = (uint16_t*)W_out;
    const int G = (int)L.G;
    if (bf16) {
        if (L.sym)
            hipLaunchKernelGGL((dequant_kernel<DT_BF16, true>), grid, block, 0, stream, p, W, L.N,
                               L.KC, L.KB, G, L.s_off, L.z_off, nwords);
        else
            hipLaunchKernelGGL((dequant_kernel<DT_BF16, false>), grid, block, 0, stream, p, W,
                               L.N, L.KC, L.KB, G, L.s_off, L.z_off, nwords);
    } else {
        if (L.sym)
            hipLaunchKernelGGL((dequant_kernel<DT_F16, true>), grid, block, 0, stream, p, W, L.N,
                               L.KC, L.KB, G, L.s_off, L.z_off, nwords);
        else
            hipLaunchKernelGGL((dequant_kernel<DT_F16, false>), grid, block, 0, stream, p, W,
                               L.N, L.KC, L.KB, G, L.s_off, L.z_off, nwords);
    }
    return hipGetLastError();
}

}  // namespace w4a16
