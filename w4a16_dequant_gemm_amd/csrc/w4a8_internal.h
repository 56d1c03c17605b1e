// w4a8_internal.h -- the W4A8 blob layout, the kernel plan and the launchers,
// shared by the C ABI layer and the HIP translation units.  Not part of the
// public interface.
//
// Blob (layout version 1), for K % 256 == 0, N % 128 == 0, G in {32, 64, 128}.
// A tile is 32 output columns (the N side of one v_mfma_i32_32x32x32_i8), a
// k-step 32 reduction indices (its K side), a chunk 2 k-steps of one tile:
// 64 lanes x 16 bytes = 1 KiB.  NT = N/32, KC = K/64, NG = K/G.
//
// Region W (offset 0, K*N/2 bytes): chunk (t, c) at byte (t*KC + c)*1024, so
// one tile's weights are one contiguous stream along K.  Lane l owns the 16
// bytes at l*16: words j = 0..3.  Word j holds the codes of column
// 32t + (l % 32) at  k = 64c + 32*(j/2) + 16*(l/32) + 8*(j%2) + i,  i = 0..7,
// code i at nibble position 2i (i < 4) or 2(i-4)+1 (i >= 4).  Masking the
// word with 0x0F0F0F0F then gives codes 0..3 one per byte, and the word
// shifted right by 4 gives codes 4..7: after the multiply-add and the XOR the
// two registers are 8 int8 weights in k order, and words 2s, 2s+1 are lane
// l's 16-byte B operand of k-step s.
//
// Region M (offset K*N/2, NG*N*2 bytes): entry (t, g, c32) at byte
// ((t*NG + g)*32 + c32)*2, the uint16 s8 | a << 8 of group g of column
// 32t + c32.
//
// Region C (N*4 bytes): the per-column fp32 scale sw[n], natural order.
//
// Trailer (16 bytes): magic, layout version, feature flags (kW8FlagOverflow:
// some group has s8 > 16 or a + 15*s8 > 255, outside the format), group size.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/w4a8.h"

namespace w4a8 {

constexpr int kTileCols = 32;
constexpr int kChunkK = 64;
constexpr int kChunkBytes = 1024;
constexpr int kKAlign = 256;
constexpr int kNAlign = 128;
constexpr int kTrailerBytes = 16;
constexpr uint32_t kLayoutVersion = W4A8_LAYOUT_VERSION;
constexpr uint32_t kTrailerMagic = 0x57384134u;   // "4A8W"
constexpr uint32_t kW8FlagOverflow = 1u;
constexpr int kMaxK = 1 << 17;                     // |acc| < 127 * 128 * K < 2^31

struct LayoutW8 {
    int64_t K, N, G;
    int64_t NT, KC, NG;
    size_t w_bytes, m_off, m_bytes, c_off, c_bytes, t_off, total;
};

inline LayoutW8 make_layout_w8(int64_t K, int64_t N, int64_t G) {
    LayoutW8 L;
    L.K = K;
    L.N = N;
    L.G = G;
    L.NT = N / kTileCols;
    L.KC = K / kChunkK;
    L.NG = K / G;
    L.w_bytes = (size_t)K * (size_t)N / 2;
    L.m_off = L.w_bytes;
    L.m_bytes = (size_t)L.NG * (size_t)N * 2;
    L.c_off = L.m_off + L.m_bytes;
    L.c_bytes = (size_t)N * 4;
    L.t_off = L.c_off + L.c_bytes;
    L.total = L.t_off + kTrailerBytes;
    return L;
}

// Output kinds (the W4A8_OUT_* flag values).
enum { OUT_F16 = 0, OUT_BF16 = 1, OUT_I32 = 2 };

// Kernel variants.
//   STREAM: M <= 32 (up to 64 when asked for).  Eight waves per workgroup =
//           (8/KP) tiles x KP parts of K; each wave streams its tile's chunks and reads its rows of X
//           straight from memory (X is small and stays in L2); the parts meet
//           in LDS (integer sums, so their order does not matter).
//   TILED:  M > 32.  Eight waves = WM x WN; a workgroup owns BM rows x BN
//           columns over all of K; X goes through a two-slot LDS ring, each
//           wave streams its own tiles' weights.
enum VariantW8 { W8_STREAM = 0, W8_TILED = 1 };
constexpr int kW8Waves = 8;
constexpr int kStreamMaxRows = 64;      // largest M the streaming kernel takes
constexpr int kStreamDefaultRows = 32;  // largest M it is chosen for by default
constexpr int kTiledRowBytes = 80;   // 64 bytes of X per row and chunk + 16 of padding

struct PlanW8 {
    VariantW8 variant;
    int rt;          // 32-row tiles per wave
    int kp;          // STREAM: parts of K per tile
    bool bd;         // STREAM, M <= 4: v_mfma_i32_16x16x64_i8 with a block-diagonal A
    int cfg;         // TILED: workgroup tile 0 = 256 x 256, 1 = 128 x 128, 2 = 256 x 128,
                     // 3 = 256 x 256 with two chunks per LDS stage, 4 = the same with
                     // the int8 weights made once per workgroup in LDS
    int grid;        // workgroups
    int nbm, nbn;    // TILED: row and column blocks
    size_t lds;      // dynamic LDS bytes
};

PlanW8 make_plan_w8(int64_t M, int64_t N, int64_t K, uint32_t flags, int cus);

hipError_t launch_w8_repack(const uint32_t* qweight, const uint8_t* s8, const uint8_t* a,
                            const float* sw, const LayoutW8& L, void* packed, hipStream_t stream);
hipError_t launch_w8_dequant(const void* packed, const LayoutW8& L, int8_t* W_out,
                             hipStream_t stream);
hipError_t launch_w8_quantize_rows(const void* X, bool bf16, int8_t* xq, float* sx, int64_t M,
                                   int64_t K, hipStream_t stream);
// One object per output kind.
#define W4A8_DECLARE_GEMM_PART(name)                                                      \
    hipError_t name(const int8_t* xq, const float* sx, const void* packed, void* Y,      \
                    int64_t M, const LayoutW8& L, const PlanW8& plan, hipStream_t stream);
W4A8_DECLARE_GEMM_PART(launch_w8_gemm_f16)
W4A8_DECLARE_GEMM_PART(launch_w8_gemm_bf16)
W4A8_DECLARE_GEMM_PART(launch_w8_gemm_i32)
#undef W4A8_DECLARE_GEMM_PART

}  // namespace w4a8
