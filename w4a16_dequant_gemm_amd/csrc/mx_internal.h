// mx_internal.h -- the MXFP4 blob layout, the kernel plan and the launchers,
// shared by the C ABI layer and the HIP translation units.  Not part of the
// public interface.
//
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 with an E4M3 A and an
// E2M1 B (measured on gfx950: D = A.B matches for random operands and block
// scales, and one-hot operands locate every element):
//   B, lane l: column l % 32, the 32 codes of k = 32*(l/32) + j, j = 0..31,
//      code j at bits 4j of the 16-byte operand; its scale byte is the E8M0
//      scale of that block of 32 (block l/32).
//   A, lane l: row l % 32, bytes j = 0..15 hold k = 16*(l/32) + j and bytes
//      16..31 hold k = 32 + 16*(l/32) + (j - 16); the scale byte of lane l is
//      the E8M0 scale of row l % 32, block l/32 (k = 32*(l/32) .. +31), even
//      though half of lane l's own bytes lie in the other block.
//
// Blob (layout version 1), K % 256 == 0, N % 128 == 0.  Tiles of 32 columns,
// k-steps of 64; NT = N/32, KS = K/64, KQ = K/256.
// Region W (offset 0, K*N/2 bytes): chunk (t, s) at byte (t*KS + s)*1024;
//   lane l owns the 16 bytes at l*16 = the canonical words of column
//   32t + (l % 32) at rows (64s + 32*(l/32))/8 + u, u = 0..3 -- the B operand
//   of k-step s as it is, with no reordering inside a word.
// Region S (K*N/32 bytes): per (tile t, quad q of 4 k-steps) 64 lanes x 4
//   bytes at ((t*KQ + q)*64 + l)*4: byte u is the scale of column 32t + l%32,
//   block 2*(4q + u) + l/32, i.e. lane l's B scale for k-step 4q + u.
// Trailer (16 bytes): magic, layout version, flags, 32 (the block size);
// flag bit 0: some weight block scale is 0xFF (the E8M0 NaN).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mxfp4.h"

namespace mxfp4 {

constexpr int kTileCols = 32;
constexpr int kStepK = 64;
constexpr int kKAlign = 256;
constexpr int kNAlign = 128;
constexpr int kTrailerBytes = 16;
constexpr uint32_t kTrailerMagic = 0x3450464Du;   // "MFP4"
constexpr uint32_t kTrailerFlagNanScale = 1u;

struct LayoutMX {
    int64_t K, N, NT, KS, KQ;
    size_t w_bytes, s_off, s_bytes, t_off, total;
};

inline LayoutMX make_layout_mx(int64_t K, int64_t N) {
    LayoutMX L;
    L.K = K;
    L.N = N;
    L.NT = N / kTileCols;
    L.KS = K / kStepK;
    L.KQ = K / kKAlign;
    L.w_bytes = (size_t)K * (size_t)N / 2;
    L.s_off = L.w_bytes;
    L.s_bytes = (size_t)K * (size_t)N / 32;
    L.t_off = L.s_off + L.s_bytes;
    L.total = L.t_off + kTrailerBytes;
    return L;
}

enum VariantMX { MX_STREAM = 0, MX_TILED = 1 };
constexpr int kMxWaves = 8;
constexpr int kMxStreamMaxRows = 64;
constexpr int kMxStreamDefaultRows = 32;
constexpr int kMxBlockDiagMaxRows = 8;   // streaming kernel on the 16x16x128 form
// ... while M * K, its X bytes, stays below this (32-bit buffer offsets)
constexpr int64_t kMxBlockDiagMaxXBytes = (int64_t)1 << 30;
constexpr int kMxRowBytes = 80;   // 64 bytes of X per row and k-step + 16 of padding

struct PlanMX {
    VariantMX variant;
    int rt;          // 32-row tiles per wave
    int kp;          // STREAM: parts of K per tile
    bool bd;         // STREAM: the 16x16x128 block-diagonal form (M <= 4)
    int cfg;         // TILED: workgroup tile 0 = 256 x 256, 1 = 128 x 128, 2 = 256 x 128,
                     // 3 = 256 x 256 with two k-steps per LDS stage
    int grid;
    int nbm, nbn;
    size_t lds;
};

PlanMX make_plan_mx(int64_t M, int64_t N, int64_t K, uint32_t flags, int cus);

hipError_t launch_mx_repack(const uint32_t* qweight, const uint8_t* ws, const LayoutMX& L,
                            void* packed, hipStream_t stream);
hipError_t launch_mx_quantize_rows(const void* X, bool bf16, uint8_t* xq, uint8_t* xs, int64_t M,
                                   int64_t K, hipStream_t stream);
#define MXFP4_DECLARE_GEMM_PART(name)                                                      \
    hipError_t name(const uint8_t* xq, const uint8_t* xs, const void* packed, void* Y,     \
                    int64_t M, const LayoutMX& L, const PlanMX& plan, hipStream_t stream);
MXFP4_DECLARE_GEMM_PART(launch_mx_gemm_f16)
MXFP4_DECLARE_GEMM_PART(launch_mx_gemm_bf16)
#undef MXFP4_DECLARE_GEMM_PART

}  // namespace mxfp4
