// w4a16_layout.h -- the repacked blob format (layout version 2), host and device.
//
// Page "量化开销对比" (laojiahuo2003.github.io), section 6.4: the scale and zero
// of a weight tile must sit next to it in the order the kernel consumes it, so
// weights, scales and zeros are reordered once, offline.  This is the order
// the gfx950 kernels consume.
//
// Units: a tile is 32 output columns (the N side of one v_mfma_f32_32x32x16);
// a k-step is 16 reduction indices (its K side); a chunk is 4 k-steps (64 of
// K) of one tile, 1 KiB; a body is 4 chunks (256 of K).  NT = N/32 tiles,
// KC = K/64 chunks and KB = K/256 bodies per tile, NG = K/G groups.
//
// Region W (offset 0, K*N/2 bytes): chunk (t, c) at byte (t*KC + c)*1024, so
// one tile's weights are one contiguous stream along K.  Inside a chunk, lane
// l (0..63) owns the 16 bytes at l*16: four uint32 words, word u (0..3) at
// l*16 + 4u.  Word u of lane l holds the eight weights of column
// 32*t + (l % 32) at reduction indices  k = 64*c + 16*u + 8*(l / 32) + j,
// j = 0..7 -- exactly the B operand lane l needs for k-step 4c+u of tile t.
// Inside the word, nibble position p (bits 4p..4p+3) holds j = 2*(p % 4) +
// p / 4, so that the masks 0x000F000F and 0x00F000F0, applied to the word and
// to the word shifted right by 8, yield the pairs (j0,j1), (j2,j3), (j4,j5),
// (j6,j7) in the two 16-bit halves of a register.  One global_load_dwordx4 per
// lane moves a whole chunk (64 lanes x 16 B = 1 KiB contiguous): four
// k-steps of one tile, however many tiles a wave works on.
//
// Region S (offset K*N/2, NG*N*2 bytes): per (tile t, body b) a record of 32
// lane entries, entry c32 at byte ((t*KB + b)*32 + c32) * SE with SE = 512/G
// bytes: the 256/G scales of the groups (256/G)*b + e, e = 0..256/G-1, that
// body b of column 32*t + c32 spans, entry e at 2e.  One 4-, 8- or 16-byte
// load per lane fetches every scale of a body.
//
// Region Z (asymmetric only; offset K*N/2 + NG*N*2, NG*N/2 bytes): per (t, b)
// a record of 32 entries of ZE = 128/G bytes at ((t*KB + b)*32 + c32) * ZE:
// nibble e is the zero point of group (256/G)*b + e of column 32*t + c32.
//
// Trailer (16 bytes, after region Z): uint32 magic kTrailerMagic, uint32 layout
// version, uint32 feature flags, uint32 group size.  Feature flag
// kFlagExactBf16 is set by the repack when some column's -(1024+z)*s
// overflows fp32 (bf16 scales above about 3.3e35); the GEMM kernels then use
// the exact dequant form for the whole launch instead of testing every group.
//
// Every byte of regions W, S and Z is an algorithmic byte of the quantized
// weight (4 bits per weight, one scale and one 4-bit zero per group and
// column), in consumption order.  Shapes: K % 256 == 0, N % 64 == 0.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

constexpr int kTileCols = 32;      // columns per tile
constexpr int kKStep = 16;         // reduction indices per k-step
constexpr int kChunkK = 64;        // reduction indices per chunk
constexpr int kBodyK = 256;        // reduction indices per body
constexpr int kChunkBytes = 1024;  // one (tile, chunk)
constexpr int kKAlign = kBodyK;    // K must be a multiple of this
constexpr int kNAlign = 64;        // N must be a multiple of this
constexpr int kTrailerBytes = 16;
constexpr uint32_t kLayoutVersion = 2;
constexpr uint32_t kTrailerMagic = 0x36314134u;   // "4A16"
constexpr uint32_t kFlagExactBf16 = 1u;

struct Layout {
    int64_t K, N, G;
    bool sym;
    int64_t NT, KC, KB, NG;
    int SE, ZE;   // bytes per lane entry of a scale / zero record
    size_t w_bytes, s_off, s_bytes, z_off, z_bytes, t_off, total;
};

inline Layout make_layout(int64_t K, int64_t N, int64_t G, bool sym) {
    Layout L;
    L.K = K;
    L.N = N;
    L.G = G;
    L.sym = sym;
    L.NT = N / kTileCols;
    L.KC = K / kChunkK;
    L.KB = K / kBodyK;
    L.NG = K / G;
    L.SE = (int)(2 * kBodyK / G);
    L.ZE = (int)(kBodyK / (2 * G));
    L.w_bytes = (size_t)K * (size_t)N / 2;
    L.s_off = L.w_bytes;
    L.s_bytes = (size_t)L.NG * (size_t)N * 2;
    L.z_off = L.s_off + L.s_bytes;
    L.z_bytes = sym ? 0 : (size_t)L.NG * (size_t)N / 2;
    L.t_off = L.z_off + L.z_bytes;
    L.total = L.t_off + kTrailerBytes;
    return L;
}

}  // namespace w4a16
