// w4a16_layout.h -- the repacked blob format (layout version 1), host and device.
//
// Page "量化开销对比" (laojiahuo2003.github.io), section 6.4: the scale and zero
// of a weight tile must sit next to it in the order the kernel consumes it, so
// weights, scales and zeros are reordered once, offline.  This is the order
// the gfx950 kernels consume.
//
// Units: a column block is 128 output columns; a k-step is 16 reduction
// indices (the k of one v_mfma_f32_32x32x16).  NB = N/128, KS = K/16,
// NG = K/G.
//
// Region W (offset 0, K*N/2 bytes): one 1 KiB chunk per (nb, ks), chunk
// index nb*KS + ks.  Inside a chunk, lane l (0..63) owns 16 bytes at l*16,
// i.e. four uint32 words, word t (0..3) at l*16 + 4t.  Word t of lane l holds
// the eight weights of column  c = 128*nb + 32*t + (l % 32)  at reduction
// indices  k = 16*ks + 8*(l / 32) + j,  j = 0..7 -- exactly the B operand lane
// l needs for column tile t of one 32x32x16 MFMA.  Inside the word, nibble
// position p (bits 4p..4p+3) holds j = 2*(p % 4) + p / 4, so that the masks
// 0x000F000F and 0x00F000F0, applied to the word and to the word shifted right
// by 8, yield the pairs (j0,j1), (j2,j3), (j4,j5), (j6,j7) in the two 16-bit
// halves of a register.  One global_load_dwordx4 per lane moves a whole chunk:
// 64 lanes x 16 B = 1 KiB contiguous.
//
// Region S (offset K*N/2, NG*N*2 bytes): one 256-byte record per (nb, g),
// record index nb*NG + g.  Entry (c32, t) at byte 8*c32 + 2*t is the scale of
// column 128*nb + 32*t + c32 for group g: lane l loads its four column scales
// with one 8-byte load at 8*(l % 32).
//
// Region Z (asymmetric only; offset K*N/2 + NG*N*2, NG*N/2 bytes): one 64-byte
// record per (nb, g).  The 16-bit entry at 2*c32 holds, in nibble t, the zero
// point of column 128*nb + 32*t + c32 for group g.
//
// Trailer (16 bytes, after region Z): uint32 magic kTrailerMagic, uint32 layout
// version, uint32 feature flags, uint32 group size.  Feature flag
// kFlagExactBf16 is set by the repack when some column's -(1024+z)*s overflows
// fp32 (bf16 scales above about 3.3e35); the GEMM kernels then use the exact
// dequant form for the whole launch instead of testing every group.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

constexpr int kColBlock = 128;     // columns per column block
constexpr int kKStep = 16;         // reduction indices per k-step
constexpr int kChunkBytes = 1024;  // one (column block, k-step) chunk
constexpr int kScaleRecBytes = 256;
constexpr int kZeroRecBytes = 64;
constexpr int kTrailerBytes = 16;
constexpr uint32_t kTrailerMagic = 0x36314134u;   // "4A16"
constexpr uint32_t kFlagExactBf16 = 1u;

struct Layout {
    int64_t K, N, G;
    bool sym;
    int64_t NB, KS, NG;
    size_t w_bytes, s_off, s_bytes, z_off, z_bytes, t_off, total;
};

inline Layout make_layout(int64_t K, int64_t N, int64_t G, bool sym) {
    Layout L;
    L.K = K;
    L.N = N;
    L.G = G;
    L.sym = sym;
    L.NB = N / kColBlock;
    L.KS = K / kKStep;
    L.NG = K / G;
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
