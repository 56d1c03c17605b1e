/*
 * mxfp4.h -- C ABI of the MXFP4 route of the MI355X (gfx950) library: 4-bit
 * E2M1 weights and 8-bit E4M3 activations, each with an E8M0 scale per block
 * of 32 reduction indices, multiplied by the block-scaled matrix instruction
 * v_mfma_scale_f32_32x32x64_f8f6f4 (fp32 accumulation).  Same shared library
 * and status codes as w4a16.h.
 *
 *   w[k][n]  = e2m1(q[k][n]) * 2^(ws[k/32][n] - 127)
 *   xa[m][k] = e4m3(xq[m][k]) * 2^(xs[m][k/32] - 127)
 *   Y[m][n]  = RNE_out( sum over k of xa[m][k] * w[k][n] )   (fp32 accumulation)
 *
 * Page "量化开销对比：各家方案的矩阵乘账本与省账手段" (laojiahuo2003.github.io),
 * section 3, closing paragraph: the MXFP4 format puts a power-of-two (E8M0)
 * scale per block of 32 into the hardware, so 4-bit weights take route A
 * (section 1) again: the matrix unit consumes the packed operands and their
 * block scales directly, with no dequantisation step in the kernel.  The
 * element formats: E2M1 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) and E4M3
 * (no infinities, largest 448, 0x7F / 0xFF are NaN).
 *
 * Conventions are those of w4a16.h (plain C types, caller-owned 16-byte
 * aligned device pointers, stream as void*, asynchronous, nothing allocated,
 * every argument validated on the host before any HIP call).  Shapes: M >= 1;
 * K % 256 == 0; N % 128 == 0; M, N, K < 2^31 and K*N < 2^40.  Other K or N:
 * W4A16_ERR_UNSUPPORTED.
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stddef.h>
#include <stdint.h>

#include "w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MXFP4_LAYOUT_VERSION 1

/* Output dtype (mxfp4_gemm flags) and X dtype (mxfp4_quantize_rows flags). */
#define MXFP4_FP16 0x0u
#define MXFP4_BF16 0x1u
/* Plan hints (mxfp4_gemm flags only; tests and benchmarks).  A hint that does
 * not apply is ignored.  W4A16_PLAN_PARAM(n): the streaming kernel's parts of
 * K per tile (2, 4 or 8), or the tiled kernel's workgroup tile (1: 256 x 256,
 * 2: 128 x 128, 3: 256 x 128, 4: 256 x 256 with two k-steps per LDS stage). */
#define MXFP4_PLAN_STREAM 0x10u   /* streaming kernel, M <= 64 */
#define MXFP4_PLAN_TILED  0x20u   /* LDS-tiled kernel */
#define MXFP4_PLAN_MASK   0x30u

/* Bytes of the repacked blob for (K, N), or 0 if the shape is invalid or
 * unsupported: K*N/2 (codes) + K*N/32 (block scales) + a 16-byte trailer. */
size_t mxfp4_packed_bytes(int64_t K, int64_t N);

/*
 * Offline repack into the kernels' order (page "量化开销对比", section 6.4).
 *   qweight  dev, uint32 [K/8][N]; nibble i (bits 4i..4i+3) of word [r][n] is
 *            the E2M1 code of w[8r+i][n].
 *   ws       dev, uint8 [K/32][N], E8M0 block scales; 0xFF (the E8M0 NaN) makes
 *            its column of Y NaN, and the repack records its presence in the blob.
 *   packed   dev, output, packed_bytes >= mxfp4_packed_bytes(K, N).
 */
w4a16_status_t mxfp4_repack(const uint32_t *qweight, const uint8_t *ws, int64_t K, int64_t N,
                            void *packed, size_t packed_bytes, void *stream);

/*
 * MX quantisation of activations per row and block of 32 (the scale taken at
 * run time, as the dynamic route of page "量化开销对比", section 4): with amax
 * the block's largest magnitude, E = floor(log2 amax) - 8 (at least -127; -127
 * for a block of zeros), xs = E + 127, and each element is X * 2^-E rounded
 * to the nearest E4M3 value, ties to the even code, magnitudes above 448
 * saturating to 448.  X must be finite.
 *   X   dev, fp16 or bf16 [M][K] per flags;  xq dev, uint8 [M][K] E4M3 codes;
 *   xs  dev, uint8 [M][K/32].
 */
w4a16_status_t mxfp4_quantize_rows(const void *X, uint8_t *xq, uint8_t *xs, int64_t M, int64_t K,
                                   uint32_t flags, void *stream);

/*
 * Y = the product defined at the top of this file.
 *   xq  dev, uint8 [M][K] E4M3 codes; xs dev, uint8 [M][K/32] E8M0 scales;
 *   packed  a blob of mxfp4_repack for (K, N);  Y dev, fp16 or bf16 [M][N].
 * Kernel choice (by M): a streaming kernel for M <= 32 (on the 16x16x128 form
 * of the instruction for M <= 4 unless the blob holds a NaN weight scale), the
 * LDS-tiled kernel above.  No workspace.
 */
w4a16_status_t mxfp4_gemm(const uint8_t *xq, const uint8_t *xs, const void *packed,
                          size_t packed_bytes, void *Y, int64_t M, int64_t N, int64_t K,
                          uint32_t flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
