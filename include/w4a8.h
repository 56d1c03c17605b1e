/*
 * w4a8.h -- C ABI of the W4A8 route of the MI355X (gfx950) library: 4-bit
 * weights turned into int8 in registers, int8 activations, int8 MFMA with
 * int32 accumulation.  Same shared library and status codes as w4a16.h.
 *
 *   w8[k][n]  = int8( ((q[k][n] * s8[g][n] + a[g][n]) mod 256) XOR 0x80 ),  g = floor(k / G)
 *   acc[m][n] = sum over k of xq[m][k] * w8[k][n]        (int32, exact)
 *   Y[m][n]   = RNE_out( (float(acc[m][n]) * sx[m]) * sw[n] )   (fp32 products)
 *
 * The weight step is the LiquidQuant congruence of page "W4A8量化计算优化：
 * 提升LLM推理效率的关键技术" (bjdmk.com.cn), section 2.1: per group of G
 * reduction indices of one column, a u8 scale s8 <= 16 and a u8 offset a
 * (128 plus the group's smallest int8 weight), so that one multiply-add and
 * one XOR per register turn 4-bit codes into int8 weights.  Here that is one
 * v_pk_mad_u16 and one v_xor_b32 per four weights.  The product is route A
 * of page "量化开销对比：各家方案的矩阵乘账本与省账手段"
 * (laojiahuo2003.github.io), section 1 (int8 times int8, int32 accumulation,
 * then the scales), with symmetric per-row activation and per-column weight
 * scales applied after the sum (section 2).  The activation scales are taken
 * per row at run time (section 4, dynamic route): w4a8_quantize_rows.
 *
 * Format bound: a group must satisfy s8 <= 16 and a + 15*s8 <= 255 (no code
 * can carry out of its byte).  The repack records a group outside it in the
 * blob trailer's feature flags (bit 0; the trailer is the last 16 bytes of
 * the blob: magic, layout version, flags, group size); the GEMM reads no
 * flag and its result for such a group is unspecified (every access stays in
 * bounds).
 *
 * Conventions are those of w4a16.h: plain C types; dev pointers are device
 * memory on the current HIP device, 16-byte aligned, owned by the caller;
 * `stream` is a hipStream_t as void* (NULL = null stream); work is enqueued
 * asynchronously, nothing is allocated, copied to the host or synchronized;
 * every argument is validated on the host before any HIP call, and a call
 * that fails validation launches nothing.  Shapes: M >= 1; K % 256 == 0 and
 * 256 <= K <= 131072 (so |acc| < 2^31); N % 128 == 0; G in {32, 64, 128};
 * M, N < 2^31 and K*N < 2^40.  Other K, N or G: W4A16_ERR_UNSUPPORTED when
 * the request is otherwise well formed.
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#include "w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

#define W4A8_LAYOUT_VERSION 1

/* Output kind, the flags of w4a8_gemm (exactly one). */
#define W4A8_OUT_FP16 0x0u   /* Y: IEEE binary16 [M][N] */
#define W4A8_OUT_BF16 0x1u   /* Y: bfloat16 [M][N] */
#define W4A8_OUT_I32  0x2u   /* Y: int32 [M][N], the raw accumulators (sx, sw unused) */
#define W4A8_OUT_MASK 0x3u
/* Plan hints (w4a8_gemm flags only; for tests and benchmarks).  A hint that
 * does not apply to the shape is ignored.  W4A16_PLAN_PARAM(n) sets the
 * streaming kernel's parts of K per tile (2, 4 or 8), or the tiled kernel's
 * workgroup tile (1: 256 x 256, 2: 128 x 128, 3: 256 x 128, 4: 256 x 256 with
 * two chunks of K per LDS stage, 5: the same with the int8 weights made once per
 * workgroup in LDS). */
#define W4A8_PLAN_STREAM 0x10u   /* streaming kernel, M <= 64 */
#define W4A8_PLAN_TILED  0x20u   /* LDS-tiled kernel */
#define W4A8_PLAN_MASK   0x30u

/* Flags of w4a8_quantize_rows: the dtype of X. */
#define W4A8_X_FP16 0x0u
#define W4A8_X_BF16 0x1u

/* Trailer feature flag: some group is outside the format bound. */
#define W4A8_TRAILER_OVERFLOW 0x1u

/*
 * Bytes of the repacked blob for (K, N, G), or 0 if the shape is invalid or
 * unsupported: K*N/2 (codes) + (K/G)*N*2 (s8 and a) + N*4 (sw) + a 16-byte
 * trailer.
 */
size_t w4a8_packed_bytes(int64_t K, int64_t N, int group_size);

/*
 * Offline repack into the kernels' order (page "量化开销对比", section 6.4:
 * the per-group constants sit next to the weights they serve).
 *   qweight  dev, uint32 [K/8][N]; nibble i (bits 4i..4i+3) of word [r][n] is
 *            q[8r+i][n] (the order of w4a16_repack).
 *   s8, a    dev, uint8 [K/G][N].
 *   sw       dev, float [N], the per-column weight scale.
 *   packed   dev, output, packed_bytes >= w4a8_packed_bytes(K, N, G).
 * Errors: INVALID_ARG (shape, NULL or misaligned pointer, short packed_bytes),
 * UNSUPPORTED (K, N or G outside the supported set), HIP.
 */
w4a16_status_t w4a8_repack(const uint32_t *qweight, const uint8_t *s8, const uint8_t *a,
                           const float *sw, int64_t K, int64_t N, int group_size, void *packed,
                           size_t packed_bytes, void *stream);

/*
 * Materialise the int8 weights w8 [K][N] (row-major, dev) of a blob, with the
 * same in-register steps the GEMM uses.  For checks; not on the token path.
 */
w4a16_status_t w4a8_dequant(const void *packed, size_t packed_bytes, int8_t *W_out, int64_t K,
                            int64_t N, int group_size, void *stream);

/*
 * Dynamic per-row symmetric int8 quantisation of activations (page
 * "量化开销对比", section 4): for each row m, sx[m] = max_k |X[m][k]| / 127
 * and xq[m][k] = round-half-even(X[m][k] / sx[m]) clamped to [-127, 127],
 * both in fp32 with IEEE division; a row of zeros gives sx = 0 and xq = 0.
 * X must be finite.
 *   X   dev, fp16 or bf16 [M][K] per flags (W4A8_X_*);  xq dev, int8 [M][K];
 *   sx  dev, float [M].
 * Shapes: M >= 1, K % 256 == 0, K <= 131072.
 */
w4a16_status_t w4a8_quantize_rows(const void *X, int8_t *xq, float *sx, int64_t M, int64_t K,
                                  uint32_t flags, void *stream);

/*
 * Y = the W4A8 product defined at the top of this file.
 *   xq      dev, int8 [M][K] row-major.
 *   sx      dev, float [M] (may be NULL with W4A8_OUT_I32).
 *   packed  dev, a blob of w4a8_repack for (K, N, G).
 *   Y       dev, [M][N] of the output kind in flags.
 * Kernel choice (by M): the streaming kernel for M <= 32, the LDS-tiled
 * kernel above (workgroup tile 128 x 128 up to M = 128, 256 x 128 up to 512,
 * 256 x 256 with two chunks of K per LDS stage beyond).
 * No workspace.  Calls on one stream may run back to back; Y must not
 * overlap the inputs.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
w4a16_status_t w4a8_gemm(const int8_t *xq, const float *sx, const void *packed,
                         size_t packed_bytes, void *Y, int64_t M, int64_t N, int64_t K,
                         int group_size, uint32_t flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
