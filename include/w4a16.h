/*
 * w4a16.h -- C ABI of the MI355X (gfx950) fused W4A16 dequantize-GEMM library.
 *
 *   Y[M][N] = X[M][K] . deq[K][N],   deq[k][n] = RNE((q[k][n] - z[g][n]) * s[g][n]),
 *   g = floor(k / G), fp32 accumulation, Y rounded to the activation dtype.
 *
 * The method: page "W4A16 GEMM 算子浅析：INT4 权重反量化的计算流水线"
 * (nxmr.cn), section "计算流水线的核心哲学" -- 4-bit weights stay packed in
 * HBM, are unpacked and dequantized (weight minus zero, times scale) in
 * registers, and only then feed the matrix unit with fp32 accumulation; and
 * page "量化开销对比：各家方案的矩阵乘账本与省账手段" (laojiahuo2003.github.io),
 * section 6: one launch, one pass over the weights, nothing materialised in
 * between (6.1); the group scale multiplies the weight operand before the
 * multiply-accumulate because it changes along k (6.2); weights, scales and
 * zeros are repacked offline into the kernel's order (6.4).
 *
 * Conventions for every entry point:
 *   - Plain C types only; no exception crosses the ABI.
 *   - "dev" pointers are device memory on the current HIP device; the caller
 *     owns every buffer.  The library never allocates, frees or synchronizes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; no host<->device copies are made,
 *     so calls may be captured into a HIP graph.
 *   - Every argument is validated on the host before any HIP call.  A call
 *     that fails validation launches nothing and writes nothing.  A launch
 *     error reported by HIP is returned as W4A16_ERR_HIP.
 *   - Supported shapes: M >= 1; K >= 1 with K % G == 0 and K % 256 == 0; N >= 1
 *     with N % 128 == 0 (other K or N: W4A16_ERR_UNSUPPORTED); G in {32, 64,
 *     128} (other G: W4A16_ERR_UNSUPPORTED); M, N, K < 2^31 and K*N < 2^40.
 *   - Every dev pointer must be 16-byte aligned.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_ABI_VERSION 1
#define W4A16_LAYOUT_VERSION 2

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_INVALID_ARG = 1,   /* bad shape, NULL/misaligned pointer, bad flags, short buffer */
    W4A16_ERR_UNSUPPORTED = 2,   /* valid request outside what this build implements */
    W4A16_ERR_WORKSPACE = 3,     /* workspace missing or smaller than w4a16_workspace_bytes() */
    W4A16_ERR_HIP = 4            /* the HIP runtime reported an error at launch */
} w4a16_status_t;

/* flags bitfield */
#define W4A16_FP16 0x0u   /* X, scales and Y are IEEE binary16 */
#define W4A16_BF16 0x1u   /* X, scales and Y are bfloat16 */
#define W4A16_ASYM 0x0u   /* zeros: uint8 [K/G][N], values 0..15 */
#define W4A16_SYM  0x2u   /* zero point fixed at 8; the zeros pointer must be NULL */
#define W4A16_FLAGS_MASK 0x3u

/*
 * Plan hints, OR-ed into the flags of w4a16_workspace_bytes and the GEMM
 * calls only (never into a blob's flags): force one kernel variant, for
 * benchmarks and tests.  Give the same flags to w4a16_workspace_bytes and to
 * the GEMM call.  A hint that does not apply to the shape is ignored (the
 * default choice is made).  W4A16_PLAN_PARAM(n), n in 1..255, sets the
 * variant's parameter: the decode or wide kernel's workgroup count, split-K
 * workgroups in units of 8, or the tiled kernel's split count.
 */
#define W4A16_PLAN_DECODE 0x10u   /* streaming kernel for M <= 8, X held in LDS */
#define W4A16_PLAN_SPLITK 0x20u   /* split-K streaming kernel (M <= 32) */
#define W4A16_PLAN_TILED  0x30u   /* LDS-tiled MFMA kernel */
#define W4A16_PLAN_WIDE   0x40u   /* block-streaming kernel for 32 < M <= 128 */
#define W4A16_PLAN_MASK   0x70u
#define W4A16_PLAN_PARAM_SHIFT 8
#define W4A16_PLAN_PARAM(n) (((uint32_t)(n) & 0xFFu) << W4A16_PLAN_PARAM_SHIFT)
#define W4A16_PLAN_BITS   (W4A16_PLAN_MASK | (0xFFu << W4A16_PLAN_PARAM_SHIFT))

/* W4A16_ABI_VERSION of the loaded library. */
int w4a16_abi_version(void);

/* W4A16_LAYOUT_VERSION: the format of the repacked blob.  A blob is only
 * valid for a library with the same layout version. */
int w4a16_layout_version(void);

/* Static, NUL-terminated description of a status code. */
const char *w4a16_status_string(w4a16_status_t status);

/*
 * Size in bytes of the repacked blob for (K, N, G, flags), or 0 if the shape
 * is invalid or unsupported: the algorithmic byte count of the quantized
 * weight, K*N/2 (packed nibbles) + (K/G)*N*2 (scales) + (K/G)*N/2 (zeros,
 * asymmetric only), plus a 16-byte trailer (format tag and feature flags).
 */
size_t w4a16_packed_bytes(int64_t K, int64_t N, int group_size, uint32_t flags);

/*
 * Offline repack of the canonical tensors into the kernels' tile order.
 * Page "量化开销对比", section 6.4: scales and zeros stored in natural group
 * order would cost one scattered global read per weight tile; they are laid
 * next to the weights in consumption order instead.  Not on the per-token path.
 *
 *   qweight  dev, uint32 [K/8][N] row-major; nibble i (bits 4i..4i+3) of word
 *            [r][n] is q[8r+i][n] (least-significant nibble first).
 *   scales   dev, [K/G][N] row-major, fp16 or bf16 per flags.
 *   zeros    dev, uint8 [K/G][N] row-major, values 0..15 (asymmetric);
 *            must be NULL when flags has W4A16_SYM.
 *   packed   dev, output, packed_bytes >= w4a16_packed_bytes(K, N, G, flags).
 * Errors: INVALID_ARG (shape, pointers, flags, SYM/zeros mismatch, short
 * packed_bytes), UNSUPPORTED (N % 128, G), HIP.
 */
w4a16_status_t w4a16_repack(const uint32_t *qweight, const void *scales, const uint8_t *zeros,
                            int64_t K, int64_t N, int group_size, uint32_t flags,
                            void *packed, size_t packed_bytes, void *stream);

/*
 * Exact inverse of w4a16_repack (for round-trip checks and export): writes
 * the canonical qweight, scales and (asymmetric) zeros back from a blob.
 * Same argument rules as w4a16_repack, with the directions reversed.
 */
w4a16_status_t w4a16_unrepack(const void *packed, size_t packed_bytes, uint32_t *qweight,
                              void *scales, uint8_t *zeros, int64_t K, int64_t N,
                              int group_size, uint32_t flags, void *stream);

/*
 * Workspace bytes w4a16_gemm needs for this problem (0 = none).  The value
 * depends on the kernel variant and split-K factor chosen for the shape; it is
 * at most 64 KiB + max(64 * M_pad * N, 262144 * M) bytes, M_pad = M rounded
 * up to 32.  The first 64 KiB always hold the per-tile counters, whatever the
 * shape, so one zero-filled buffer can serve calls of different shapes one
 * after another.
 */
size_t w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int group_size, uint32_t flags);

/*
 * The fused product Y = X . deq(packed), fp32 accumulation, Y rounded to
 * nearest even into the activation dtype.  One pass over the packed weights;
 * dequantized weights exist only in registers.
 *
 *   X          dev, [M][K] row-major, fp16 or bf16 per flags.
 *   packed     dev, blob from w4a16_repack with the same K, N, G and dtype/sym
 *              flags.
 *   flags      the blob's W4A16_FP16|BF16 and ASYM|SYM bits, plus optional
 *              W4A16_PLAN_* hints (the same as given to w4a16_workspace_bytes).
 *   Y          dev, output [M][N] row-major, same dtype as X.  Must not overlap
 *              X, packed or workspace.
 *   workspace  dev, >= w4a16_workspace_bytes(M, N, K, G, flags) bytes (may be
 *              NULL when that is 0).  It must be zero-filled before its first
 *              use; every call leaves its counters zero again, so one
 *              zero-fill suffices for any number of calls.  Calls that share a
 *              workspace must not run concurrently.
 * Kernel choice (W4A16_PLAN_* hints override it): M <= 8 whose activations
 * fit in LDS (M*(2K+16) bytes plus a few KiB, up to 160 KiB) uses the decode
 * kernel (each workgroup streams whole 32-column tiles over all of K, its
 * waves splitting K; when the tiles do not divide evenly over the
 * workgroups, the left-over tiles are split along K and their parts meet in
 * the workspace); other M <= 32 use a split-K streaming
 * kernel (every wave streams an equal contiguous share of the weight chunks;
 * partial sums of a split column block are reduced in a fixed order);
 * 32 < M <= 128 uses a block-streaming kernel (each workgroup streams whole
 * 128-column blocks, its waves 4 tiles x 2 halves of K, the activations
 * staged through LDS; K is split across workgroups through the workspace
 * when there are fewer blocks than CUs); larger M uses an LDS-tiled MFMA
 * kernel.  All reduce in a fixed order, so
 * results are bitwise reproducible run to run, and all use
 * v_mfma_f32_32x32x16.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
w4a16_status_t w4a16_gemm(const void *X, const void *packed, size_t packed_bytes, void *Y,
                          int64_t M, int64_t N, int64_t K, int group_size, uint32_t flags,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Activations and auxiliary-operand combinations of the output epilogue. */
#define W4A16_ACT_NONE 0
#define W4A16_ACT_RELU 1
#define W4A16_ACT_SILU 2
#define W4A16_AUX_ADD 0
#define W4A16_AUX_MUL 1

/*
 * Output epilogue of w4a16_gemm_ex.  Page "量化开销对比", sections 6.2, 6.6
 * and 6.7: the per-channel scale, the bias and a residual or activation are
 * applied to the accumulator inside the GEMM kernel, before its single store,
 * instead of in further launches that re-read Y.  For output element (m, n),
 * with v the fp32 accumulator, in this order and each step optional:
 *   t = v * col_scale[n] + bias[n];   u = act(t);
 *   y = u + aux[m][n]  (aux_op ADD)  or  u * aux[m][n]  (aux_op MUL);
 *   Y[m][n] = y rounded to nearest even into the activation dtype.
 * act: NONE (identity), RELU (max(t, 0)) or SILU (t / (1 + exp(-t))).  All
 * arithmetic is fp32.  The struct is read on the host during the call only.
 *
 *   col_scale  dev, fp32 [N], 4-byte aligned, or NULL (no scale).
 *   bias       dev, [N] in the activation dtype, 2-byte aligned, or NULL.
 *   aux        dev, [M][N] row-major in the activation dtype, 2-byte aligned,
 *              or NULL.  It may be Y itself (an in-place residual add) but
 *              must not otherwise overlap Y.
 *   activation W4A16_ACT_*.   aux_op  W4A16_AUX_* (ignored when aux is NULL).
 */
typedef struct {
    const float *col_scale;
    const void *bias;
    const void *aux;
    int32_t activation;
    int32_t aux_op;
} w4a16_epilogue_t;

/*
 * w4a16_gemm with an output epilogue (see w4a16_epilogue_t): the same
 * arguments, kernels, workspace rules and errors, plus INVALID_ARG for an
 * unknown activation or aux_op, a misaligned epilogue pointer, or an aux that
 * partly overlaps Y.  epilogue == NULL is exactly w4a16_gemm.
 */
w4a16_status_t w4a16_gemm_ex(const void *X, const void *packed, size_t packed_bytes, void *Y,
                             int64_t M, int64_t N, int64_t K, int group_size, uint32_t flags,
                             const w4a16_epilogue_t *epilogue, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * Size of the device scratch array behind w4a16_gemm_noalloc: 16 MiB per GPU
 * the library runs on, held until the process ends.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * w4a16_gemm_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace.  The kernels' scratch (cross-
 * workgroup counters and fp32 partial tiles) lives in a static device array of
 * W4A16_NOALLOC_SCRATCH_BYTES per GPU instead.  The call allocates nothing
 * and frees nothing.  The caller still provides X, packed and Y.
 *   - The first call on a GPU looks up that GPU's array and enqueues one small
 *     kernel on `stream` that zeroes its counter area; every call leaves the
 *     counters zero again.
 *   - Every call on one GPU shares that GPU's array: calls that may overlap in
 *     time on one GPU (different streams, or concurrent host threads) race and
 *     can return wrong results.  Serialize them (one stream, or events).
 * Errors: those of w4a16_gemm_ex, and W4A16_ERR_WORKSPACE when the shape needs
 * more scratch than W4A16_NOALLOC_SCRATCH_BYTES (w4a16_workspace_bytes() tells
 * how much it needs); nothing is launched then.
 */
w4a16_status_t w4a16_gemm_noalloc(const void *X, const void *packed, size_t packed_bytes,
                                  void *Y, int64_t M, int64_t N, int64_t K, int group_size,
                                  uint32_t flags, const w4a16_epilogue_t *epilogue,
                                  void *stream);

/*
 * Test and export aid: writes deq[K][N] row-major (activation dtype) from a
 * blob, using the same device dequantization code as w4a16_gemm.  This is the
 * materialising "route B" the fused path avoids (page "量化开销对比",
 * section 3); it exists for bit-exact checks and for the unfused comparator.
 */
w4a16_status_t w4a16_dequant(const void *packed, size_t packed_bytes, void *W_out,
                             int64_t K, int64_t N, int group_size, uint32_t flags,
                             void *stream);

/*
 * Measurement aid: the practical read ceiling of the weight stream.  Reads
 * `bytes` (a multiple of 1024, buf 16-byte aligned, device memory) once with
 * the split-K kernel's load pattern (balanced contiguous ranges of 1 KiB
 * chunks over 256 workgroups of 8 waves, 16-byte non-temporal loads, two
 * batches of two in flight per wave) and no arithmetic besides an XOR; each
 * of the w4a16_read_probe_out_bytes() / 16 threads writes its XOR (16 bytes)
 * to out, so the XOR of out is the XOR of the buffer.  The GEMM's HBM rate
 * is reported against this ceiling as well as against the 8 TB/s figure.
 * Errors: INVALID_ARG (pointers, alignment, size), HIP.
 */
size_t w4a16_read_probe_out_bytes(void);
w4a16_status_t w4a16_read_probe(const void *buf, size_t bytes, void *out, size_t out_bytes,
                                void *stream);

/*
 * Diagnostic: one v_mfma_f32_32x32x16 (fp16 or bf16 per flags) on A[32][16]
 * and B[16][32] (row-major, dev), loaded into the operand registers the way
 * the GEMM kernels load them, with D[32][32] (fp32, row-major, dev) written
 * back the way the kernels read the accumulators.  D == A.B checks the
 * operand and accumulator layouts the kernels rely on.
 */
w4a16_status_t w4a16_mfma_layout_probe(const void *A, const void *B, float *D, uint32_t flags,
                                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
