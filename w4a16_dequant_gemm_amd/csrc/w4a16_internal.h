// w4a16_internal.h -- launchers and the kernel plan, shared by the C ABI layer
// and the HIP translation units.  Not part of the public interface.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/w4a16.h"
#include "w4a16_layout.h"

namespace w4a16 {

// The split-K and tiled kernels work on column blocks of four tiles.
constexpr int kColBlock = 4 * kTileCols;

enum Variant { VARIANT_SPLITK = 0, VARIANT_TILED = 1, VARIANT_DECODE = 2, VARIANT_WIDE = 3 };

// Split-K kernel geometry, shared by the plan and the kernel.
constexpr int kSplitKWaves = 8;   // waves per workgroup (two per SIMD), one workgroup per CU
constexpr int kSplitKBatch = 4;   // k-steps per batch
constexpr int kTiledStage = 8;    // k-steps per stage of the tiled kernel (128 of K)

// Decode kernel geometry: one workgroup of kDecodeWaves waves per CU; each
// wave keeps kDecodePrefetch bodies of weights in flight, of which the first
// kDecodeEarlyBodies are issued before the activations are written to LDS
// (the rest right after).
constexpr int kDecodeWaves = 8;
constexpr int kDecodeMaxRows = 8;   // M served by the decode kernel (one 8-row group)
constexpr int kDecodePrefetch = 1;
constexpr int kDecodeEarlyBodies = 3;
// Ramp: a wave waits for X and its early bodies before issuing the rest.
constexpr bool kDecodeRamp = false;
// Balance: the two waves of a SIMD keep equal progress (wave priorities).
constexpr bool kDecodeBalance = true;
// fp16, M <= 8: the group scale multiplies the MFMA's product of X and the
// exact (q - z) instead of every weight.
constexpr bool kDecodeScaleAfter = true;
// With fewer tiles than workgroups, the decode kernel keeps tiles whole (no
// split along K) up to this K.
constexpr int64_t kDecodeWholeTileMaxK = 8192;
// LDS budget of the decode kernel (X rows + partial-tile slots), per workgroup.
constexpr size_t kDecodeLdsMax = 160 * 1024;

// Wide kernel (32 < M <= 128): 8 waves = 4 tiles x 2 halves of K per
// workgroup; steps of 256 k for M <= 64, 128 k above.
constexpr int kWideWaves = 8;
constexpr int kWideMinRows = 33;
constexpr int kWideMaxRows = 128;
constexpr int kWidePrefetch = 1;   // weight steps in flight per wave (2 or 3 measured no faster)
inline int wide_step_k(int64_t M) { return M <= 64 ? 256 : 128; }
// LDS bytes of a wide launch: two slots of [2 halves][M rows][2*SK + 16
// bytes] and a flag.
inline size_t wide_lds_bytes(int64_t M, int sk) { return (size_t)4 * M * (2 * sk + 16) + 16; }

// LDS bytes of a decode launch: M rows of X (2K bytes + 16 padding each), the
// [2 items][waves][tiles per item][row groups][64 lanes] fp32x4 partial-tile
// slots, four counters, one progress counter per wave and the zero strip that
// the empty blocks of the MFMA's A operand read (one body of k, 512 bytes).
constexpr int kDecodeZeroBytes = 512;
inline size_t decode_lds_bytes(int64_t M, int64_t K, int tpi, int mb) {
    return (size_t)M * (size_t)(2 * K + 16) + (size_t)2 * kDecodeWaves * tpi * (mb / 8) * 64 * 16 +
           16 + 4 * kDecodeWaves + kDecodeZeroBytes;
}

// How one w4a16_gemm call is executed.  Computed on the host from the shape
// only, so w4a16_workspace_bytes and w4a16_gemm always agree.
struct Plan {
    Variant variant;
    int splits;            // S: workgroups that share one output tile along K
    int steps_per_split;   // k-steps per split (tiled)
    int nbat;              // split-K: batches (kSplitKBatch k-steps) per column block
    int base, rem;         // split-K: wave w owns base (+1 if w < rem) batches
    int mt;                // 32-row MFMA tiles per wave
    int waves;             // waves per workgroup
    int grid_x, grid_y, grid_z;
    int tiles;             // output tiles that own a counter (0 if splits == 1); decode:
                           // the items split along K (their parts: splits)
    int items;             // decode: items of tpi tiles (32 columns each)
    int tpi;               // decode: tiles per item
    size_t tile_floats;    // fp32 partial values per (tile, split)
    size_t counters_bytes; // counter area at the start of the workspace
    size_t workspace;      // total workspace bytes (0 if splits == 1)
};

Plan make_plan(int64_t M, int64_t N, int64_t K, int G, uint32_t flags);

// Output epilogue of one call.  When any step is active every pointer is
// valid device memory: an absent column scale or bias points at the blob and
// an absent aux at Y (read, never used), so the kernels load unconditionally.
constexpr int kActNone = 0;
constexpr int kActRelu = 1;
constexpr int kActSilu = 2;
struct Epilogue {
    const float* col_scale;   // [N]
    const uint16_t* bias;     // [N] in the activation dtype
    const uint16_t* aux;      // [M][N] in the activation dtype
    int has_scale, has_bias, has_aux;
    int act;                  // kAct*
    int aux_mul;              // 0: y = u + aux, 1: y = u * aux
    int any;                  // nonzero when some step is active
};

// Launchers return the hipError_t of the launch (hipGetLastError()).
hipError_t launch_repack(const uint32_t* qweight, const void* scales, const uint8_t* zeros,
                         const Layout& L, bool bf16, void* packed, hipStream_t stream);
hipError_t launch_unrepack(const void* packed, const Layout& L, bool bf16, uint32_t* qweight,
                           void* scales, uint8_t* zeros, hipStream_t stream);
hipError_t launch_dequant(const void* packed, const Layout& L, bool bf16, void* W_out,
                          hipStream_t stream);
hipError_t launch_gemm(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                       bool bf16, const Plan& plan, void* workspace, const Epilogue& ep,
                       hipStream_t stream);
// The four objects of w4a16_gemm.hip, one per (dtype, epilogue) pair.
#define W4A16_DECLARE_GEMM_PART(name)                                                        \
    hipError_t name(const void* X, const void* packed, void* Y, int64_t M, const Layout& L, \
                    const Plan& plan, void* workspace, const Epilogue& ep, hipStream_t stream);
W4A16_DECLARE_GEMM_PART(launch_gemm_f16)
W4A16_DECLARE_GEMM_PART(launch_gemm_f16_ep)
W4A16_DECLARE_GEMM_PART(launch_gemm_bf16)
W4A16_DECLARE_GEMM_PART(launch_gemm_bf16_ep)
#undef W4A16_DECLARE_GEMM_PART
// One validated w4a16_gemm_ex request: the blob layout, the plan and the
// epilogue.  prepare_gemm checks every argument on the host (no HIP call);
// run_gemm launches the kernels with the given workspace (which must hold at
// least plan.workspace bytes when that is nonzero).
struct GemmCall {
    Layout layout;
    Plan plan;
    Epilogue ep;
    bool bf16;
};
w4a16_status_t prepare_gemm(const void* X, const void* packed, size_t packed_bytes, void* Y,
                            int64_t M, int64_t N, int64_t K, int group_size, uint32_t flags,
                            const w4a16_epilogue_t* epilogue, GemmCall* out);
w4a16_status_t run_gemm(const GemmCall& c, const void* X, const void* packed, void* Y, int64_t M,
                        void* workspace, hipStream_t stream);
// Byte size of the counter area at the start of every workspace (the same
// for every shape).
constexpr size_t kCounterBytes = 64 * 1024;
#define W4A16_DECLARE_DECODE_PART(name)                                                       \
    hipError_t name(const void* X, const void* packed, void* Y, int64_t M, const Layout& L, \
                    const Plan& plan, void* workspace, const Epilogue& ep, hipStream_t stream);
W4A16_DECLARE_DECODE_PART(launch_decode_f16)
W4A16_DECLARE_DECODE_PART(launch_decode_f16_ep)
W4A16_DECLARE_DECODE_PART(launch_decode_bf16)
W4A16_DECLARE_DECODE_PART(launch_decode_bf16_ep)
W4A16_DECLARE_DECODE_PART(launch_wide_f16)
W4A16_DECLARE_DECODE_PART(launch_wide_f16_ep)
W4A16_DECLARE_DECODE_PART(launch_wide_bf16)
W4A16_DECLARE_DECODE_PART(launch_wide_bf16_ep)
#undef W4A16_DECLARE_DECODE_PART
// Read-bandwidth probe geometry: one workgroup of 8 waves per CU.
constexpr int kProbeBlocks = 256;
constexpr int kProbeThreads = 512;
hipError_t launch_read_probe(const void* buf, size_t bytes, void* out, hipStream_t stream);
hipError_t launch_mfma_probe(const void* A, const void* B, float* D, bool bf16,
                             hipStream_t stream);

}  // namespace w4a16
