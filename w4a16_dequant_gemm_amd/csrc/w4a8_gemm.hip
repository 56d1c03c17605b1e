// w4a8_gemm.hip -- the W4A8 GEMM kernels for gfx950: 4-bit codes streamed
// from HBM, turned into int8 in registers (one v_pk_mad_u16 and one
// v_xor_b32 per four weights), v_mfma_i32_32x32x32_i8 with int32
// accumulation, the per-row and per-column fp32 scales applied once per
// output after the sum.
//
// Page "W4A8量化计算优化：提升LLM推理效率的关键技术": section 2.1 (the u4 -> i8
// step), section 2.2 (one 128-bit load per lane feeds two matrix
// instructions: here one global_load_dwordx4 per lane holds a tile's B
// operands for two k-steps), section 4.2 (a memory-bound kernel for small
// batches and a compute-bound one above).  Page "量化开销对比", section 1
// (route A: int8 x int8 -> int32 -> scale) and section 2 (symmetric scales
// leave the integer sum as the only term).
//
// Compiled once per output kind (W4A8_TU_OUT = 0 fp16, 1 bf16, 2 int32).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "w4a8_device.h"
#include "w4a8_internal.h"

#ifndef W4A8_TU_OUT
#define W4A8_TU_OUT 0
#endif


namespace w4a8 {

namespace {

template <int OUT>
__device__ __forceinline__ void store_out(void* Y, int64_t idx, int acc, float sxm, float swn) {
    if constexpr (OUT == OUT_I32) {
        ((int*)Y)[idx] = acc;
    } else {
        const float v = ((float)acc * sxm) * swn;
        uint16_t b;
        if constexpr (OUT == OUT_F16)
            b = __builtin_bit_cast(uint16_t, (_Float16)v);
        else
            b = __builtin_bit_cast(uint16_t, (__bf16)v);
        ((uint16_t*)Y)[idx] = b;
    }
}

// Group constants of k-step s of chunk c: G32 -> group 2c + s, else
// group c >> gshift (gshift = log2(G / 64)).
template <bool G32>
__device__ __forceinline__ int group_of(int c, int s, int gshift) {
    return G32 ? 2 * c + s : (c >> gshift);
}

// ---------------------------------------------------------------------------
// Streaming kernel (M <= 64).  Wave w of a workgroup works on tile
// blockIdx.x * (8/KP) + w / KP over part w % KP of the chunks.  Per chunk a
// lane needs its 16 bytes of weights, the group constants and its 16 bytes of
// X per row tile and k-step (X is small and stays in L2); all three ride in a
// ring of P chunks in flight.  Then two k-steps of RT MFMAs.  The KP parts of
// a tile add up in LDS.
//
// BD (M <= 8; the plan uses it up to M = 4): v_mfma_i32_16x16x64_i8 instead
// of the 32x32x32 form, half the matrix-core cycles per k-step, on the same B
// operands.  In the 16x16x64 instruction lane l feeds column l % 16 of
// reduction slot o = l / 16; with
// the B operand of the 32x32 layout (column l % 32, k-half l / 32) slot o
// holds the columns of tile half o % 2 at k-half o / 2.  The A operand is
// block diagonal: row i of the 16 belongs to half (i / 4) % 2, carries X row
// i % 4 + 4 * (i / 8) in the slots of its own half and zeros elsewhere (and
// for X rows >= M), so D row i sums only tile column 16 * ((i / 4) % 2) + j.
// Lane l's four accumulator registers are then its own column l % 32, X rows
// 4 * (l / 32) + r.  The zeros cost nothing: those lanes read X through a
// buffer resource at an offset past its end, which returns zeros.
// ---------------------------------------------------------------------------
constexpr int kStreamDepth = 4;   // chunks in flight per wave
constexpr uint32_t kPastEnd = 0x40000000u;   // > M * K of any stream launch

template <int RT, int KP, bool G32, int OUT, bool BD>
__global__ __launch_bounds__(kW8Waves * 64) void w8_stream_kernel(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ blob,
    void* __restrict__ Y, int M, int N, int K, int gshift, size_t m_off, size_t c_off) {
    static_assert(!BD || RT == 1, "the block-diagonal form holds 8 rows");
    using Acc = typename std::conditional<BD, i32x4, i32x16>::type;
    constexpr int NR = BD ? 4 : 16;   // accumulator registers per lane
    constexpr int CTW = kW8Waves / KP;
    constexpr int P = kStreamDepth;
    extern __shared__ int red[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int part = wave % KP;
    const int ctl = wave / KP;
    const int KC = K / kChunkK;
    const int NG = G32 ? K / 32 : (K / kChunkK) >> gshift;
    const int t = blockIdx.x * CTW + ctl;
    const int per = (KC + KP - 1) / KP;
    const int c0 = min(part * per, KC);
    const int c1 = min(c0 + per, KC);
    const int n = c1 - c0;   // chunks of this wave (0 only if KC < KP, which the plan avoids)

    const u32x4* wsrc = (const u32x4*)blob + (size_t)t * KC * 64 + lane;
    const uint16_t* msrc = (const uint16_t*)(blob + m_off) + (size_t)t * NG * 32 + (lane & 31);
    const int8_t* xsrc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
        xsrc[r] = X + (size_t)min(32 * r + (lane & 31), M - 1) * K + 16 * (lane >> 5);
    // BD: lane l is A row i = l % 16 of slot l / 16; its X row, or past the end
    const __amdgpu_buffer_rsrc_t xrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, BD ? M * K : 0, kRawBufferWord3);
    uint32_t xoff = 0;
    if constexpr (BD) {
        const int ai = lane & 15;
        const int axr = (ai & 3) + 4 * (ai >> 3);
        const bool alive = ((ai >> 2) & 1) == ((lane >> 4) & 1) && axr < M;
        xoff = alive ? (uint32_t)axr * (uint32_t)K + 16u * (uint32_t)(lane >> 5) : kPastEnd;
    }

    Acc acc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int i = 0; i < NR; ++i) acc[r][i] = 0;

    // Ring of P chunks in flight: slot i holds chunk c0 + base + i -- its
    // codes, its group constants and its X operands.  Slot i is refilled with
    // chunk c + P as soon as chunk c has been copied out of it.
    u32x4 wb[P];
    i32x4 xb[P][RT][2];
    uint32_t mb[P][2];
    auto fill = [&](int i, int c) __attribute__((always_inline)) {
        wb[i] = __builtin_nontemporal_load(wsrc + (size_t)c * 64);
        if constexpr (BD) {
            const uint32_t o = xoff + (uint32_t)c * kChunkK;
            xb[i][0][0] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, o, 0, 0));
            xb[i][0][1] =
                __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, o + 32, 0, 0));
        } else {
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                xb[i][r][0] = *(const i32x4*)(xsrc[r] + (size_t)c * kChunkK);
                xb[i][r][1] = *(const i32x4*)(xsrc[r] + (size_t)c * kChunkK + 32);
            }
        }
        mb[i][0] = msrc[(size_t)group_of<G32>(c, 0, gshift) * 32];
        mb[i][1] = G32 ? msrc[(size_t)group_of<G32>(c, 1, gshift) * 32] : 0u;
    };
#pragma unroll
    for (int i = 0; i < P; ++i) fill(i, min(c0 + i, c1 - 1));

    for (int base = 0; base < n; base += P) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int c = c0 + base + i;
            if (base + i < n) {
                const u32x4 w = wb[i];
                i32x4 xa[RT][2];
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    xa[r][0] = xb[i][r][0];
                    xa[r][1] = xb[i][r][1];
                }
                const uint32_t m0 = mb[i][0];
                const uint32_t m1 = G32 ? mb[i][1] : m0;
                fill(i, min(c + P, c1 - 1));
                const i32x4 b0 = operand_b(w[0], w[1], group_w8(m0));
                const i32x4 b1 = operand_b(w[2], w[3], group_w8(m1));
                if constexpr (BD) {
                    acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[0][0], b0, acc[0], 0, 0, 0);
                    acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[0][1], b1, acc[0], 0, 0, 0);
                } else {
#pragma unroll
                    for (int r = 0; r < RT; ++r)
                        acc[r] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa[r][0], b0, acc[r], 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < RT; ++r)
                        acc[r] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xa[r][1], b1, acc[r], 0, 0, 0);
                }
            }
        }
    }

    if constexpr (KP > 1) {
        // parts 1..KP-1 leave their sums in LDS; part 0 adds them
        if (part > 0) {
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int i = 0; i < NR; ++i)
                    red[((((part - 1) * CTW + ctl) * RT + r) * NR + i) * 64 + lane] = acc[r][i];
        }
        __syncthreads();
        if (part > 0) return;
#pragma unroll 1
        for (int p = 1; p < KP; ++p)
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int i = 0; i < NR; ++i)
                    acc[r][i] += red[((((p - 1) * CTW + ctl) * RT + r) * NR + i) * 64 + lane];
    }

    const int col = t * kTileCols + (lane & 31);
    const float swn = OUT == OUT_I32 ? 0.0f : ((const float*)(blob + c_off))[col];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int row = BD ? 4 * (lane >> 5) + i : 32 * r + acc_row_w8(i, lane);
            if (row < M) store_out<OUT>(Y, (int64_t)row * N + col, acc[r][i],
                                        OUT == OUT_I32 ? 0.0f : sx[row], swn);
        }
}

// ---------------------------------------------------------------------------
// Tiled kernel (M > 64).  A workgroup owns BM = WM*RT*32 rows and BN =
// WN*CT*32 columns over all of K.  Per chunk (64 of K) the workgroup copies
// its BM x 64 bytes of X into one slot of a two-slot LDS ring (rows padded to
// 80 bytes: the 16-byte operand reads of 16 consecutive rows then cover all
// 64 banks once).  Each wave keeps its CT tiles' codes and group constants
// PD chunks ahead in a register ring, and turns chunk c+1's codes into int8
// B operands while the MFMAs of chunk c run (the two sets of operands are
// independent, so the VALU work hides under the matrix pipe).  One barrier
// per chunk.  Tiles are ordered so that the workgroups resident on one XCD at
// a time share rows of X and columns of W in that XCD's L2.
// ---------------------------------------------------------------------------
template <int RT, int CT, int WM, int WN, int PD, int XD, bool G32, int OUT>
__global__ __launch_bounds__(kW8Waves * 64) void w8_tiled_kernel(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ blob,
    void* __restrict__ Y, int M, int N, int K, int gshift, size_t m_off, size_t c_off, int nbm,
    int nbn) {
    static_assert(WM * WN == kW8Waves, "eight waves");
    // the ring must divide the chunk count: KC is a multiple of 4, and of 8
    // where the launcher picks PD = 8
    static_assert(PD == 2 || PD == 4 || PD == 8, "ring depth");
    static_assert(XD == 1 || XD == 2, "X is loaded one or two chunks ahead");
    constexpr int BM = WM * RT * 32;
    constexpr int BN = WN * CT * 32;
    constexpr int RB = kTiledRowBytes;
    constexpr int SLOT = BM * RB;
    constexpr int PIECES = BM * 4 / (kW8Waves * 64);   // 16-byte X pieces per thread and chunk
    static_assert(PIECES >= 1 && BM * 4 == PIECES * kW8Waves * 64, "X staging");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int KC = K / kChunkK;
    const int NT = N / kTileCols;
    const int NG = G32 ? K / 32 : KC >> gshift;

    // task -> (row block, column block): first spread over the 8 XCDs in
    // contiguous runs (dispatch goes round-robin over XCDs), then groups of 4
    // row blocks walked column block by column block.
    const int T = nbm * nbn;
    int task = blockIdx.x;
    if (T % 8 == 0) task = (blockIdx.x % 8) * (T / 8) + blockIdx.x / 8;
    constexpr int GM = 4;
    const int group = task / (GM * nbn);
    const int first_m = group * GM;
    const int gsz = min(nbm - first_m, GM);
    const int in_group = task % (GM * nbn);
    const int mb = first_m + in_group % gsz;
    const int nb = in_group / gsz;
    const int m0 = mb * BM;

    int tile[CT];
    bool tile_ok[CT];
    const u32x4* wsrc[CT];
    const uint16_t* msrc[CT];
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        const int tt = nb * (BN / 32) + wn * CT + j;
        tile_ok[j] = tt < NT;
        tile[j] = min(tt, NT - 1);
        wsrc[j] = (const u32x4*)blob + (size_t)tile[j] * KC * 64 + lane;
        msrc[j] = (const uint16_t*)(blob + m_off) + (size_t)tile[j] * NG * 32 + (lane & 31);
    }

    // X staging: piece p = tid + 512*i is 16-byte quarter p%4 of a row.
    const int8_t* xg[PIECES];
    int xl[PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
        // 16 consecutive pieces: quarters 0..3 of rows b, b+4, b+8, b+12 (an
        // 80-byte row stride puts those at dword offsets 0, 16, 32, 48 mod 64,
        // so the 16-byte LDS writes of 16 lanes meet all 64 banks once)
        const int p = tid + kW8Waves * 64 * i;
        const int row = ((p >> 6) << 4) + (((p >> 2) & 3) << 2) + ((p >> 4) & 3);
        xg[i] = X + (size_t)min(m0 + row, M - 1) * K + 16 * (p & 3);
        xl[i] = row * RB + 16 * (p & 3);
    }
    // A operand of row tile r, k-step s: row wm*RT*32 + 32r + lane%32, bytes 32s + 16*(lane/32)
    const int arow = (wm * RT * 32 + (lane & 31)) * RB + 16 * (lane >> 5);

    i32x16 acc[RT][CT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < CT; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[r][j][i] = 0;

    // ring slot s holds the codes and group constants of the chunk c with c % PD == s
    u32x4 wb[PD][CT];
    uint32_t mt[PD][CT][2];
    auto fill = [&](int s, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            wb[s][j] = __builtin_nontemporal_load(wsrc[j] + (size_t)c * 64);
            mt[s][j][0] = msrc[j][(size_t)group_of<G32>(c, 0, gshift) * 32];
            mt[s][j][1] = G32 ? msrc[j][(size_t)group_of<G32>(c, 1, gshift) * 32] : 0u;
        }
    };
    auto operands = [&](int s, i32x4 (&bq)[CT][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            const u32x4 w = wb[s][j];
            bq[j][0] = operand_b(w[0], w[1], group_w8(mt[s][j][0]));
            bq[j][1] = operand_b(w[2], w[3], group_w8(G32 ? mt[s][j][1] : mt[s][j][0]));
        }
    };

    // prologue: X of chunk 0 into LDS slot 0, the ring filled, B of chunk 0 made
    // X ring (XD = 2): xr[c % 2] receives chunk c + 2 while chunk c + 1 waits in the other
    i32x4 xr[XD][PIECES];
    {
#pragma unroll
        for (int i = 0; i < PIECES; ++i) xr[0][i] = *(const i32x4*)xg[i];
        if constexpr (XD == 2) {
#pragma unroll
            for (int i = 0; i < PIECES; ++i)
                xr[1][i] = *(const i32x4*)(xg[i] + (size_t)min(1, KC - 1) * kChunkK);
        }
#pragma unroll
        for (int s = 0; s < PD; ++s) fill(s, min(s, KC - 1));
#pragma unroll
        for (int i = 0; i < PIECES; ++i) *(i32x4*)(lds + xl[i]) = xr[0][i];
    }
    i32x4 bqa[CT][2], bqb[CT][2];
    operands(0, bqa);
    fill(0, min(PD, KC - 1));
    __syncthreads();

    for (int cb = 0; cb < KC; cb += PD) {   // KC is a multiple of PD
#pragma unroll
        for (int q = 0; q < PD; ++q) {
            const int c = cb + q;
            // chunk c's B operands are in bqa (q even) or bqb (q odd); chunk c+1's go to the other
            i32x4 (&cur)[CT][2] = (q & 1) ? bqb : bqa;
            i32x4 (&nxt)[CT][2] = (q & 1) ? bqa : bqb;
            const uint8_t* slot = lds + (q & 1) * SLOT;   // chunk c lives in LDS slot c % 2
            // X of chunk c + XD (clamped; the last ones are harmless repeats)
            i32x4 (&xin)[PIECES] = xr[XD == 2 ? (q & 1) : 0];
            const int cn = min(c + XD, KC - 1);
#pragma unroll
            for (int i = 0; i < PIECES; ++i) xin[i] = *(const i32x4*)(xg[i] + (size_t)cn * kChunkK);
            // B of chunk c+1, then its ring slot refilled with chunk c+1+PD
            const int sn = (q + 1) % PD;
            operands(sn, nxt);
            fill(sn, min(c + 1 + PD, KC - 1));
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                i32x4 a[RT];
#pragma unroll
                for (int r = 0; r < RT; ++r)
                    a[r] = *(const i32x4*)(slot + arow + r * 32 * RB + 32 * s);
#pragma unroll
                for (int r = 0; r < RT; ++r)
#pragma unroll
                    for (int j = 0; j < CT; ++j)
                        acc[r][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[r], cur[j][s],
                                                                          acc[r][j], 0, 0, 0);
            }
            // LDS slot (c+1) % 2 was last read in chunk c-1, before the previous barrier
            uint8_t* next = lds + (1 - (q & 1)) * SLOT;
            i32x4 (&xout)[PIECES] = xr[XD == 2 ? 1 - (q & 1) : 0];   // chunk c + 1
#pragma unroll
            for (int i = 0; i < PIECES; ++i) *(i32x4*)(next + xl[i]) = xout[i];
            __syncthreads();
        }
    }

    const float* colscale = (const float*)(blob + c_off);
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        if (!tile_ok[j]) continue;
        const int col = tile[j] * kTileCols + (lane & 31);
        const float swn = OUT == OUT_I32 ? 0.0f : colscale[col];
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + wm * RT * 32 + 32 * r + acc_row_w8(i, lane);
                if (row < M) store_out<OUT>(Y, (int64_t)row * N + col, acc[r][j][i],
                                            OUT == OUT_I32 ? 0.0f : sx[row], swn);
            }
    }
}

// The tiled kernel with two chunks (128 of K) per LDS stage: half the
// barriers, each covering 2 x RT x CT x 2 MFMAs per wave.  Rows of 128 bytes
// of X padded to 144; the 16-byte writes of 16 lanes go to rows b and b+8
// (144-byte stride: 32 dwords apart), so they meet every bank once; the
// operand reads of 16 consecutive rows do too (36-dword stride).  X one stage
// ahead through registers, codes and group constants PD chunks ahead.
template <int RT, int CT, int WM, int WN, int PD, bool G32, int OUT>
__global__ __launch_bounds__(kW8Waves * 64) void w8_tiled2_kernel(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ blob,
    void* __restrict__ Y, int M, int N, int K, int gshift, size_t m_off, size_t c_off, int nbm,
    int nbn) {
    static_assert(WM * WN == kW8Waves, "eight waves");
    static_assert(4 % PD == 0, "the ring divides two stages");
    constexpr int CK = 2;                               // chunks per LDS stage
    constexpr int BM = WM * RT * 32;
    constexpr int BN = WN * CT * 32;
    constexpr int RB = 64 * CK + 16;
    constexpr int SLOT = BM * RB;
    constexpr int PIECES = BM * 4 * CK / (kW8Waves * 64);
    static_assert(PIECES >= 1 && BM * 4 * CK == PIECES * kW8Waves * 64, "X staging");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int KC = K / kChunkK;
    const int NT = N / kTileCols;
    const int NG = G32 ? K / 32 : KC >> gshift;

    const int T = nbm * nbn;
    int task = blockIdx.x;
    if (T % 8 == 0) task = (blockIdx.x % 8) * (T / 8) + blockIdx.x / 8;
    constexpr int GM = 4;
    const int group = task / (GM * nbn);
    const int first_m = group * GM;
    const int gsz = min(nbm - first_m, GM);
    const int in_group = task % (GM * nbn);
    const int mb = first_m + in_group % gsz;
    const int nb = in_group / gsz;
    const int m0 = mb * BM;

    int tile[CT];
    bool tile_ok[CT];
    const u32x4* wsrc[CT];
    const uint16_t* msrc[CT];
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        const int tt = nb * (BN / 32) + wn * CT + j;
        tile_ok[j] = tt < NT;
        tile[j] = min(tt, NT - 1);
        wsrc[j] = (const u32x4*)blob + (size_t)tile[j] * KC * 64 + lane;
        msrc[j] = (const uint16_t*)(blob + m_off) + (size_t)tile[j] * NG * 32 + (lane & 31);
    }

    // X staging: piece p covers 16-byte piece p%8 of a row: 16 consecutive
    // pieces are rows b and b+8 of a group of 16 rows
    const int8_t* xg[PIECES];
    int xl[PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
        const int p = tid + kW8Waves * 64 * i;
        const int q = p & 7;
        const int row = ((p >> 7) << 4) + (((p >> 3) & 1) << 3) + ((p >> 4) & 7);
        xg[i] = X + (size_t)min(m0 + row, M - 1) * K + 16 * q;
        xl[i] = row * RB + 16 * q;
    }
    const int arow = (wm * RT * 32 + (lane & 31)) * RB + 16 * (lane >> 5);

    i32x16 acc[RT][CT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < CT; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[r][j][i] = 0;

    u32x4 wb[PD][CT];
    uint32_t mt[PD][CT][2];
    auto fill = [&](int s, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            wb[s][j] = __builtin_nontemporal_load(wsrc[j] + (size_t)c * 64);
            mt[s][j][0] = msrc[j][(size_t)group_of<G32>(c, 0, gshift) * 32];
            mt[s][j][1] = G32 ? msrc[j][(size_t)group_of<G32>(c, 1, gshift) * 32] : 0u;
        }
    };
    auto operands = [&](int s, i32x4 (&bq)[CT][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            const u32x4 w = wb[s][j];
            bq[j][0] = operand_b(w[0], w[1], group_w8(mt[s][j][0]));
            bq[j][1] = operand_b(w[2], w[3], group_w8(G32 ? mt[s][j][1] : mt[s][j][0]));
        }
    };

    const int NS = KC / CK;   // stages (KC is a multiple of 4)
    i32x4 xr[PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) xr[i] = *(const i32x4*)xg[i];
#pragma unroll
    for (int s = 0; s < PD; ++s) fill(s, min(s, KC - 1));
#pragma unroll
    for (int i = 0; i < PIECES; ++i) *(i32x4*)(lds + xl[i]) = xr[i];
    i32x4 bqa[CT][2], bqb[CT][2];
    operands(0, bqa);
    fill(0, min(PD, KC - 1));
    __syncthreads();

    for (int st0 = 0; st0 < NS; st0 += 2) {   // two stages per turn (NS is even)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            const int st = st0 + sp;
            const uint8_t* slot = lds + sp * SLOT;   // stage st lives in LDS slot st % 2
            const int sn = min(st + 1, NS - 1);
#pragma unroll
            for (int i = 0; i < PIECES; ++i)
                xr[i] = *(const i32x4*)(xg[i] + (size_t)sn * (kChunkK * CK));
#pragma unroll
            for (int j2 = 0; j2 < CK; ++j2) {
                const int q = sp * CK + j2;            // chunk index inside the turn (static)
                const int c = st * CK + j2;
                i32x4 (&cur)[CT][2] = (q & 1) ? bqb : bqa;
                i32x4 (&nxt)[CT][2] = (q & 1) ? bqa : bqb;
                const int sl = (q + 1) % PD;           // ring slot of chunk c+1
                operands(sl, nxt);
                fill(sl, min(c + 1 + PD, KC - 1));
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    i32x4 a[RT];
#pragma unroll
                    for (int r = 0; r < RT; ++r)
                        a[r] = *(const i32x4*)(slot + arow + r * 32 * RB + j2 * kChunkK + 32 * s);
#pragma unroll
                    for (int r = 0; r < RT; ++r)
#pragma unroll
                        for (int j = 0; j < CT; ++j)
                            acc[r][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[r], cur[j][s],
                                                                              acc[r][j], 0, 0, 0);
                }
            }
            // LDS slot (st+1) % 2 was last read in stage st-1, before the previous barrier
            uint8_t* next = lds + (1 - sp) * SLOT;
#pragma unroll
            for (int i = 0; i < PIECES; ++i) *(i32x4*)(next + xl[i]) = xr[i];
            __syncthreads();
        }
    }

    const float* colscale = (const float*)(blob + c_off);
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        if (!tile_ok[j]) continue;
        const int col = tile[j] * kTileCols + (lane & 31);
        const float swn = OUT == OUT_I32 ? 0.0f : colscale[col];
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + wm * RT * 32 + 32 * r + acc_row_w8(i, lane);
                if (row < M) store_out<OUT>(Y, (int64_t)row * N + col, acc[r][j][i],
                                            OUT == OUT_I32 ? 0.0f : sx[row], swn);
            }
    }
}

// The 256 x 256 tiled kernel with the int8 weights made once per workgroup
// (page "W4A8量化计算优化", section 3.1: the weights of a tile are loaded and
// prepared once for all the matrix work on them).  Per stage of two chunks
// each of the 8 waves turns one column tile's codes into int8 B operands and
// writes them to LDS in the operand order (lane l's 16 bytes of tile t, chunk
// j, k-step s at ((t*2 + j)*2 + s)*1024 + 16*l), beside the stage's X rows;
// after the barrier every wave reads the B operands of its CT tiles from LDS.
// The dequant work per wave halves against the kernels above (there, the WM
// waves sharing a column tile each make its operands), at the cost of 4 KiB
// of LDS writes and 8 KiB of reads per wave and stage.  Stage s+1's operands
// and X rows are made while stage s's MFMAs run; one barrier per stage.
template <int RT, int CT, int WM, int WN, int PD, bool G32, int OUT>
__global__ __launch_bounds__(kW8Waves * 64) void w8_coop_kernel(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ blob,
    void* __restrict__ Y, int M, int N, int K, int gshift, size_t m_off, size_t c_off, int nbm,
    int nbn) {
    static_assert(WM * WN == kW8Waves && WN * CT == kW8Waves, "eight waves, eight column tiles");
    static_assert(4 % PD == 0, "the ring divides two stages");
    constexpr int CK = 2;                               // chunks per LDS stage
    constexpr int NTB = WN * CT;                        // column tiles per workgroup (8)
    constexpr int BM = WM * RT * 32;
    constexpr int RB = 64 * CK + 16;
    constexpr int XBYTES = BM * RB;
    constexpr int BBYTES = NTB * CK * 2 * 1024;         // [tile][chunk][k-step][lane] 16 B
    constexpr int SLOT = XBYTES + BBYTES;
    constexpr int PIECES = BM * 4 * CK / (kW8Waves * 64);
    static_assert(PIECES >= 1 && BM * 4 * CK == PIECES * kW8Waves * 64, "X staging");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int KC = K / kChunkK;
    const int NT = N / kTileCols;
    const int NG = G32 ? K / 32 : KC >> gshift;

    const int T = nbm * nbn;
    int task = blockIdx.x;
    if (T % 8 == 0) task = (blockIdx.x % 8) * (T / 8) + blockIdx.x / 8;
    constexpr int GM = 4;
    const int group = task / (GM * nbn);
    const int first_m = group * GM;
    const int gsz = min(nbm - first_m, GM);
    const int in_group = task % (GM * nbn);
    const int mb = first_m + in_group % gsz;
    const int nb = in_group / gsz;
    const int m0 = mb * BM;

    // the tile this wave prepares: workgroup tile `wave`
    const int ptile = min(nb * NTB + wave, NT - 1);
    const u32x4* wsrc = (const u32x4*)blob + (size_t)ptile * KC * 64 + lane;
    const uint16_t* msrc = (const uint16_t*)(blob + m_off) + (size_t)ptile * NG * 32 + (lane & 31);
    const int boff_w = wave * (CK * 2 * 1024) + lane * 16;   // its operands inside a slot's B area

    const int8_t* xg[PIECES];
    int xl[PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
        const int p = tid + kW8Waves * 64 * i;
        const int q = p & 7;
        const int row = ((p >> 7) << 4) + (((p >> 3) & 1) << 3) + ((p >> 4) & 7);
        xg[i] = X + (size_t)min(m0 + row, M - 1) * K + 16 * q;
        xl[i] = row * RB + 16 * q;
    }
    const int arow = (wm * RT * 32 + (lane & 31)) * RB + 16 * (lane >> 5);

    i32x16 acc[RT][CT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < CT; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[r][j][i] = 0;

    // ring slot s: codes and group constants of this wave's tile for the chunk c with c % PD == s
    u32x4 wb[PD];
    uint32_t mt[PD][2];
    auto fill = [&](int s, int c) __attribute__((always_inline)) {
        wb[s] = __builtin_nontemporal_load(wsrc + (size_t)c * 64);
        mt[s][0] = msrc[(size_t)group_of<G32>(c, 0, gshift) * 32];
        mt[s][1] = G32 ? msrc[(size_t)group_of<G32>(c, 1, gshift) * 32] : 0u;
    };
    // the operands of chunk c (ring slot s) into chunk position j of an LDS slot's B area
    auto produce = [&](uint8_t* bslot, int s, int j) __attribute__((always_inline)) {
        const u32x4 w = wb[s];
        const i32x4 b0 = operand_b(w[0], w[1], group_w8(mt[s][0]));
        const i32x4 b1 = operand_b(w[2], w[3], group_w8(G32 ? mt[s][1] : mt[s][0]));
        *(i32x4*)(bslot + boff_w + (j * 2 + 0) * 1024) = b0;
        *(i32x4*)(bslot + boff_w + (j * 2 + 1) * 1024) = b1;
    };

    const int NS = KC / CK;   // stages (KC is a multiple of 4)
    i32x4 xr[PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) xr[i] = *(const i32x4*)xg[i];
#pragma unroll
    for (int s = 0; s < PD; ++s) fill(s, min(s, KC - 1));
#pragma unroll
    for (int i = 0; i < PIECES; ++i) *(i32x4*)(lds + xl[i]) = xr[i];
    // stage 0's operands (chunks 0 and 1, ring slots 0 and 1), then their slots refilled
#pragma unroll
    for (int j = 0; j < CK; ++j) {
        produce(lds + XBYTES, j % PD, j);
        fill(j % PD, min(j + PD, KC - 1));
    }
    __syncthreads();

    for (int st0 = 0; st0 < NS; st0 += 2) {   // two stages per turn (NS is even)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            const int st = st0 + sp;
            const uint8_t* slot = lds + sp * SLOT;      // stage st lives in LDS slot st % 2
            uint8_t* next = lds + (1 - sp) * SLOT;     // read in stage st-1, before the previous barrier
            const int sn = min(st + 1, NS - 1);
#pragma unroll
            for (int i = 0; i < PIECES; ++i)
                xr[i] = *(const i32x4*)(xg[i] + (size_t)sn * (kChunkK * CK));
#pragma unroll
            for (int j2 = 0; j2 < CK; ++j2) {
                // this wave's share of stage st+1: chunk (st+1)*CK + j2, ring slot ((sp+1)*CK + j2) % PD
                const int cq = ((sp + 1) * CK + j2) % PD;
                produce(next + XBYTES, cq, j2);
                fill(cq, min((st + 1) * CK + j2 + PD, KC - 1));
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    i32x4 a[RT];
                    i32x4 bq[CT];
#pragma unroll
                    for (int r = 0; r < RT; ++r)
                        a[r] = *(const i32x4*)(slot + arow + r * 32 * RB + j2 * kChunkK + 32 * s);
#pragma unroll
                    for (int j = 0; j < CT; ++j)
                        bq[j] = *(const i32x4*)(slot + XBYTES + (wn * CT + j) * (CK * 2 * 1024) +
                                               (j2 * 2 + s) * 1024 + lane * 16);
#pragma unroll
                    for (int r = 0; r < RT; ++r)
#pragma unroll
                        for (int j = 0; j < CT; ++j)
                            acc[r][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[r], bq[j],
                                                                              acc[r][j], 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < PIECES; ++i) *(i32x4*)(next + xl[i]) = xr[i];
            __syncthreads();
        }
    }

    const float* colscale = (const float*)(blob + c_off);
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        const int tt = nb * NTB + wn * CT + j;
        if (tt >= NT) continue;
        const int col = tt * kTileCols + (lane & 31);
        const float swn = OUT == OUT_I32 ? 0.0f : colscale[col];
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + wm * RT * 32 + 32 * r + acc_row_w8(i, lane);
                if (row < M) store_out<OUT>(Y, (int64_t)row * N + col, acc[r][j][i],
                                            OUT == OUT_I32 ? 0.0f : sx[row], swn);
            }
    }
}

template <int RT, int KP, bool G32>
hipError_t launch_stream_t(const int8_t* xq, const float* sx, const void* packed, void* Y,
                           int64_t M, const LayoutW8& L, const PlanW8& plan, int gshift,
                           hipStream_t stream) {
    if constexpr (RT == 1) {
        if (plan.bd) {
            if (M > 8) return hipErrorInvalidValue;   // the plan never asks for it
            w8_stream_kernel<1, KP, G32, W4A8_TU_OUT, true>
                <<<plan.grid, kW8Waves * 64, plan.lds, stream>>>(xq, sx, (const uint8_t*)packed, Y,
                                                                 (int)M, (int)L.N, (int)L.K, gshift,
                                                                 L.m_off, L.c_off);
            return hipGetLastError();
        }
    }
    w8_stream_kernel<RT, KP, G32, W4A8_TU_OUT, false><<<plan.grid, kW8Waves * 64, plan.lds, stream>>>(
        xq, sx, (const uint8_t*)packed, Y, (int)M, (int)L.N, (int)L.K, gshift, L.m_off, L.c_off);
    return hipGetLastError();
}

template <int RT, bool G32>
hipError_t launch_stream_kp(const int8_t* xq, const float* sx, const void* packed, void* Y,
                            int64_t M, const LayoutW8& L, const PlanW8& plan, int gshift,
                            hipStream_t stream) {
    switch (plan.kp) {
        case 2: return launch_stream_t<RT, 2, G32>(xq, sx, packed, Y, M, L, plan, gshift, stream);
        case 4: return launch_stream_t<RT, 4, G32>(xq, sx, packed, Y, M, L, plan, gshift, stream);
        default: return launch_stream_t<RT, 8, G32>(xq, sx, packed, Y, M, L, plan, gshift, stream);
    }
}

template <bool G32>
hipError_t launch_g(const int8_t* xq, const float* sx, const void* packed, void* Y, int64_t M,
                    const LayoutW8& L, const PlanW8& plan, int gshift, hipStream_t stream) {
    const uint8_t* b = (const uint8_t*)packed;
    if (plan.variant == W8_STREAM) {
        if (plan.rt == 1)
            return launch_stream_kp<1, G32>(xq, sx, packed, Y, M, L, plan, gshift, stream);
        return launch_stream_kp<2, G32>(xq, sx, packed, Y, M, L, plan, gshift, stream);
    }
    if (plan.cfg == 0)
        w8_tiled_kernel<4, 2, 2, 4, 2, (G32 ? 1 : 2), G32, W4A8_TU_OUT>
            <<<plan.grid, kW8Waves * 64, plan.lds, stream>>>(xq, sx, b, Y, (int)M, (int)L.N,
                                                             (int)L.K, gshift, L.m_off, L.c_off,
                                                             plan.nbm, plan.nbn);
    else if (plan.cfg == 1 && L.KC % 8 == 0)   // codes 8 chunks ahead where the ring divides K
        w8_tiled_kernel<2, 1, 2, 4, 8, 2, G32, W4A8_TU_OUT>
            <<<plan.grid, kW8Waves * 64, plan.lds, stream>>>(xq, sx, b, Y, (int)M, (int)L.N,
                                                             (int)L.K, gshift, L.m_off, L.c_off,
                                                             plan.nbm, plan.nbn);
    else if (plan.cfg == 1)
        w8_tiled_kernel<2, 1, 2, 4, 4, 2, G32, W4A8_TU_OUT>
            <<<plan.grid, kW8Waves * 64, plan.lds, stream>>>(xq, sx, b, Y, (int)M, (int)L.N,
                                                             (int)L.K, gshift, L.m_off, L.c_off,
                                                             plan.nbm, plan.nbn);
    else if (plan.cfg == 4)
        w8_coop_kernel<4, 2, 2, 4, 4, G32, W4A8_TU_OUT>
            <<<plan.grid, kW8Waves * 64, plan.lds, stream>>>(xq, sx, b, Y, (int)M, (int)L.N,
                                                             (int)L.K, gshift, L.m_off, L.c_off,
                                                             plan.nbm, plan.nbn);
    else if (plan.cfg == 3)
        w8_tiled2_kernel<4, 2, 2, 4, 2, G32, W4A8_TU_OUT>
            <<<plan.grid, kW8Waves * 64, plan.lds, stream>>>(xq, sx, b, Y, (int)M, (int)L.N,
                                                             (int)L.K, gshift, L.m_off, L.c_off,
                                                             plan.nbm, plan.nbn);
    else
        w8_tiled_kernel<4, 1, 2, 4, 4, 2, G32, W4A8_TU_OUT>
            <<<plan.grid, kW8Waves * 64, plan.lds, stream>>>(xq, sx, b, Y, (int)M, (int)L.N,
                                                             (int)L.K, gshift, L.m_off, L.c_off,
                                                             plan.nbm, plan.nbn);
    return hipGetLastError();
}

hipError_t launch_part(const int8_t* xq, const float* sx, const void* packed, void* Y, int64_t M,
                       const LayoutW8& L, const PlanW8& plan, hipStream_t stream) {
    if (L.G == 32) return launch_g<true>(xq, sx, packed, Y, M, L, plan, 0, stream);
    const int gshift = L.G == 64 ? 0 : 1;
    return launch_g<false>(xq, sx, packed, Y, M, L, plan, gshift, stream);
}

}  // namespace

#if W4A8_TU_OUT == 0
#define W4A8_PART_NAME launch_w8_gemm_f16
#elif W4A8_TU_OUT == 1
#define W4A8_PART_NAME launch_w8_gemm_bf16
#else
#define W4A8_PART_NAME launch_w8_gemm_i32
#endif

hipError_t W4A8_PART_NAME(const int8_t* xq, const float* sx, const void* packed, void* Y,
                          int64_t M, const LayoutW8& L, const PlanW8& plan, hipStream_t stream) {
    return launch_part(xq, sx, packed, Y, M, L, plan, stream);
}

}  // namespace w4a8
