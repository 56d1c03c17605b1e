// mx_gemm.hip -- the MXFP4 GEMM kernels for gfx950: E2M1 weight codes and
// E4M3 activations go straight into v_mfma_scale_f32_32x32x64_f8f6f4 with
// their E8M0 block scales (one scale byte per lane and operand), fp32
// accumulation, one rounding to the output dtype.
//
// Page "量化开销对比" (laojiahuo2003.github.io), section 3, closing paragraph
// (hardware block scales of 32 bring 4-bit weights back to route A: no
// dequantisation in the kernel) and section 1 (route A).  The operand layouts
// are described in mx_internal.h.
//
// Compiled once per output dtype (MXFP4_TU_BF16 = 0 fp16, 1 bf16).
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "mx_internal.h"

#ifndef MXFP4_TU_BF16
#define MXFP4_TU_BF16 0
#endif

namespace mxfp4 {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int acc_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

template <bool BF16>
__device__ __forceinline__ void store_out(void* Y, int64_t idx, float v) {
    uint16_t b;
    if constexpr (BF16)
        b = __builtin_bit_cast(uint16_t, (__bf16)v);
    else
        b = __builtin_bit_cast(uint16_t, (_Float16)v);
    ((uint16_t*)Y)[idx] = b;
}

// A operand (32 E4M3 bytes) from its two 16-byte halves; B operand (32 E2M1
// codes in 16 bytes, the upper half unused).
__device__ __forceinline__ i32x8 cat(i32x4 lo, i32x4 hi) {
    i32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

__device__ __forceinline__ i32x8 widen(u32x4 w) {
    i32x8 r;
    r[0] = (int)w[0]; r[1] = (int)w[1]; r[2] = (int)w[2]; r[3] = (int)w[3];
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    return r;
}

// A: E4M3 (format 0), B: E2M1 (format 4); the scales are byte SA of sa and
// byte SB of sb (the instruction's byte select).
template <int SA, int SB>
__device__ __forceinline__ f32x16 mma(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, SA, sa, SB, sb);
}

// The same on the 16x16x128 form.
template <int SA, int SB>
__device__ __forceinline__ f32x4 mma16(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, SA, sa, SB, sb);
}

// Buffer resource word 3 of a raw (unstrided) buffer with range checking:
// a load at an offset past num_records returns zeros.
constexpr int kRawBufferWord3 = 0x00020000;

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order:
// a loop whose index is a compile-time constant in the body.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Scale words of one quad (4 k-steps) for a lane: B -- the dword whose byte u
// is the tile's scale for k-step u; A -- per row tile the two dwords of the
// row's 8 block scales, shifted right by 8*(lane/32) so that byte 2*(u%2) of
// word u/2 is the lane's block 2u + lane/32.
template <int RT, int CT>
struct QuadScales {
    uint32_t b[CT];
    uint32_t a[RT][2];
};

// ---------------------------------------------------------------------------
// Streaming kernel (M <= 64).  Wave w of a workgroup works on tile
// blockIdx.x * (8/KP) + w / KP over part w % KP of the k-steps (whole quads);
// per k-step a lane needs 16 bytes of codes and 2 x 16 bytes of X per row
// tile, in a ring of P k-steps in flight, and the quad's scale words, loaded
// a quad ahead.  The KP parts of a tile add up in LDS in part order.
//
// BD (M <= 8; the plan uses it up to M = 4): v_mfma_scale_f32_16x16x128_f8f6f4,
// half the matrix-core cycles of the 32x32x64 form, on the same B operands and
// B scales.  In the
// 16x16x128 instruction B lane l holds column l % 16 at reduction indices
// 32 * (l / 16) .. +31 (block l / 16), so block p carries the columns of tile
// half p % 2 at k-half p / 2 of the k-step; A lane l holds row l % 16, bytes
// 0..15 at 16 * (l / 16) + j and bytes 16..31 at 64 + 16 * (l / 16) + j (block
// (l / 16) / 2 and 2 + (l / 16) / 2); each lane's scale byte is that of row
// l % 16, block l / 16 (measured on gfx950).  The A operand is block
// diagonal: row i of the 16 belongs to half (i / 4) % 2 and carries X row
// x(i) = i % 4 + 4 * (i / 8); its lane in group o = l / 16 is live iff o / 2
// is that half (then bytes 0..15 are X at k = 64s + 16 * (o % 2) + j and
// bytes 16..31 at 64s + 32 + 16 * (o % 2) + j, the pattern of the 32x32 form
// with l / 32 replaced by o % 2) and x(i) < M; other lanes read zeros past
// the end of a buffer resource.  Lane l's A scale is row x(i)'s, block
// 2s + l / 32, as in the 32x32 form.  Lane l's four accumulator registers
// are its own column l % 32, X rows 4 * (l / 32) + r.  An empty A block
// still meets the B scale of the other half's column, so a NaN (0xFF) weight
// scale would reach a second column: blobs whose repack flagged one take
// the 32x32 form.
// ---------------------------------------------------------------------------
constexpr int kStreamDepth = 4;
constexpr uint32_t kPastEnd = 0x40000000u;   // >= M * K of any block-diagonal launch

template <int RT, int KP, bool BF16, bool BD>
__device__ __forceinline__ void stream_body(const uint8_t* __restrict__ X,
                                            const uint8_t* __restrict__ XS,
                                            const uint8_t* __restrict__ blob, void* __restrict__ Y,
                                            int M, int N, int K, size_t s_off, float* red) {
    static_assert(!BD || RT == 1, "the block-diagonal form holds 8 rows");
    using Acc = typename std::conditional<BD, f32x4, f32x16>::type;
    constexpr int NR = BD ? 4 : 16;   // accumulator registers per lane
    constexpr int CTW = kMxWaves / KP;
    constexpr int P = kStreamDepth;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int part = wave % KP;
    const int ctl = wave / KP;
    const int KS = K / kStepK;
    const int KQ = K / kKAlign;
    const int t = blockIdx.x * CTW + ctl;
    const int per = ((KS + KP - 1) / KP + 3) & ~3;   // k-steps per part, whole quads
    const int c0 = min(part * per, KS);
    const int c1 = min(c0 + per, KS);
    const int n = c1 - c0;
    const int h = lane >> 5;

    const u32x4* wsrc = (const u32x4*)blob + (size_t)t * KS * 64 + lane;
    const uint8_t* ssrc = blob + s_off + (size_t)t * KQ * 256 + lane * 4;
    const uint8_t* xsrc[RT];
    const uint8_t* xssrc[RT];   // the row's block scales, 8 per quad
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int row = min(32 * r + (lane & 31), M - 1);
        xsrc[r] = X + (size_t)row * K + 16 * h;
        xssrc[r] = XS + (size_t)row * (K / 32);
    }
    const __amdgpu_buffer_rsrc_t xrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, BD ? M * K : 0, kRawBufferWord3);
    uint32_t xoff = 0;
    if constexpr (BD) {
        const int ai = lane & 15;
        const int axr = (ai & 3) + 4 * (ai >> 3);
        const bool alive = (lane >> 5) == ((ai >> 2) & 1) && axr < M;
        xoff = alive ? (uint32_t)axr * (uint32_t)K + 16u * (uint32_t)((lane >> 4) & 1) : kPastEnd;
        xssrc[0] = XS + (size_t)min(axr, M - 1) * (K / 32);
    }

    Acc acc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int i = 0; i < NR; ++i) acc[r][i] = 0.0f;

    // codes and X in a ring of P = 4 k-steps; scales one quad ahead (the
    // parts start on quad boundaries, so k-step c of the ring is byte c % 4)
    static_assert(P == 4, "one quad of scales per ring turn");
    u32x4 wb[P];
    i32x4 xb[P][RT][2];
    auto fill = [&](int i, int c) __attribute__((always_inline)) {
        wb[i] = __builtin_nontemporal_load(wsrc + (size_t)c * 64);
        if constexpr (BD) {
            const uint32_t o = xoff + (uint32_t)c * kStepK;
            xb[i][0][0] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, o, 0, 0));
            xb[i][0][1] =
                __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, o + 32, 0, 0));
        } else {
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                xb[i][r][0] = *(const i32x4*)(xsrc[r] + (size_t)c * kStepK);
                xb[i][r][1] = *(const i32x4*)(xsrc[r] + (size_t)c * kStepK + 32);
            }
        }
    };
    QuadScales<RT, 1> cur, nxt;
    auto load_quad = [&](QuadScales<RT, 1>& qs, int quad) __attribute__((always_inline)) {
        qs.b[0] = *(const uint32_t*)(ssrc + (size_t)quad * 256);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const uint2 v = *(const uint2*)(xssrc[r] + (size_t)quad * 8);
            qs.a[r][0] = v.x;
            qs.a[r][1] = v.y;
        }
    };
    auto shift_a = [&](QuadScales<RT, 1>& qs) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            qs.a[r][0] >>= 8 * h;
            qs.a[r][1] >>= 8 * h;
        }
    };
    load_quad(cur, min(c0, c1 - 1) >> 2);
#pragma unroll
    for (int i = 0; i < P; ++i) fill(i, min(c0 + i, c1 - 1));
    shift_a(cur);

    for (int base = 0; base < n; base += P) {
        load_quad(nxt, min(c0 + base + P, c1 - 1) >> 2);
        static_for<P>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            const int c = c0 + base + i;
            if (base + i < n) {
                const i32x8 b = widen(wb[i]);
                i32x8 a[RT];
#pragma unroll
                for (int r = 0; r < RT; ++r) a[r] = cat(xb[i][r][0], xb[i][r][1]);
                fill(i, min(c + P, c1 - 1));
                if constexpr (BD) {
                    acc[0] = mma16<2 * (i & 1), i>(a[0], b, acc[0], (int)cur.a[0][i >> 1],
                                                   (int)cur.b[0]);
                } else {
#pragma unroll
                    for (int r = 0; r < RT; ++r)
                        acc[r] = mma<2 * (i & 1), i>(a[r], b, acc[r], (int)cur.a[r][i >> 1],
                                                     (int)cur.b[0]);
                }
            }
        });
        shift_a(nxt);
        cur = nxt;
    }

    if constexpr (KP > 1) {
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
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int row = BD ? 4 * h + i : 32 * r + acc_row(i, lane);
            if (row < M) store_out<BF16>(Y, (int64_t)row * N + col, acc[r][i]);
        }
}

// BDOK: the block-diagonal form unless the blob's trailer flags a NaN weight
// scale (a uniform branch at the start).
template <int RT, int KP, bool BF16, bool BDOK>
__global__ __launch_bounds__(kMxWaves * 64) void mx_stream_kernel(
    const uint8_t* __restrict__ X, const uint8_t* __restrict__ XS, const uint8_t* __restrict__ blob,
    void* __restrict__ Y, int M, int N, int K, size_t s_off, size_t t_off) {
    extern __shared__ float red[];
    if constexpr (BDOK) {
        const uint32_t flags =
            __builtin_amdgcn_readfirstlane(*(const uint32_t*)(blob + t_off + 8));
        if (flags & kTrailerFlagNanScale)
            stream_body<RT, KP, BF16, false>(X, XS, blob, Y, M, N, K, s_off, red);
        else
            stream_body<RT, KP, BF16, true>(X, XS, blob, Y, M, N, K, s_off, red);
    } else {
        stream_body<RT, KP, BF16, false>(X, XS, blob, Y, M, N, K, s_off, red);
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel (M > 32).  A workgroup owns BM = WM*RT*32 rows and BN =
// WN*CT*32 columns over all of K.  X goes through a two-slot LDS ring of CK
// k-steps per slot (rows of 64*CK bytes padded by 16; CK = 1: loaded two
// k-steps ahead; CK = 2: one stage ahead, half the barriers), each wave's
// codes through a register ring of PD = 4 k-steps; the scale words of a quad
// of k-steps (B: one dword per tile, A: 8 bytes per row tile) are loaded a
// quad ahead and each k-step picks its byte with the instruction's byte
// select.  One barrier per k-step; the XCD-grouped tile order of the W4A8
// tiled kernel.
// ---------------------------------------------------------------------------
template <int RT, int CT, int WM, int WN, int PD, int CK, bool BF16>
__global__ __launch_bounds__(kMxWaves * 64) void mx_tiled_kernel(
    const uint8_t* __restrict__ X, const uint8_t* __restrict__ XS, const uint8_t* __restrict__ blob,
    void* __restrict__ Y, int M, int N, int K, size_t s_off, int nbm, int nbn) {
    static_assert(WM * WN == kMxWaves, "eight waves");
    // the ring must divide the k-step count: KS is a multiple of 4, and of 8
    // where the launcher picks PD = 8
    static_assert(PD == 4 || PD == 8, "ring depth");
    constexpr int BM = WM * RT * 32;
    constexpr int BN = WN * CT * 32;
    static_assert(CK == 1 || CK == 2, "one or two k-steps per LDS stage");
    constexpr int RB = kStepK * CK + 16;
    constexpr int SLOT = BM * RB;
    constexpr int PIECES = BM * 4 * CK / (kMxWaves * 64);
    static_assert(PIECES >= 1 && BM * 4 * CK == PIECES * kMxWaves * 64, "X staging");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int KS = K / kStepK;
    const int KQ = K / kKAlign;
    const int NT = N / kTileCols;
    const int h = lane >> 5;

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
    const uint8_t* ssrc[CT];
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        const int tt = nb * (BN / 32) + wn * CT + j;
        tile_ok[j] = tt < NT;
        tile[j] = min(tt, NT - 1);
        wsrc[j] = (const u32x4*)blob + (size_t)tile[j] * KS * 64 + lane;
        ssrc[j] = blob + s_off + (size_t)tile[j] * KQ * 256 + lane * 4;
    }
    const uint8_t* xssrc[RT];   // each row's block scales, 8 per quad
#pragma unroll
    for (int r = 0; r < RT; ++r)
        xssrc[r] = XS + (size_t)min(m0 + wm * RT * 32 + 32 * r + (lane & 31), M - 1) * (K / 32);

    const uint8_t* xg[PIECES];
    int xl[PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
        // 16 consecutive pieces: quarters 0..3 of rows b, b+4, b+8, b+12 (an
        // 80-byte row stride puts those at dword offsets 0, 16, 32, 48 mod 64,
        // so the 16-byte LDS writes of 16 lanes meet all 64 banks once)
        const int p = tid + kMxWaves * 64 * i;
        // CK = 2: 16 consecutive pieces are the 8 pieces of rows b and b+8
        // (144-byte stride: 32 dwords apart)
        const int q = CK == 1 ? (p & 3) : (p & 7);
        const int row = CK == 1 ? ((p >> 6) << 4) + (((p >> 2) & 3) << 2) + ((p >> 4) & 3)
                                : ((p >> 7) << 4) + (((p >> 3) & 1) << 3) + ((p >> 4) & 7);
        xg[i] = X + (size_t)min(m0 + row, M - 1) * K + 16 * q;
        xl[i] = row * RB + 16 * q;
    }
    const int arow = (wm * RT * 32 + (lane & 31)) * RB + 16 * h;

    f32x16 acc[RT][CT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < CT; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[r][j][i] = 0.0f;

    // ring slot s: the codes of the k-step c with c % PD == s; scales one
    // quad ahead (k-step c is byte c % 4 of its quad's scale words)

    u32x4 wb[PD][CT];
    auto fill = [&](int s, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CT; ++j) wb[s][j] = __builtin_nontemporal_load(wsrc[j] + (size_t)c * 64);
    };
    QuadScales<RT, CT> cur, nxt;
    auto load_quad = [&](QuadScales<RT, CT>& qs, int quad) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < CT; ++j) qs.b[j] = *(const uint32_t*)(ssrc[j] + (size_t)quad * 256);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const uint2 v = *(const uint2*)(xssrc[r] + (size_t)quad * 8);
            qs.a[r][0] = v.x;
            qs.a[r][1] = v.y;
        }
    };
    auto shift_a = [&](QuadScales<RT, CT>& qs) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            qs.a[r][0] >>= 8 * h;
            qs.a[r][1] >>= 8 * h;
        }
    };

    // X: CK = 1, two k-steps ahead (xr[c % 2] receives k-step c + 2 while c + 1
    // waits in the other); CK = 2, one stage (two k-steps) ahead
    constexpr int XR = CK == 1 ? 2 : 1;
    i32x4 xr[XR][PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
        xr[0][i] = *(const i32x4*)xg[i];
        if constexpr (CK == 1) xr[1][i] = *(const i32x4*)(xg[i] + (size_t)min(1, KS - 1) * kStepK);
    }
    load_quad(cur, 0);
#pragma unroll
    for (int s = 0; s < PD; ++s) fill(s, min(s, KS - 1));
#pragma unroll
    for (int i = 0; i < PIECES; ++i) *(i32x4*)(lds + xl[i]) = xr[0][i];
    shift_a(cur);
    __syncthreads();

    for (int cb = 0; cb < KS; cb += PD) {   // KS is a multiple of PD
        static_for<PD>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            const int c = cb + q;
            if constexpr (q % 4 == 0) load_quad(nxt, min(c + 4, KS - 1) >> 2);
            constexpr int j2 = q % CK;                 // k-step inside its LDS stage
            constexpr int sp = (q / CK) & 1;           // LDS slot of this stage
            const uint8_t* slot = lds + sp * SLOT;
            if constexpr (j2 == 0) {
                // X of the stage CK k-steps ahead of this one (XR = 2: two ahead)
                i32x4 (&xin)[PIECES] = xr[XR == 2 ? (q & 1) : 0];
                const int cn = min(c + (CK == 1 ? 2 : CK), KS - CK);
#pragma unroll
                for (int i = 0; i < PIECES; ++i)
                    xin[i] = *(const i32x4*)(xg[i] + (size_t)cn * kStepK);
            }
            i32x8 b[CT];
#pragma unroll
            for (int j = 0; j < CT; ++j) b[j] = widen(wb[q][j]);
            fill(q, min(c + PD, KS - 1));
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int off = arow + r * 32 * RB + j2 * kStepK;
                const i32x8 a = cat(*(const i32x4*)(slot + off), *(const i32x4*)(slot + off + 32));
#pragma unroll
                for (int j = 0; j < CT; ++j)
                    acc[r][j] = mma<2 * (q & 1), q % 4>(a, b[j], acc[r][j],
                                                        (int)cur.a[r][(q % 4) >> 1], (int)cur.b[j]);
            }
            if constexpr (j2 == CK - 1) {
                // the other LDS slot was last read in the stage before, before the previous barrier
                uint8_t* next = lds + (1 - sp) * SLOT;
                i32x4 (&xout)[PIECES] = xr[XR == 2 ? 1 - (q & 1) : 0];   // the next stage
#pragma unroll
                for (int i = 0; i < PIECES; ++i) *(i32x4*)(next + xl[i]) = xout[i];
                __syncthreads();
            }
            if constexpr (q % 4 == 3) {
                shift_a(nxt);
                cur = nxt;
            }
        });
    }

#pragma unroll
    for (int j = 0; j < CT; ++j) {
        if (!tile_ok[j]) continue;
        const int col = tile[j] * kTileCols + (lane & 31);
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + wm * RT * 32 + 32 * r + acc_row(i, lane);
                if (row < M) store_out<BF16>(Y, (int64_t)row * N + col, acc[r][j][i]);
            }
    }
}

template <int RT, int KP>
hipError_t launch_stream_t(const uint8_t* xq, const uint8_t* xs, const void* packed, void* Y,
                           int64_t M, const LayoutMX& L, const PlanMX& plan, hipStream_t stream) {
    constexpr bool BF = MXFP4_TU_BF16 != 0;
    if constexpr (RT == 1) {
        if (plan.bd) {
            if (M > kMxBlockDiagMaxRows || M * L.K > kMxBlockDiagMaxXBytes)
                return hipErrorInvalidValue;   // the plan never asks for it
            mx_stream_kernel<1, KP, BF, true><<<plan.grid, kMxWaves * 64, plan.lds, stream>>>(
                xq, xs, (const uint8_t*)packed, Y, (int)M, (int)L.N, (int)L.K, L.s_off, L.t_off);
            return hipGetLastError();
        }
    }
    mx_stream_kernel<RT, KP, BF, false><<<plan.grid, kMxWaves * 64, plan.lds, stream>>>(
        xq, xs, (const uint8_t*)packed, Y, (int)M, (int)L.N, (int)L.K, L.s_off, L.t_off);
    return hipGetLastError();
}

template <int RT>
hipError_t launch_stream_kp(const uint8_t* xq, const uint8_t* xs, const void* packed, void* Y,
                            int64_t M, const LayoutMX& L, const PlanMX& plan, hipStream_t stream) {
    switch (plan.kp) {
        case 2: return launch_stream_t<RT, 2>(xq, xs, packed, Y, M, L, plan, stream);
        case 4: return launch_stream_t<RT, 4>(xq, xs, packed, Y, M, L, plan, stream);
        default: return launch_stream_t<RT, 8>(xq, xs, packed, Y, M, L, plan, stream);
    }
}

hipError_t launch_part(const uint8_t* xq, const uint8_t* xs, const void* packed, void* Y,
                       int64_t M, const LayoutMX& L, const PlanMX& plan, hipStream_t stream) {
    constexpr bool BF = MXFP4_TU_BF16 != 0;
    const uint8_t* b = (const uint8_t*)packed;
    if (plan.variant == MX_STREAM) {
        if (plan.rt == 1) return launch_stream_kp<1>(xq, xs, packed, Y, M, L, plan, stream);
        return launch_stream_kp<2>(xq, xs, packed, Y, M, L, plan, stream);
    }
    if (plan.cfg == 0)
        mx_tiled_kernel<4, 2, 2, 4, 4, 1, BF><<<plan.grid, kMxWaves * 64, plan.lds, stream>>>(
            xq, xs, b, Y, (int)M, (int)L.N, (int)L.K, L.s_off, plan.nbm, plan.nbn);
    else if (plan.cfg == 1 && L.KS % 8 == 0)   // codes 8 k-steps ahead where the ring divides K
        mx_tiled_kernel<2, 1, 2, 4, 8, 1, BF><<<plan.grid, kMxWaves * 64, plan.lds, stream>>>(
            xq, xs, b, Y, (int)M, (int)L.N, (int)L.K, L.s_off, plan.nbm, plan.nbn);
    else if (plan.cfg == 1)
        mx_tiled_kernel<2, 1, 2, 4, 4, 1, BF><<<plan.grid, kMxWaves * 64, plan.lds, stream>>>(
            xq, xs, b, Y, (int)M, (int)L.N, (int)L.K, L.s_off, plan.nbm, plan.nbn);
    else if (plan.cfg == 3)
        mx_tiled_kernel<4, 2, 2, 4, 4, 2, BF><<<plan.grid, kMxWaves * 64, plan.lds, stream>>>(
            xq, xs, b, Y, (int)M, (int)L.N, (int)L.K, L.s_off, plan.nbm, plan.nbn);
    else
        mx_tiled_kernel<4, 1, 2, 4, 4, 1, BF><<<plan.grid, kMxWaves * 64, plan.lds, stream>>>(
            xq, xs, b, Y, (int)M, (int)L.N, (int)L.K, L.s_off, plan.nbm, plan.nbn);
    return hipGetLastError();
}

}  // namespace

#if MXFP4_TU_BF16
hipError_t launch_mx_gemm_bf16(const uint8_t* xq, const uint8_t* xs, const void* packed, void* Y,
                               int64_t M, const LayoutMX& L, const PlanMX& plan,
                               hipStream_t stream) {
    return launch_part(xq, xs, packed, Y, M, L, plan, stream);
}
#else
hipError_t launch_mx_gemm_f16(const uint8_t* xq, const uint8_t* xs, const void* packed, void* Y,
                              int64_t M, const LayoutMX& L, const PlanMX& plan,
                              hipStream_t stream) {
    return launch_part(xq, xs, packed, Y, M, L, plan, stream);
}
#endif

}  // namespace mxfp4
