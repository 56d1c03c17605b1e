// w4a16_gemm.hip -- the fused W4A16 dequantize-GEMM kernels for gfx950.
//
// Page "量化开销对比" (laojiahuo2003.github.io), section 6.2: per output tile,
// walk along k; at each k-block load the packed 4-bit weights, unpack,
// multiply by the group scale and feed the matrix instruction, keeping the
// accumulators in registers, with the next block's loads in flight while the
// current one computes.  Section 6.5: the weights are streamed exactly once;
// at decode, reuse is mainly along N.
//
// Two variants (page "W4A16 GEMM 算子浅析", section "硬件性能拐点": small
// batches are bound by memory bandwidth, large batches by the matrix units):
//
//  * splitk_kernel (M <= 32).  Memory-bound streaming.  A workgroup owns one
//    128-column block and a slice of K; its 8 waves split that slice further.
//    Each lane issues one 16-byte load per k-step (the whole 1 KiB chunk per
//    wave), eight k-steps per batch, two batches in flight.  The activation
//    rows come straight from global memory (they are tiny and L2-resident).
//    Partial sums are reduced across waves through LDS and across workgroups
//    through a workspace, both in a fixed order.  The multiply-accumulate
//    runs on v_mfma_f32_32x32x16 even at M = 1: the vector ALUs are the
//    scarce resource on MI355X at this bandwidth (they carry the unpack and
//    dequant), while the matrix units are idle.
//
//  * tiled_kernel (M > 32).  A workgroup of 4 waves owns 32*MT rows by 512
//    columns; each wave owns one 128-column block, dequantizes each weight
//    word once and reuses it across MT row tiles.  Activation tiles are
//    staged through LDS (double-buffered) and shared by the 4 waves.
//
// MFMA operand layout (v_mfma_f32_32x32x16_{f16,bf16}): lane l holds A row
// l%32 and B column l%32, reduction indices 8*(l/32)..+7 of the 16; the
// accumulator register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column
// l%32.  Only the row/column placement matters: A and B use the same
// placement of k inside the 16, so the sum is the same whatever the hardware's
// internal k order is.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {


// k-steps per split-K load batch.  Two waves share a SIMD, so each has 256
// registers including the 64 accumulators; the bf16 dequant (eight fp32
// temporaries per word) needs the smaller batch to stay out of scratch.
template <int DT>
constexpr int splitk_batch() { return DT == DT_BF16 ? 4 : 8; }

__device__ __forceinline__ u32x4 load_weights(const u32x4* p) {
    return __builtin_nontemporal_load(p);   // streamed once: do not keep in cache
}

// Whether this blob needs the exact bf16 dequant form (a trailer flag set by
// the repack); read once per wave, so the hot loop carries no test.
template <int DT>
__device__ __forceinline__ bool uses_exact_form(const uint8_t* packed, size_t t_off) {
    if constexpr (DT == DT_F16) {
        return false;
    } else {
        const uint32_t flags = *(const uint32_t*)(packed + t_off + 8);
        return (flags & kFlagExactBf16) != 0;
    }
}

// ---------------------------------------------------------------------------
// Cross-workgroup partial sums.
//
// Workgroups that share an output tile along K write their fp32 partial tile
// to a workspace slot with device-scope stores (global_store ... sc1, which
// bypass the per-XCD L2), wait until those stores have completed, and then
// bump the tile's counter with a device-scope atomic.  The workgroup that
// sees the count reach S-1 reads all S slots with device-scope loads, adds
// them in slot order 0..S-1 (bitwise reproducible), writes Y and resets the
// counter to 0 for the next call.  Nobody waits on anybody: there is no spin.
// A seq_cst __threadfence() here would write back and invalidate a whole
// XCD's L2 per workgroup, which costs far more than the GEMM itself.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_done() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// Returns true in every thread of the workgroup that arrives last.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, int S, uint32_t* s_flag) {
    wait_stores_done();
    __syncthreads();
    if (threadIdx.x == 0)
        *s_flag = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(S - 1);
    __syncthreads();
    return *s_flag != 0;
}
__device__ __forceinline__ void reset_counter(uint32_t* counter) {
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Split-K streaming kernel, M <= 32 ("stream-K" over workgroups).
//
// The weight chunks are numbered c = nb*KS + ks (column block major).
// Workgroup g (8 waves, one per CU) owns the contiguous range [g*L, (g+1)*L):
// every workgroup streams the same number of bytes and all of them run in one
// round.  The range crosses column blocks, so the workgroup works through one
// or more segments (nb, [kb, ke)).
//
// Inside a segment the workgroup advances in super-batches of 8 batches: wave
// w computes batch w of each super-batch.  Each wave keeps its next NBUF-1
// batches of weights in flight in registers (the HBM stream), while the
// activation rows of the super-batch are staged once through LDS (double
// buffered, one barrier per super-batch) instead of occupying registers: they
// carry no HBM traffic and would otherwise take half of each batch's
// registers.  At the segment's end the waves reduce their partial tiles
// through LDS in a fixed order, and then
//   * a segment that covers a whole column block writes Y;
//   * otherwise the workgroup stores its partial tile (rows < M only) in slot
//     (nb, g - first workgroup of nb) and bumps nb's counter; the workgroup
//     that arrives last adds the column block's slots in workgroup order
//     (bitwise reproducible) and writes Y.
// L and KS are multiples of 8 k-steps (or L is a multiple of KS), so every
// segment starts on a batch and group boundary.
// ---------------------------------------------------------------------------
constexpr int SK_WAVES = 8;

template <int DT>
constexpr int splitk_nbuf() { return DT == DT_BF16 ? 4 : 3; }   // weight batches per wave

template <int DT>
constexpr int splitk_xpitch() {   // LDS row pitch of a staged activation tile, halves
    return SK_WAVES * splitk_batch<DT>() * kKStep + 8;   // +16 B against bank conflicts
}

template <int DT, int MB>
constexpr int splitk_lds_bytes() {
    const int xs = 2 * MB * splitk_xpitch<DT>() * 2;
    const int red = (SK_WAVES / 2) * 4 * 4 * 64 * 16;
    return xs > red ? xs : red;
}

// MB: rows of the activation tile (8, 16 or 32 >= M), sizes the staging.
template <int DT, bool SYM, int GS, int MB>
__global__ __launch_bounds__(SK_WAVES * 64) void splitk_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed, uint16_t* __restrict__ Y,
    float* __restrict__ part, uint32_t* __restrict__ cnt, int M, int N, int K, int L, int maxc,
    size_t s_off, size_t z_off, size_t t_off) {
    constexpr int SK_U = splitk_batch<DT>();
    constexpr int NBUF = splitk_nbuf<DT>();
    constexpr int SB = SK_WAVES * SK_U;          // k-steps per super-batch
    constexpr int XP = splitk_xpitch<DT>();      // LDS row pitch (halves)
    constexpr int XCPR = SB * 2;                 // 16-byte activation chunks per row
    constexpr int SPG = GS < SK_U ? GS : SK_U;   // k-steps per group inside a batch
    constexpr int NGB = SK_U / SPG;              // groups (or group parts) per batch
    constexpr int XCH = MB * XCPR / (SK_WAVES * 64);   // activation chunks per thread
    static_assert(XCH >= 1 && MB * XCPR == XCH * SK_WAVES * 64, "tile split");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wg = blockIdx.x;
    const int KS = K / kKStep;
    const int NB = N / kColBlock;
    const int NG = K / (kKStep * GS);
    const int64_t total = (int64_t)NB * KS;
    const int64_t c0 = (int64_t)wg * L;
    const int64_t c1 = min(c0 + (int64_t)L, total);
    if (c0 >= c1) return;

    __shared__ __align__(16) uint8_t lds[splitk_lds_bytes<DT, MB>()];
    __shared__ uint32_t s_last;
    uint16_t* xs = (uint16_t*)lds;                 // [2][MB rows][XP], during the main loop
    f32x4(*red)[4][4][64] = (f32x4(*)[4][4][64])lds;   // [4][t][q][lane], after it

    const bool exact = uses_exact_form<DT>(packed, t_off);
    const int lrow = 4 * (lane >> 5);   // accumulator register r: row 8*(r/4) + r%4 + lrow
    const int lcol = lane & 31;
    // A operand of this lane: activation row min(lane%32, M-1) (rows >= M only
    // feed output rows that are never stored), 8 halves at 8*(lane/32).
    const int arow = min(lane & 31, M - 1);

    struct Batch {
        u32x2 sc[NGB];
        uint32_t zw[NGB];
        u32x4 w[SK_U];
    };

    f32x16 acc[4];
    const int nb_first = (int)(c0 / KS);
    const int nb_last = (int)((c1 - 1) / KS);
    for (int nb = nb_first; nb <= nb_last; ++nb) {
        const int kb = (int)(max(c0, (int64_t)nb * KS) - (int64_t)nb * KS);
        const int ke = (int)(min(c1, (int64_t)(nb + 1) * KS) - (int64_t)nb * KS);
        const int nsb = (ke - kb + SB - 1) / SB;
        const u32x4* wbase = (const u32x4*)packed + (size_t)nb * KS * 64 + lane;
        const uint8_t* srec = packed + s_off + (size_t)nb * NG * kScaleRecBytes + (lane & 31) * 8;
        const uint8_t* zrec = packed + z_off + (size_t)nb * NG * kZeroRecBytes + (lane & 31) * 2;

        // Weights of this wave's batch in super-batch j.  Loads are issued
        // unconditionally (exact wait counts for the compiler); past the end
        // they re-read the segment's last step (values never used).
        auto load_w = [&](Batch& b, int j) {
            const int sb = kb + j * SB + wave * SK_U;
            const bool real = sb < ke;
#pragma unroll
            for (int q = 0; q < NGB; ++q) {
                const int g = (real ? min(sb + q * SPG, ke - 1) : ke - 1) / GS;
                b.sc[q] = *(const u32x2*)(srec + (size_t)g * kScaleRecBytes);
                b.zw[q] = SYM ? 0u : (uint32_t)*(const uint16_t*)(zrec + (size_t)g * kZeroRecBytes);
            }
#pragma unroll
            for (int u = 0; u < SK_U; ++u) {
                const int s = real ? min(sb + u, ke - 1) : ke - 1;
                b.w[u] = load_weights(wbase + (size_t)s * 64);
            }
        };

        // Activation tile of super-batch j: MB rows (rows >= M repeat row
        // M-1), 16*SB reduction indices (past K: column K-8, never used);
        // thread chunk i covers row c / XCPR, 8 halves at 8 * (c % XCPR).
        u32x4 xr[XCH];
        auto load_x = [&](int j) {
#pragma unroll
            for (int i = 0; i < XCH; ++i) {
                const int c = tid + SK_WAVES * 64 * i;
                const int r = min(c / XCPR, M - 1);
                const int k = min(kKStep * (kb + j * SB) + 8 * (c % XCPR), K - 8);
                xr[i] = *(const u32x4*)(X + (size_t)r * K + k);
            }
        };
        auto store_x = [&](int buf) {
#pragma unroll
            for (int i = 0; i < XCH; ++i) {
                const int c = tid + SK_WAVES * 64 * i;
                *(u32x4*)&xs[(buf * MB + c / XCPR) * XP + 8 * (c % XCPR)] = xr[i];
            }
        };

        auto compute = [&](const Batch& b, int j, auto ex) {
            const int nvalid = min(SK_U, ke - (kb + j * SB + wave * SK_U));   // <= 0 past the end
            const uint16_t* xa = &xs[((j & 1) * MB + arow) * XP + wave * SK_U * kKStep + 8 * (lane >> 5)];
#pragma unroll
            for (int q = 0; q < NGB; ++q) {
                if (q * SPG >= nvalid) break;
                ColParams<DT> prm[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) prm[t] = tile_params<DT, SYM>(b.sc[q], b.zw[q], t);
#pragma unroll
                for (int uu = 0; uu < SPG; ++uu) {
                    const int u = q * SPG + uu;
                    if (u >= nvalid) break;
                    const u32x4 a = *(const u32x4*)(xa + kKStep * u);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const u32x4 bop = dequant_sel<decltype(ex)::value>(b.w[u][t], prm[t]);
                        acc[t] = mfma32x32x16<DT>(a, bop, acc[t]);
                    }
                }
            }
        };

        // NBUF register buffers rotate: super-batch j computes while the next
        // NBUF-1 of this wave's batches are in flight.  One loop exit; the
        // super-batch count is rounded up to NBUF with empty trailing rounds.
        auto mainloop = [&](auto ex) {
            Batch bw[NBUF];
#pragma unroll
            for (int r = 0; r < NBUF - 1; ++r) load_w(bw[r], r);
            load_x(0);
            store_x(0);
            __syncthreads();
            int jj = 0;
            do {
#pragma unroll
                for (int r = 0; r < NBUF; ++r) {
                    const int j = jj + r;
                    load_w(bw[(r + NBUF - 1) % NBUF], j + NBUF - 1);
                    load_x(j + 1);
                    compute(bw[r], j, ex);
                    store_x((j + 1) & 1);
                    __syncthreads();
                }
                jj += NBUF;
            } while (jj < nsb);
        };

#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = f32x16{};
        if (exact)
            mainloop(std::true_type{});
        else
            mainloop(std::false_type{});

        // Reduce the 8 waves' tiles through LDS (reusing the activation
        // buffers): halve the active waves each round, always adding slot w
        // into wave w (a fixed order).
#pragma unroll
        for (int h = SK_WAVES / 2; h >= 1; h >>= 1) {
            if (wave >= h && wave < 2 * h) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        red[wave - h][t][q][lane] = f32x4{acc[t][4 * q], acc[t][4 * q + 1],
                                                          acc[t][4 * q + 2], acc[t][4 * q + 3]};
            }
            __syncthreads();
            if (wave < h) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 v = red[wave][t][q][lane];
                        acc[t][4 * q] += v.x;
                        acc[t][4 * q + 1] += v.y;
                        acc[t][4 * q + 2] += v.z;
                        acc[t][4 * q + 3] += v.w;
                    }
            }
            __syncthreads();
        }

        const int64_t colw = (int64_t)nb * kColBlock + lcol;
        if (kb == 0 && ke == KS) {
            // the whole column block is this workgroup's: write Y directly
            if (wave == 0) {
                uint16_t* ybase = Y + (int64_t)lrow * N + colw;
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int r0 = 8 * (r >> 2) + (r & 3);
                        if (r0 + lrow < M) ybase[(int64_t)r0 * N + 32 * t] = round_out<DT>(acc[t][r]);
                    }
            }
            continue;
        }

        // Partial tile: rows < M only; float index (t*M + row)*32 + col.
        const int first = (int)(((int64_t)nb * KS) / L);
        const int last = (int)(((int64_t)(nb + 1) * KS - 1) / L);
        const int ncontrib = last - first + 1;
        const int slot_floats = 4 * M * 32;
        float* slots = part + (size_t)nb * maxc * slot_floats;
        if (wave == 0) {
            float* pbase = slots + (size_t)(wg - first) * slot_floats + lrow * 32 + lcol;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int r0 = 8 * (r >> 2) + (r & 3);
                    if (r0 + lrow < M) st_dev(&pbase[(t * M + r0) * 32], acc[t][r]);
                }
        }
        if (!arrive_last(&cnt[nb], ncontrib, &s_last)) continue;

        // Last arrival: all threads add the slots in workgroup order.
        for (int f = tid; f < slot_floats; f += SK_WAVES * 64) {
            float sum = ld_dev(&slots[f]);
            int c = 1;
            for (; c + 3 < ncontrib; c += 4) {
                const float v1 = ld_dev(&slots[(size_t)c * slot_floats + f]);
                const float v2 = ld_dev(&slots[(size_t)(c + 1) * slot_floats + f]);
                const float v3 = ld_dev(&slots[(size_t)(c + 2) * slot_floats + f]);
                const float v4 = ld_dev(&slots[(size_t)(c + 3) * slot_floats + f]);
                sum = (((sum + v1) + v2) + v3) + v4;
            }
            for (; c < ncontrib; ++c) sum += ld_dev(&slots[(size_t)c * slot_floats + f]);
            const int col = f & 31;
            const int rr = (f >> 5) % M;
            const int t = (f >> 5) / M;
            Y[(int64_t)rr * N + (int64_t)nb * kColBlock + 32 * t + col] = round_out<DT>(sum);
        }
        if (tid == 0) reset_counter(&cnt[nb]);
        __syncthreads();   // the LDS tiles are reused by the next segment
    }
}

// ---------------------------------------------------------------------------
// LDS-tiled kernel, M > 32.
// ---------------------------------------------------------------------------
template <int DT, bool SYM, int GS, int MT>
__global__ __launch_bounds__(256) void tiled_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed, uint16_t* __restrict__ Y,
    float* __restrict__ part, uint32_t* __restrict__ cnt, int M, int N, int K,
    int steps_per_split, int S, size_t s_off, size_t z_off, size_t t_off) {
    constexpr int KT = MT == 4 ? 4 : 8;         // k-steps per stage (fits the registers)
    constexpr int ROWS = 32 * MT;
    constexpr int LDX = KT * kKStep + 8;        // LDS row pitch in halves (+16 B against bank conflicts)
    constexpr int SPG = GS < KT ? GS : KT;      // k-steps per group inside a stage
    constexpr int NGST = KT / SPG;              // groups per stage
    constexpr int XCH = ROWS * KT * kKStep / 8 / 256;   // 16-byte X chunks per thread per stage
    __shared__ __align__(16) uint16_t xs[2][ROWS * LDX];
    __shared__ uint32_t s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int NB = N / kColBlock;
    const int KS = K / kKStep;
    const int NG = K / (kKStep * GS);
    const int nb = blockIdx.x * 4 + wave;
    const bool nb_ok = nb < NB;
    const int nbc = nb_ok ? nb : NB - 1;
    const int m0 = blockIdx.y * ROWS;
    const int split = blockIdx.z;
    const int s_beg = split * steps_per_split;   // a multiple of 8 (so of KT)
    const int s_end = min(KS, s_beg + steps_per_split);
    const int nst = s_end > s_beg ? (s_end - s_beg + KT - 1) / KT : 0;

    const u32x4* wbase = (const u32x4*)packed + (size_t)nbc * KS * 64 + lane;
    const uint8_t* srec = packed + s_off + (size_t)nbc * NG * kScaleRecBytes + (lane & 31) * 8;
    const uint8_t* zrec = packed + z_off + (size_t)nbc * NG * kZeroRecBytes + (lane & 31) * 2;

    struct Stage {
        u32x2 sc[NGST];
        uint32_t zw[NGST];
        u32x4 w[KT];
    };

    // X stage copy: chunk c = tid + 256*i covers row c / (2*KT) of the tile,
    // 8 halves at column 8 * (c % (2*KT)).  Rows >= M re-read row M-1 and
    // columns >= K re-read column K-8 (never used), so loads are unconditional.
    auto load_x = [&](u32x4 (&xr)[XCH], int si) {
        const int st = s_beg + min(si, nst - 1) * KT;
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + 256 * i;
            const int row = min(m0 + c / (KT * 2), M - 1);
            const int kk = min(kKStep * st + 8 * (c % (KT * 2)), K - 8);
            xr[i] = *(const u32x4*)(X + (size_t)row * K + kk);
        }
    };
    auto store_x = [&](int buf, const u32x4 (&xr)[XCH]) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + 256 * i;
            *(u32x4*)&xs[buf][(c / (KT * 2)) * LDX + 8 * (c % (KT * 2))] = xr[i];
        }
    };
    auto load_w = [&](Stage& b, int si) {
        const int st = s_beg + min(si, nst - 1) * KT;
#pragma unroll
        for (int j = 0; j < NGST; ++j) {
            const int g = min(st + j * SPG, s_end - 1) / GS;
            b.sc[j] = *(const u32x2*)(srec + (size_t)g * kScaleRecBytes);
            b.zw[j] = SYM ? 0u : (uint32_t)*(const uint16_t*)(zrec + (size_t)g * kZeroRecBytes);
        }
#pragma unroll
        for (int u = 0; u < KT; ++u) b.w[u] = load_weights(wbase + (size_t)min(st + u, s_end - 1) * 64);
    };

    f32x16 acc[MT][4];
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[r][t] = f32x16{};

    auto compute = [&](const Stage& b, int buf, int si, auto exact) {
        const int nvalid = min(KT, s_end - (s_beg + si * KT));   // <= 0 past the end
        const uint16_t* xb = &xs[buf][(lane & 31) * LDX + 8 * (lane >> 5)];
#pragma unroll
        for (int j = 0; j < NGST; ++j) {
            if (j * SPG >= nvalid) break;
            ColParams<DT> prm[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) prm[t] = tile_params<DT, SYM>(b.sc[j], b.zw[j], t);
#pragma unroll
            for (int uu = 0; uu < SPG; ++uu) {
                const int u = j * SPG + uu;
                if (u >= nvalid) break;
                u32x4 a[MT];
#pragma unroll
                for (int r = 0; r < MT; ++r) a[r] = *(const u32x4*)(xb + 32 * r * LDX + kKStep * u);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const u32x4 bop = dequant_sel<decltype(exact)::value>(b.w[u][t], prm[t]);
#pragma unroll
                    for (int r = 0; r < MT; ++r) acc[r][t] = mfma32x32x16<DT>(a[r], bop, acc[r][t]);
                }
            }
        }
    };

    // Stage i sits in LDS buffer i%2 and register set A or B; the next
    // stage's loads are in flight while it computes.  One loop exit; a stage
    // index >= nst loads dummies and computes nothing.
    auto mainloop = [&](auto exact) {
        Stage A, B;
        u32x4 xr[XCH];
        load_x(xr, 0);
        load_w(A, 0);
        store_x(0, xr);
        __syncthreads();
        int i = 0;
        do {
            load_x(xr, i + 1);
            load_w(B, i + 1);
            compute(A, 0, i, exact);
            store_x(1, xr);
            __syncthreads();
            load_x(xr, i + 2);
            load_w(A, i + 2);
            compute(B, 1, i + 1, exact);
            store_x(0, xr);
            __syncthreads();
            i += 2;
        } while (i < nst);
    };
    if (nst > 0) {
        if (uses_exact_form<DT>(packed, t_off))
            mainloop(std::true_type{});
        else
            mainloop(std::false_type{});
    }

    const int64_t colw = (int64_t)nb * kColBlock + (lane & 31);
    if (S == 1) {
        if (nb_ok) {
#pragma unroll
            for (int r = 0; r < MT; ++r)
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int rr = m0 + 32 * r + acc_row(i, lane);
                        if (rr < M) Y[(int64_t)rr * N + colw + 32 * t] = round_out<DT>(acc[r][t][i]);
                    }
        }
        return;
    }

    // Cross-workgroup reduction; slot float index
    // (((wave*MT + r)*4 + t)*16 + i)*64 + lane.
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;
    constexpr int RPW = MT * 4 * 16;   // accumulator registers per lane
    const size_t slot_floats = (size_t)4 * RPW * 64;
    float* base = part + (size_t)tile * S * slot_floats + (size_t)wave * RPW * 64 + lane;
    {
        float* mine = base + (size_t)split * slot_floats;
#pragma unroll
        for (int r = 0; r < MT; ++r)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) st_dev(&mine[((r * 4 + t) * 16 + i) * 64], acc[r][t][i]);
    }
    if (!arrive_last(&cnt[tile], S, &s_last)) return;

    // Sum the S slots in split order 0..S-1, one 32x32 tile at a time (this
    // workgroup's own slot is read back too, so every tile is summed the same
    // way whichever workgroup is last).
#pragma unroll 1
    for (int rt = 0; rt < MT * 4; ++rt) {
        const int r = rt >> 2;
        const int t = rt & 3;
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = ld_dev(&base[(rt * 16 + i) * 64]);
        for (int s = 1; s < S; ++s) {
            const float* src = base + (size_t)s * slot_floats;
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] += ld_dev(&src[(rt * 16 + i) * 64]);
        }
        if (nb_ok) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int rr = m0 + 32 * r + acc_row(i, lane);
                if (rr < M) Y[(int64_t)rr * N + colw + 32 * t] = round_out<DT>(v[i]);
            }
        }
    }
    if (tid == 0) reset_counter(&cnt[tile]);
}
// ---------------------------------------------------------------------------
// One MFMA with the kernels' operand and accumulator placement.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(64) void mfma_probe_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B,
                                                        float* __restrict__ D) {
    const int lane = threadIdx.x;
    const u32x4 a = *(const u32x4*)(A + (lane & 31) * 16 + 8 * (lane >> 5));
    uint32_t bw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = B[(8 * (lane >> 5) + 2 * i) * 32 + (lane & 31)];
        const uint32_t hi = B[(8 * (lane >> 5) + 2 * i + 1) * 32 + (lane & 31)];
        bw[i] = lo | (hi << 16);
    }
    const u32x4 b = {bw[0], bw[1], bw[2], bw[3]};
    f32x16 c = {};
    c = mfma32x32x16<DT>(a, b, c);
#pragma unroll
    for (int r = 0; r < 16; ++r) D[acc_row(r, lane) * 32 + (lane & 31)] = c[r];
}

template <int DT, bool SYM, int GS, int MB>
void launch_splitk_mb(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                      const Plan& p, float* part, uint32_t* cnt, hipStream_t stream) {
    hipLaunchKernelGGL((splitk_kernel<DT, SYM, GS, MB>), dim3(p.grid_x), dim3(SK_WAVES * 64), 0,
                       stream, (const uint16_t*)X, (const uint8_t*)packed, (uint16_t*)Y, part, cnt,
                       (int)M, (int)L.N, (int)L.K, p.steps_per_split, p.splits, L.s_off, L.z_off,
                       L.t_off);
}

template <int DT, bool SYM, int GS>
void launch_splitk(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                   const Plan& p, float* part, uint32_t* cnt, hipStream_t stream) {
    if (M <= 8) launch_splitk_mb<DT, SYM, GS, 8>(X, packed, Y, M, L, p, part, cnt, stream);
    else if (M <= 16) launch_splitk_mb<DT, SYM, GS, 16>(X, packed, Y, M, L, p, part, cnt, stream);
    else launch_splitk_mb<DT, SYM, GS, 32>(X, packed, Y, M, L, p, part, cnt, stream);
}

template <int DT, bool SYM, int GS>
void launch_tiled(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                  const Plan& p, float* part, uint32_t* cnt, hipStream_t stream) {
    const dim3 grid(p.grid_x, p.grid_y, p.grid_z), block(256);
    if (p.mt == 2)
        hipLaunchKernelGGL((tiled_kernel<DT, SYM, GS, 2>), grid, block, 0, stream,
                           (const uint16_t*)X, (const uint8_t*)packed, (uint16_t*)Y, part, cnt,
                           (int)M, (int)L.N, (int)L.K, p.steps_per_split, p.splits, L.s_off,
                           L.z_off, L.t_off);
    else
        hipLaunchKernelGGL((tiled_kernel<DT, SYM, GS, 4>), grid, block, 0, stream,
                           (const uint16_t*)X, (const uint8_t*)packed, (uint16_t*)Y, part, cnt,
                           (int)M, (int)L.N, (int)L.K, p.steps_per_split, p.splits, L.s_off,
                           L.z_off, L.t_off);
}

template <int DT, bool SYM>
void launch_variant(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                    const Plan& p, float* part, uint32_t* cnt, hipStream_t stream) {
    const int GS = (int)(L.G / kKStep);
    if (p.variant == VARIANT_SPLITK) {
        if (GS == 8) launch_splitk<DT, SYM, 8>(X, packed, Y, M, L, p, part, cnt, stream);
        else if (GS == 4) launch_splitk<DT, SYM, 4>(X, packed, Y, M, L, p, part, cnt, stream);
        else launch_splitk<DT, SYM, 2>(X, packed, Y, M, L, p, part, cnt, stream);
    } else {
        if (GS == 8) launch_tiled<DT, SYM, 8>(X, packed, Y, M, L, p, part, cnt, stream);
        else if (GS == 4) launch_tiled<DT, SYM, 4>(X, packed, Y, M, L, p, part, cnt, stream);
        else launch_tiled<DT, SYM, 2>(X, packed, Y, M, L, p, part, cnt, stream);
    }
}

}  // namespace

hipError_t launch_gemm(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                       bool bf16, const Plan& p, void* workspace, hipStream_t stream) {
    uint32_t* cnt = nullptr;
    float* part = nullptr;
    if (p.splits > 1) {
        cnt = (uint32_t*)workspace;
        part = (float*)((uint8_t*)workspace + p.counters_bytes);
    }
    if (bf16) {
        if (L.sym) launch_variant<DT_BF16, true>(X, packed, Y, M, L, p, part, cnt, stream);
        else launch_variant<DT_BF16, false>(X, packed, Y, M, L, p, part, cnt, stream);
    } else {
        if (L.sym) launch_variant<DT_F16, true>(X, packed, Y, M, L, p, part, cnt, stream);
        else launch_variant<DT_F16, false>(X, packed, Y, M, L, p, part, cnt, stream);
    }
    return hipGetLastError();
}

hipError_t launch_mfma_probe(const void* A, const void* B, float* D, bool bf16,
                             hipStream_t stream) {
    if (bf16)
        hipLaunchKernelGGL(mfma_probe_kernel<DT_BF16>, dim3(1), dim3(64), 0, stream,
                           (const uint16_t*)A, (const uint16_t*)B, D);
    else
        hipLaunchKernelGGL(mfma_probe_kernel<DT_F16>, dim3(1), dim3(64), 0, stream,
                           (const uint16_t*)A, (const uint16_t*)B, D);
    return hipGetLastError();
}

}  // namespace w4a16
