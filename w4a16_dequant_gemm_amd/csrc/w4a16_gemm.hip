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
//  * splitk_kernel (M <= 32).  Memory-bound streaming.  The weight chunks
//    (one 1 KiB chunk per k-step of a 128-column block) are dealt out in equal
//    contiguous ranges to every wave of the grid; each lane issues one
//    16-byte load per k-step, and each wave keeps the next 4-k-step batch in
//    flight while it computes the current one.  The activation rows come straight
//    from global memory (they are tiny and L2-resident).  Partial sums of a
//    column block split between waves are reduced through LDS and between
//    workgroups through a workspace, both in a fixed order.  The
//    multiply-accumulate runs on v_mfma_f32_32x32x16 even at M = 1: the
//    vector ALUs are the scarce resource on MI355X at this bandwidth (they
//    carry the unpack and dequant), while the matrix units are idle.
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
#include "w4a16_epilogue.h"
#include "w4a16_internal.h"

// This file is compiled once per (activation dtype, epilogue) pair, each
// object holding one quarter of the kernel instantiations (they compile in
// parallel): W4A16_TU_BF16 selects bf16 over fp16, W4A16_TU_EP the kernels
// with the output epilogue.  The (fp16, no epilogue) object also holds the
// MFMA layout probe.
#ifndef W4A16_TU_BF16
#define W4A16_TU_BF16 0
#endif
#ifndef W4A16_TU_EP
#define W4A16_TU_EP 0
#endif

namespace w4a16 {

namespace {


// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16*l (lds must be wave-uniform).  The builtin exists only for the
// device target, so the host pass sees an empty body.
__device__ __forceinline__ void load_to_lds16(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
#else
    (void)g;
    (void)lds;
#endif
}

// Workgroup barrier after this wave's loads (copies into LDS included) and
// LDS operations have all completed.
__device__ __forceinline__ void stage_barrier_all() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroup barrier between LDS stages: waits for this wave's LDS operations
// only, not for its vector memory loads (which stay in flight across it; the
// compiler waits for each where its value is used).  The asm statement also
// keeps the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void stage_barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

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
// Split-K streaming kernel, M <= 32.
//
// The weight chunks (one 1 KiB chunk = one k-step of one 128-column block)
// are grouped in batches of SK_U k-steps inside a column block; batch
// B = nb * nbat + i covers k-steps [i*SK_U, min(KS, (i+1)*SK_U)) of column
// block nb.  The TB = NB * nbat batches are dealt out in balanced contiguous
// ranges to every wave of the grid (one workgroup of SK_WAVES waves per CU,
// two waves per SIMD so that one wave's dequantization overlaps the other's
// matrix instructions).  A wave streams its range as one continuous
// pipeline: while it computes batch b, batch b+1 (weights, their scale/zero
// records and the activation operands) is in flight in registers, across
// column-block boundaries.  No barrier and no LDS traffic in the main loop.
// (Measured on MI355X: one batch ahead beats two or three -- with 16 waves'
// worth of loads per CU in flight the memory system is kept busy, and the
// smaller register footprint and loop body win over the deeper prefetch.)
//
// Where the range leaves a column block, a block the wave covered entirely
// is written to Y; the wave's first block, if partial, goes to the wave's LDS
// slot (its "head"); the last segment of the range stays in the accumulators
// (its "tail") and is written to Y at once if it is a whole block.  At the end
// the workgroup handles its partial blocks in increasing order: waves whose
// tail is that block copy it to their slot (free by then), and the slots are
// added in wave order.  A block inside the workgroup's range goes to Y; a block
// shared with other workgroups goes through the workspace: a partial tile per
// workgroup, a counter per block, and the last arrival adds the partial tiles
// in workgroup order (bitwise reproducible) and writes Y.
// ---------------------------------------------------------------------------
constexpr int SK_WAVES = kSplitKWaves;
constexpr int SK_U = kSplitKBatch;
constexpr int SK_NBUF = 2;   // batches held in registers per wave
// The 8-row split-K form reads X through a buffer resource: its lanes with
// an empty A block use an offset past the end (zeros); X's bytes stay at most
// kBdMaxXBytes so that every offset fits 32 bits.
constexpr uint32_t kBdPastEnd = 0x40000000u;
constexpr int64_t kBdMaxXBytes = (int64_t)1 << 30;

// Balanced contiguous split of TB batches over the grid's waves: wave gw
// starts at gw*base + min(gw, rem) and owns base (+1 if gw < rem) batches.
__device__ __forceinline__ int range_start(int gw, int base, int rem) {
    return gw * base + min(gw, rem);
}
__device__ __forceinline__ int wave_of_batch(int b, int base, int rem) {
    const int big = rem * (base + 1);
    return b < big ? b / (base + 1) : rem + (b - big) / base;
}

// The partial column blocks of the wave range [s, e): the head (first block,
// written to the LDS slot in the main loop) and the tail (last segment, left
// in the accumulators); -1 if none.
struct WaveParts {
    int head, tail;
};
__device__ __forceinline__ WaveParts wave_parts(int s, int e, int nbat) {
    WaveParts w{-1, -1};
    if (s >= e) return w;
    const int hb = s / nbat, tb = (e - 1) / nbat;
    if (hb != tb && s % nbat != 0) w.head = hb;
    if (!(e % nbat == 0 && (tb != hb || s % nbat == 0))) w.tail = tb;
    return w;
}

// MB: 8, 16 or 32 >= M (sizes the LDS slots).
template <int DT, bool SYM, int GS, int MB, bool EP>
__global__ __launch_bounds__(SK_WAVES * 64) void splitk_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed, uint16_t* __restrict__ Y,
    float* __restrict__ part, uint32_t* __restrict__ cnt, int M, int N, int K, int nbat, int base,
    int rem, size_t s_off, size_t z_off, size_t t_off, Epilogue ep) {
    constexpr int G = GS * kKStep;               // group size
    constexpr int EPB = kBodyK / G;              // groups per body
    constexpr int SE = 2 * EPB;                  // scale entry bytes
    constexpr int ZE = EPB / 2;                  // zero entry bytes
    constexpr int QMAX = MB / 8;                 // 8-row accumulator groups that can hold rows < M
    static_assert(SK_U == kChunkK / kKStep, "a batch is one chunk of each tile of the block");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wg = blockIdx.x;
    const int KC = K / kChunkK;
    const int KB = K / kBodyK;
    const int QM = (M + 7) >> 3;
    const int gw = wg * SK_WAVES + wave;
    const int s_w = range_start(gw, base, rem);
    const int len = base + (gw < rem ? 1 : 0);

    __shared__ f32x4 slots[SK_WAVES][4][QMAX][64];   // [wave][t][q][lane]
    __shared__ uint32_t s_last;
    __shared__ int s_prog[SK_WAVES];                 // batches computed, per wave
    __shared__ WaveParts s_parts[SK_WAVES];

    const bool exact = uses_exact_form<DT>(packed, t_off);
    // A operand of this lane: activation row min(lane%32, M-1) (rows >= M only
    // feed accumulator rows that are never stored), 8 halves at 8*(lane/32).
    const int arow = min(lane & 31, M - 1);
    const uint16_t* xlane = X + (size_t)arow * K + 8 * (lane >> 5);
    // MB = 8: v_mfma_f32_16x16x32 with a block-diagonal A operand, as in the
    // decode kernel (half the matrix-core cycles on the same B operands):
    // lane l is A row i = l % 16 of slot l / 16, X row i % 4 + 4 * (i / 8)
    // if row i's tile half (i / 4) % 2 is the slot's (l / 16) % 2 and that
    // row is < M; other lanes read zeros past the end of a buffer resource
    // over X.  The launcher uses it only while M * K * 2 <= 2^30.
    constexpr bool BD = MB == 8;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)X, (short)0, BD ? M * K * 2 : 0, kBufferRsrcWord3);
    uint32_t xoff = 0;
    if constexpr (BD) {
        const int ai = lane & 15;
        const int axr = (ai & 3) + 4 * (ai >> 3);
        const bool alive = ((ai >> 2) & 1) == ((lane >> 4) & 1) && axr < M;
        xoff = alive ? 2u * ((uint32_t)axr * (uint32_t)K + 8u * (uint32_t)(lane >> 5)) : kBdPastEnd;
    }
    const int c32 = lane & 31;
    const uint32_t lane16 = (uint32_t)lane * 16;

    // Batch i of block nb: chunk i (k-steps 4i..4i+3) of each of the block's
    // four tiles, and the scale/zero entries of the body that holds it.
    struct Batch {
        u32x4 w[4];          // tile t's chunk: word u = k-step u
        u32x4 x[SK_U];       // A operand of k-step u
        SEnt<G> s[4];
        uint32_t z[4];
    };

    // Loads of one batch, all unconditional so that the compiler can count
    // exactly how many are still in flight.  Past the end of the range they
    // read cache-resident data instead (the lane's activations and the first
    // scale/zero entries; values never used), so that the final wait for
    // outstanding loads does not wait for HBM.
    const int hb = s_w / nbat, ib = s_w - hb * nbat;   // first batch: block, batch in block
    int nbL = hb, iL = ib, issued = 0;
    auto issue = [&](Batch& b) {
        const bool real = issued < len;
        const int c = real ? iL : 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const size_t tile = real ? (size_t)4 * nbL + t : 0;
            const size_t ent = (tile * KB + (c >> 2)) * 32 + c32;
            b.s[t] = load_sent<G>(packed + s_off + ent * SE);
            b.z[t] = SYM ? 0u : load_zent<G>(packed + z_off + ent * ZE);
            b.w[t] = load_weights(real ? (const u32x4*)(packed + (tile * KC + c) * kChunkBytes + lane16)
                                       : (const u32x4*)xlane);
        }
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            if constexpr (BD)
                b.x[u] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               xrs, xoff + (uint32_t)(4 * c + u) * (2 * kKStep), 0, 0));
            else
                b.x[u] = *(const u32x4*)(xlane + (size_t)(4 * c + u) * kKStep);
        }
        ++issued;
        if (++iL == nbat) {
            iL = 0;
            ++nbL;
        }
    };

    using Acc = typename std::conditional<BD, f32x4, f32x16>::type;
    Acc acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = Acc{};
    const Magic mg = make_magic();
    const uint32_t zsh = zent_shift<G>(c32);   // this lane's zero entry in its dword

    // k-step u of batch i is k-step 4*(i % 4) + u of its body: group entry
    // (4*(i % 4) + u) / GS of the body's scale/zero entries.
    auto compute = [&](const Batch& b, int i, auto ex) {
        ColParams<DT> prm[4];
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            if (u % GS == 0) {
                const int e = (4 * (i & 3) + u) / GS;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    prm[t] = entry_params<DT, SYM>(b.s[t].word(e >> 1), b.z[t] >> zsh, e);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x4 bop = dequant_sel<decltype(ex)::value>(b.w[t][u], prm[t], mg);
                if constexpr (BD)
                    acc[t] = mfma16x16x32<DT>(b.x[u], bop, acc[t]);
                else
                    acc[t] = mfma32x32x16<DT>(b.x[u], bop, acc[t]);
            }
        }
    };

    auto to_slot = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < QMAX; ++q) {
            if (q >= QM) break;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                slots[wave][t][q][lane] = f32x4{acc[t][4 * q], acc[t][4 * q + 1],
                                                acc[t][4 * q + 2], acc[t][4 * q + 3]};
        }
    };

    // Accumulators of a whole column block straight to Y.
    auto to_y = [&](int nb) __attribute__((always_inline)) {
        const int64_t col0 = (int64_t)nb * kColBlock + (lane & 31);
        uint16_t* ybase = Y + (size_t)(4 * (lane >> 5)) * N + col0;
#pragma unroll
        for (int q = 0; q < QMAX; ++q) {
            if (q >= QM) break;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 8 * q + 4 * (lane >> 5) + i;
                    if (row < M)
                        ybase[(size_t)(8 * q + i) * N + 32 * t] =
                            out_value<DT, EP>(acc[t][4 * q + i], row, col0 + 32 * t, N, ep);
                }
        }
    };

    // Waves w and w + SK_WAVES/2 share a SIMD, whose arbiter favours the
    // older wave: left alone, that wave runs ahead and the other finishes its
    // equal share by itself at the end, without a partner to overlap its
    // matrix instructions with.  The wave that is behind its partner takes
    // the higher issue priority.
    // (LDS accesses through the __shared__ array itself: a generic pointer
    // would turn them into flat accesses, which count as vector memory
    // operations and would make the loop wait for every load in flight.)
    auto balance = [&](int done_batches) __attribute__((always_inline)) {
        __hip_atomic_store(&s_prog[wave], done_batches, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
        const int partner = __builtin_amdgcn_readfirstlane(__hip_atomic_load(
            &s_prog[wave ^ (SK_WAVES / 2)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (done_batches > partner)
            __builtin_amdgcn_s_setprio(0);
        else
            __builtin_amdgcn_s_setprio(1);
    };

    auto mainloop = [&](auto ex) {
        Batch bf[SK_NBUF];
#pragma unroll
        for (int i = 0; i < SK_NBUF - 1; ++i) issue(bf[i]);
        if (lane == 0) s_prog[wave] = 0;
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0) only: the first loads stay in flight
        __builtin_amdgcn_s_barrier();
        int nbC = hb, iC = ib, b = 0;
        // One loop exit; the batch count is rounded up to SK_NBUF with empty
        // trailing rounds (their loads are the harmless dummies above).
        do {
#pragma unroll
            for (int r = 0; r < SK_NBUF; ++r) {
                issue(bf[(r + SK_NBUF - 1) % SK_NBUF]);
                if (b < len) {
                    compute(bf[r], iC, ex);
                    const bool block_end = iC == nbat - 1;
                    const bool range_end = b == len - 1;
                    if (block_end || range_end) {
                        if (block_end && (nbC != hb || s_w % nbat == 0)) {
                            to_y(nbC);             // a whole block
                        } else if (!range_end) {
                            to_slot();             // the head
                        }
                        if (!range_end) {
#pragma unroll
                            for (int t = 0; t < 4; ++t) acc[t] = Acc{};
                        }
                    }
                    if (++iC == nbat) {
                        iC = 0;
                        ++nbC;
                    }
                    balance(b + 1);
                }
                ++b;
            }
        } while (b < len);
        __hip_atomic_store(&s_prog[wave], 1 << 30, __ATOMIC_RELAXED,   // finished: never
                           __HIP_MEMORY_SCOPE_WORKGROUP);               // hold the partner back
        __builtin_amdgcn_s_setprio(0);
    };
    if (exact)
        mainloop(std::true_type{});
    else
        mainloop(std::false_type{});

    // ---- workgroup epilogue: the partial blocks in increasing order.
    auto B0_of = [&](int g) { return range_start(g * SK_WAVES, base, rem); };   // first batch of g
    if (lane == 0) s_parts[wave] = wave_parts(s_w, s_w + len, nbat);
    __syncthreads();
    const int my_tail = s_parts[wave].tail;
    // Elements of a partial tile: (t, q) pairs of f32x4 per lane, pair t*QM + q
    // handled by wave (t*QM + q) % SK_WAVES.
    auto mine = [&](int t, int q) { return q < QM && ((t * QM + q) % SK_WAVES) == wave; };
    // The waves' partial blocks, read once into (wave-uniform) registers;
    // blocks are visited in increasing order, each once.
    int heads[SK_WAVES], tails[SK_WAVES];
#pragma unroll
    for (int w = 0; w < SK_WAVES; ++w) {
        const WaveParts pw = s_parts[w];
        heads[w] = __builtin_amdgcn_readfirstlane(pw.head);
        tails[w] = __builtin_amdgcn_readfirstlane(pw.tail);
    }
    auto next_part = [&](int after) {   // smallest partial block > after, or -1
        int n = 0x7fffffff;
#pragma unroll
        for (int w = 0; w < SK_WAVES; ++w) {
            if (heads[w] > after) n = min(n, heads[w]);
            if (tails[w] > after) n = min(n, tails[w]);
        }
        return n == 0x7fffffff ? -1 : n;
    };
    for (int nb = next_part(-1); nb >= 0; nb = next_part(nb)) {
        __syncthreads();   // the previous block's slots have been read
        if (my_tail == nb) to_slot();
        __syncthreads();
        const bool inside = nb * nbat >= B0_of(wg) && (nb + 1) * nbat <= B0_of(wg + 1);
        const int row0 = 4 * (lane >> 5);
        const size_t col0 = (size_t)nb * kColBlock + (lane & 31);
        // Shared with other workgroups: partial tile [t][row < M][32] into
        // this workgroup's workspace slot 0 (its first block) or 1 (its last).
        const int g0 = inside ? 0 : wave_of_batch(nb * nbat, base, rem) / SK_WAVES;
        const int g1 = inside ? 0 : wave_of_batch((nb + 1) * nbat - 1, base, rem) / SK_WAVES;
        const int tile_floats = 4 * M * 32;
        // Workgroups after g0 start inside block nb (their slot 0); g0 holds
        // it as its last block (slot 1) unless its range starts at nb too.
        const int s0 = inside ? 0 : 2 * g0 + (nb == B0_of(g0) / nbat ? 0 : 1);
        auto slot_of = [&](int g) {
            return part + (size_t)(g == g0 ? s0 : 2 * g) * tile_floats;
        };
        float* my_slot = slot_of(wg);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int q = 0; q < QMAX; ++q) {
                if (!mine(t, q)) continue;
                // the workgroup's partial of block nb: slots added in wave order
                f32x4 v = f32x4{};
                bool first = true;
#pragma unroll
                for (int w = 0; w < SK_WAVES; ++w) {
                    if (heads[w] != nb && tails[w] != nb) continue;
                    const f32x4 sv = slots[w][t][q][lane];
                    v = first ? sv : v + sv;
                    first = false;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 8 * q + row0 + j;
                    if (row >= M) continue;
                    if (inside)
                        Y[(size_t)row * N + col0 + 32 * t] =
                            out_value<DT, EP>(v[j], row, (int64_t)col0 + 32 * t, N, ep);
                    else
                        st_dev(&my_slot[(t * M + row) * 32 + (lane & 31)], v[j]);
                }
            }
        if (inside) continue;
        if (!arrive_last(&cnt[g0], g1 - g0 + 1, &s_last)) continue;
        // Last arrival: add the workgroups' tiles in workgroup order; thread
        // tid handles column tid % 32 of rows tid / 32 and tid / 32 + 16.
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = (tid >> 5) + 16 * i;
                if (row >= M) continue;
                const int f = (t * M + row) * 32 + (tid & 31);
                float sum = ld_dev(&slot_of(g0)[f]);
                for (int g = g0 + 1; g <= g1; ++g) sum += ld_dev(&slot_of(g)[f]);
                const int64_t col = (int64_t)nb * kColBlock + 32 * t + (tid & 31);
                Y[(size_t)row * N + col] = out_value<DT, EP>(sum, row, col, N, ep);
            }
        if (tid == 0) reset_counter(&cnt[g0]);
    }
}

// ---------------------------------------------------------------------------
// LDS-tiled kernel, M > 32.
//
// A workgroup of 8 waves owns ROWS = 32*MT rows by 512 columns.  Wave w
// owns the 64 columns of half w/4 of column block 4*blockIdx.x + w%4 for
// all ROWS rows: it dequantizes each of its weight words once and feeds it
// to MT row tiles.  Two waves share a SIMD (w and w+4), so one wave's
// dequantization runs while the other's matrix instructions execute -- a
// wave does not issue vector ALU work while its own MFMA executes, so a
// single wave per SIMD would add the two.  The activation tile of a stage
// (KT k-steps) is staged through LDS (copied straight into it for MT = 4),
// two or three stages deep, one barrier per stage.  LDS layout: 16-byte slot (row, chunk) holds halves 8*chunk..+7 of
// the stage's k range for that row, at position row*16 + (chunk ^ (row & 15))
// -- the XOR spreads the 16 rows a quarter-wave reads at one chunk over all
// banks.  Inside a stage the next k-step's A operands (LDS) and B operands
// (dequantized weights) are prepared before the current k-step's MFMAs.
// ---------------------------------------------------------------------------
constexpr int TK_WAVES = 8;

template <int DT, bool SYM, int GS, int MT, bool EP>
__global__ __launch_bounds__(TK_WAVES * 64) void tiled_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed, uint16_t* __restrict__ Y,
    float* __restrict__ part, uint32_t* __restrict__ cnt, int M, int N, int K,
    int steps_per_split, int S, size_t s_off, size_t z_off, size_t t_off,
    Epilogue ep) {
    constexpr int KT = kTiledStage;             // k-steps per stage
    constexpr int ROWS = 32 * MT;
    constexpr int CPR = 2 * KT;                 // 16-byte chunks per row and stage
    constexpr int SLOTS = ROWS * CPR;           // 16-byte slots per stage buffer
    constexpr int XI = SLOTS / (TK_WAVES * 64); // direct loads per thread and stage
    constexpr int SPG = GS < KT ? GS : KT;      // k-steps per group inside a stage
    constexpr int NGST = KT / SPG;              // groups per stage
    static_assert(CPR == 16, "the swizzle assumes 16 chunks per row");
    static_assert(2 * XI <= KT, "the activation copies of a stage fit in its first half");
    constexpr int NW = MT == 2 ? 3 : 2;         // stages in flight (LDS buffers, weight sets)
    __shared__ __align__(16) u32x4 xs0[SLOTS];
    __shared__ __align__(16) u32x4 xs1[SLOTS];
    __shared__ __align__(16) u32x4 xs2[NW == 3 ? SLOTS : 1];
    __shared__ uint32_t s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int half = wave >> 2;                 // column tiles 2*half, 2*half+1 of the block
    constexpr int G = GS * kKStep;              // group size
    constexpr int EPB = kBodyK / G;             // groups per body
    constexpr int SE = 2 * EPB;                 // scale entry bytes (a body)
    constexpr int ZE = EPB / 2;                 // zero entry bytes (a body)
    const int NB = N / kColBlock;
    const int KS = K / kKStep;
    const int KC = K / kChunkK;
    const int KB = K / kBodyK;
    const int nb = blockIdx.x * 4 + (wave & 3);
    const bool nb_ok = nb < NB;
    const int nbc = nb_ok ? nb : NB - 1;
    const int m0 = blockIdx.y * ROWS;
    const int split = blockIdx.z;
    const int s_beg = split * steps_per_split;   // a multiple of 2*KT (a body)
    const int s_end = min(KS, s_beg + steps_per_split);
    const int nst = s_end > s_beg ? (s_end - s_beg) / KT : 0;

    // this wave's two tiles: 4*nb + 2*half + tt; chunk c of tile t at
    // (t*KC + c) KiB, lane l's 16 bytes at l*16
    const size_t tile0 = (size_t)4 * nbc + 2 * half;
    const uint8_t* wbase = packed + tile0 * KC * kChunkBytes + (uint32_t)lane * 16;
    const uint8_t* sbase = packed + s_off + (tile0 * KB * 32 + (lane & 31)) * SE;
    const uint8_t* zbase = packed + z_off + (tile0 * KB * 32 + (lane & 31)) * ZE;

    // Activation copies: copy i of this thread covers slot
    // s = (8*i + wave)*64 + lane, i.e. row s/16 (rows >= M re-read row M-1,
    // never stored), position s%16 = lane%16, which holds chunk
    // (lane%16) ^ (row & 15); row & 15 does not depend on i.
    //  * MT = 4: straight from global memory into LDS (global_load_lds, no
    //    registers: MT = 4 has none to spare).  The compiler cannot tell
    //    which loads such a copy depends on and waits for all loads in
    //    flight before it next reads a loaded register, so the next stage's
    //    loads are issued only after this stage's first operands are read.
    //  * MT = 2: global -> VGPR one stage ahead of the LDS store, which keeps
    //    every wait exact and allows a third stage in flight.
    constexpr bool DMA = MT == 4;
    const int xchunk = (lane & 15) ^ ((4 * wave + (lane >> 4)) & 15);
    const uint16_t* xrow[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i)
        xrow[i] = X + (size_t)min(m0 + (TK_WAVES * i + wave) * 4 + (lane >> 4), M - 1) * K;
    u32x4 xr[DMA ? 1 : XI];
    auto x_col = [&](int si) {
        const int st = s_beg + min(si, nst - 1) * KT;
        return min(kKStep * st + 8 * xchunk, K - 8);   // past K: never used
    };
    // The loads of one stage come in parts, one call per k-step of the stage
    // before, so that they interleave with its matrix instructions.
    auto load_x_part = [&](int si, int i) {   // MT = 2: copy i into xr[i]
        if constexpr (!DMA) xr[i] = *(const u32x4*)(xrow[i] + x_col(si));
    };
    auto store_x_part = [&](u32x4* buf, int i) {   // MT = 2
        if constexpr (!DMA) buf[(TK_WAVES * i + wave) * 64 + lane] = xr[i];
    };
    auto copy_x_part = [&](u32x4* buf, int si, int i) {   // MT = 4: straight into LDS
        load_to_lds16(xrow[i] + x_col(si), &buf[(TK_WAVES * i + wave) * 64]);
    };

    // One stage (KT = 8 k-steps, half a body): chunks 2c', 2c'+1 of both tiles
    // (c' = the stage's index), the stage's scales and the tiles' zero entries
    // of the body.  Scales: G = 128, the body's two (the stage uses half
    // `par`); G = 64 and 32, the stage's half of the body entry (2 or 4
    // scales).  All loads are dword-aligned (see load_zent).
    struct Stage {
        uint32_t sc[2][NGST > 2 ? 2 : 1];   // scale dwords of tile tt (two scales each)
        uint32_t zw[2];                      // the dword holding tile tt's zero entry
        u32x4 w[2][2];                       // [tile][chunk]: word u = k-step u of the chunk
    };
    auto load_w_part = [&](Stage& b, int si, int part) {
        const int st = s_beg + min(si, nst - 1) * KT;   // first k-step of the stage
        const int tt = part & 1, cc = part >> 1;
        if (part == 0) {
            const int body = st >> 4, par = (st >> 3) & 1;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint8_t* se = sbase + ((size_t)t * KB + body) * 32 * SE;
                if constexpr (NGST == 1) {
                    b.sc[t][0] = *(const uint32_t*)se;
                } else if constexpr (NGST == 2) {
                    b.sc[t][0] = *(const uint32_t*)(se + par * (SE / 2));
                } else {
                    const u32x2 v = *(const u32x2*)(se + par * (SE / 2));
                    b.sc[t][0] = v.x;
                    b.sc[t][NGST > 2 ? 1 : 0] = v.y;
                }
                b.zw[t] = SYM ? 0u : load_zent<G>(zbase + ((size_t)t * KB + body) * 32 * ZE);
            }
        }
        b.w[tt][cc] = __builtin_nontemporal_load(
            (const u32x4*)(wbase + ((size_t)tt * KC + (st >> 2) + cc) * kChunkBytes));
    };
    auto load_w = [&](Stage& b, int si) {
#pragma unroll
        for (int p = 0; p < 4; ++p) load_w_part(b, si, p);
    };

    const Magic mg = make_magic();
    const uint32_t zsh = zent_shift<G>(lane & 31);   // this lane's zero entry in its dword
    f32x16 acc[MT][2];
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) acc[r][tt] = f32x16{};

    // A operand of row tile r at k-step u: row 32r + lane%32, chunk
    // 2u + lane/32, stored at position (2u + lane/32) ^ (lane & 15) =
    // 2u ^ ((lane/32) ^ (lane & 15)).
    const int aswz = (lane >> 5) ^ (lane & 15);
    const int arow = (lane & 31) * CPR;
    // One stage.  The operands of k-step 0 are prepared first; during k-step
    // u the wave prepares those of k-step u+1 between its matrix
    // instructions: while the MT MFMAs of column tile 0 run, tile 1's next
    // weight word is dequantized into a spare register; while those of tile
    // 1 run (tile 0's B operand is free by then), tile 0's next word, and the
    // next A operands are read from LDS as each row tile's last MFMA has
    // issued.  A wave hides a few vector instructions under each of its own
    // MFMAs, and the other wave on the SIMD fills the rest.  issue(u) issues
    // part u of a later stage's loads.
    auto compute = [&](const Stage& b, const u32x4* buf, int si, auto exact, auto issue) {
        auto read_a = [&](u32x4 (&a)[MT], int u) {
#pragma unroll
            for (int r = 0; r < MT; ++r) a[r] = buf[arow + 32 * CPR * r + ((2 * u) ^ aswz)];
        };
        const int par = ((s_beg + si * KT) >> 3) & 1;   // stage inside its body
        auto make_b1 = [&](int u, int tt) {
            const int j = u / SPG;                 // group of k-step u inside the stage
            const uint32_t sw = NGST == 1 ? b.sc[tt][0] >> (16 * par) : b.sc[tt][j >> 1];
            const uint32_t zw = SYM ? 0u : b.zw[tt] >> (zsh + 4 * NGST * par);
            const ColParams<DT> prm = entry_params<DT, SYM>(sw, zw, NGST == 1 ? 0 : j);
            return dequant_sel<decltype(exact)::value>(b.w[tt][u >> 2][u & 3], prm, mg);
        };
        if (si >= nst) return;   // a stage past the last one: nothing to do
        u32x4 a[MT], bo[2];
        read_a(a, 0);
        bo[0] = make_b1(0, 0);
        bo[1] = make_b1(0, 1);
        {
#pragma unroll
            for (int u = 0; u < KT; ++u) {
                __builtin_amdgcn_sched_barrier(0);
                issue(u);
                const bool nx = u + 1 < KT;
                u32x4 bn1;
#pragma unroll
                for (int r = 0; r < MT; ++r) acc[r][0] = mfma32x32x16<DT>(a[r], bo[0], acc[r][0]);
                if (nx) bn1 = make_b1(u + 1, 1);
#pragma unroll
                for (int r = 0; r < MT; ++r) acc[r][1] = mfma32x32x16<DT>(a[r], bo[1], acc[r][1]);
                if (nx) {
                    bo[0] = make_b1(u + 1, 0);
                    read_a(a, u + 1);
                    bo[1] = bn1;
                }
                // MFMA / vector ALU / LDS-read interleave of this k-step
#pragma unroll
                for (int r = 0; r < MT; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 20 / MT, 0);
                }
#pragma unroll
                for (int r = 0; r < MT; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 20 / MT, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // NW stages in flight.  Stage i computes from LDS buffer i%NW and weight
    // set i%NW.  MT = 2 (NW = 3), during stage i: the activations of stage i+1
    // (in VGPRs since stage i-1) go to LDS buffer (i+1)%3, those of stage i+2
    // are loaded into the VGPRs, and the weights of stage i+2 into set
    // (i+2)%3 -- the activation loads first, so that waiting for them never
    // waits for the younger weight loads; one barrier per stage, for LDS only.
    // MT = 4 (NW = 2), during stage i: stage i+1's activations are copied into
    // LDS buffer (i+1)%2 and its weights loaded into set (i+1)%2; the barrier
    // at the end of stage i waits for all of them.  One loop exit; a stage
    // index >= nst loads in-bounds dummies and computes nothing.
    auto mainloop = [&](auto exact) {
        if constexpr (NW == 3) {
            Stage A, B, C;
#pragma unroll
            for (int i = 0; i < XI; ++i) load_x_part(0, i);
            load_w(A, 0);
            load_w(B, 1);
#pragma unroll
            for (int i = 0; i < XI; ++i) store_x_part(xs0, i);
#pragma unroll
            for (int i = 0; i < XI; ++i) load_x_part(1, i);
            stage_barrier_lds();
            // during stage i: at k-step 0 the activations of stage i+1 (in xr
            // since k-step 0 of stage i-1) go to LDS and those of stage i+2 are
            // loaded into xr -- first, so that waiting for them never waits
            // for the weight loads after them; the weights of stage i+2 two
            // k-steps at a time in the first half of the stage
            auto part = [&](u32x4* to, int si, Stage& w, int u) {
                if (u == 0) {
#pragma unroll
                    for (int i = 0; i < XI; ++i) store_x_part(to, i);
#pragma unroll
                    for (int i = 0; i < XI; ++i) load_x_part(si, i);
                }
                if (u < 4) load_w_part(w, si, u);
            };
            int i = 0;
            do {
                compute(A, xs0, i, exact, [&](int u) { part(xs1, i + 2, C, u); });
                stage_barrier_lds();
                compute(B, xs1, i + 1, exact, [&](int u) { part(xs2, i + 3, A, u); });
                stage_barrier_lds();
                compute(C, xs2, i + 2, exact, [&](int u) { part(xs0, i + 4, B, u); });
                stage_barrier_lds();
                i += 3;
            } while (i < nst);
        } else {
            Stage A, B;
#pragma unroll
            for (int i = 0; i < XI; ++i) copy_x_part(xs0, 0, i);
            load_w(A, 0);
            stage_barrier_all();
            // during stage i: stage i+1's activations are copied into LDS and
            // its weights loaded in the first half of the stage (one copy and
            // two weight loads per k-step), so that all of them have the
            // second half to arrive before the barrier that ends the stage
            auto part = [&](u32x4* to, int si, Stage& w, int u) {
                if (u < XI) copy_x_part(to, si, u);
                if (u < 4) load_w_part(w, si, u);
            };
            int i = 0;
            do {
                compute(A, xs0, i, exact, [&](int u) { part(xs1, i + 1, B, u); });
                stage_barrier_all();
                compute(B, xs1, i + 1, exact, [&](int u) { part(xs0, i + 2, A, u); });
                stage_barrier_all();
                i += 2;
            } while (i < nst);
        }
    };
    if (nst > 0) {
        if (uses_exact_form<DT>(packed, t_off))
            mainloop(std::true_type{});
        else
            mainloop(std::false_type{});
    }

    const int64_t colw = (int64_t)nb * kColBlock + 64 * half + (lane & 31);
    if (S == 1) {
        if (nb_ok) {
#pragma unroll
            for (int r = 0; r < MT; ++r)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int rr = m0 + 32 * r + acc_row(i, lane);
                        if (rr < M)
                            Y[(int64_t)rr * N + colw + 32 * tt] =
                                out_value<DT, EP>(acc[r][tt][i], rr, (int64_t)colw + 32 * tt, N, ep);
                    }
        }
        return;
    }

    // Cross-workgroup reduction.  A split's partial tile is Q chunks of four
    // accumulator registers per lane, chunk q of wave w at 16-byte slot
    // (w*Q + q)*64 + lane: each store and load instruction of a wave moves
    // 1 KiB, through device-scope (sc1) buffer accesses.
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;
    constexpr int Q = MT * 2 * 4;                               // chunks per lane
    constexpr uint32_t slot_bytes = TK_WAVES * Q * 64 * 16;    // one split's tile
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        part + (size_t)tile * S * (slot_bytes / 4), (short)0, (int)(S * slot_bytes), kBufferRsrcWord3);
    const uint32_t lane_off = ((uint32_t)wave * Q * 64 + lane) * 16;
    auto chunk = [&](int q) {   // registers 4j..4j+3 of tile (r, tt), q = (2r + tt)*4 + j
        const f32x16& c = acc[q >> 3][(q >> 2) & 1];
        const int j = q & 3;
        return f32x4{c[4 * j], c[4 * j + 1], c[4 * j + 2], c[4 * j + 3]};
    };
#pragma unroll
    for (int q = 0; q < Q; ++q)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, chunk(q)), rs,
                                               (int)(split * slot_bytes + lane_off + q * 1024), 0,
                                               kDeviceScope);
    if (!arrive_last(&cnt[tile], S, &s_last)) return;

    // Sum the S partials in split order 0..S-1 (this workgroup's own from its
    // registers, the same values that it stored), QG chunks at a time, with
    // the loads of up to SB splits in flight together.
    constexpr int QG = 4, SB = 4;
    auto load_chunk = [&](int sp, int q) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rs, (int)(sp * slot_bytes + lane_off + q * 1024), 0,
                                             kDeviceScope));
    };
#pragma unroll
    for (int q0 = 0; q0 < Q; q0 += QG) {
        f32x4 v[QG];
#pragma unroll
        for (int g = 0; g < QG; ++g) v[g] = split == 0 ? chunk(q0 + g) : load_chunk(0, q0 + g);
        for (int s0 = 1; s0 < S; s0 += SB) {
            f32x4 t[SB][QG];
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                const int sp = min(s0 + k, S - 1);
#pragma unroll
                for (int g = 0; g < QG; ++g) t[k][g] = sp == split ? chunk(q0 + g) : load_chunk(sp, q0 + g);
            }
#pragma unroll
            for (int k = 0; k < SB; ++k)
                if (s0 + k < S) {
#pragma unroll
                    for (int g = 0; g < QG; ++g) v[g] += t[k][g];
                }
        }
        if (nb_ok) {
#pragma unroll
            for (int g = 0; g < QG; ++g) {
                const int q = q0 + g;
                const int r = q >> 3, tt = (q >> 2) & 1, j = q & 3;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int rr = m0 + 32 * r + acc_row(4 * j + e, lane);
                    if (rr < M)
                        Y[(int64_t)rr * N + colw + 32 * tt] =
                            out_value<DT, EP>(v[g][e], rr, (int64_t)colw + 32 * tt, N, ep);
                }
            }
        }
    }
    if (tid == 0) reset_counter(&cnt[tile]);
}
// ---------------------------------------------------------------------------
// One MFMA with the kernels' operand and accumulator placement.
// ---------------------------------------------------------------------------
#if !W4A16_TU_BF16 && !W4A16_TU_EP
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
#endif

template <int DT, bool SYM, int GS, int MB>
void launch_splitk_mb(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                      const Plan& p, float* part, uint32_t* cnt, hipStream_t stream,
                   const Epilogue& ep) {
    hipLaunchKernelGGL((splitk_kernel<DT, SYM, GS, MB, W4A16_TU_EP != 0>), dim3(p.grid_x),
                       dim3(SK_WAVES * 64), 0, stream, (const uint16_t*)X, (const uint8_t*)packed,
                       (uint16_t*)Y, part, cnt, (int)M, (int)L.N, (int)L.K, p.nbat, p.base,
                       p.rem, L.s_off, L.z_off, L.t_off, ep);
}

template <int DT, bool SYM, int GS>
void launch_splitk(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                   const Plan& p, float* part, uint32_t* cnt, hipStream_t stream,
                   const Epilogue& ep) {
    // the 8-row form addresses X with 32-bit buffer offsets
    if (M <= 8 && M * L.K * 2 <= kBdMaxXBytes)
        launch_splitk_mb<DT, SYM, GS, 8>(X, packed, Y, M, L, p, part, cnt, stream, ep);
    else if (M <= 16) launch_splitk_mb<DT, SYM, GS, 16>(X, packed, Y, M, L, p, part, cnt, stream, ep);
    else launch_splitk_mb<DT, SYM, GS, 32>(X, packed, Y, M, L, p, part, cnt, stream, ep);
}

template <int DT, bool SYM, int GS, int MT>
void launch_tiled_mt(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                     const Plan& p, float* part, uint32_t* cnt, hipStream_t stream,
                     const Epilogue& ep) {
    hipLaunchKernelGGL((tiled_kernel<DT, SYM, GS, MT, W4A16_TU_EP != 0>),
                       dim3(p.grid_x, p.grid_y, p.grid_z), dim3(TK_WAVES * 64), 0, stream,
                       (const uint16_t*)X, (const uint8_t*)packed, (uint16_t*)Y, part, cnt, (int)M,
                       (int)L.N, (int)L.K, p.steps_per_split, p.splits, L.s_off, L.z_off, L.t_off,
                       ep);
}

template <int DT, bool SYM, int GS>
void launch_tiled(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                  const Plan& p, float* part, uint32_t* cnt, hipStream_t stream,
                  const Epilogue& ep) {
    if (p.mt == 2) launch_tiled_mt<DT, SYM, GS, 2>(X, packed, Y, M, L, p, part, cnt, stream, ep);
    else launch_tiled_mt<DT, SYM, GS, 4>(X, packed, Y, M, L, p, part, cnt, stream, ep);
}

template <int DT, bool SYM>
void launch_variant(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                    const Plan& p, float* part, uint32_t* cnt, hipStream_t stream,
                   const Epilogue& ep) {
    const int GS = (int)(L.G / kKStep);
    if (p.variant == VARIANT_SPLITK) {
        if (GS == 8) launch_splitk<DT, SYM, 8>(X, packed, Y, M, L, p, part, cnt, stream, ep);
        else if (GS == 4) launch_splitk<DT, SYM, 4>(X, packed, Y, M, L, p, part, cnt, stream, ep);
        else launch_splitk<DT, SYM, 2>(X, packed, Y, M, L, p, part, cnt, stream, ep);
    } else {
        if (GS == 8) launch_tiled<DT, SYM, 8>(X, packed, Y, M, L, p, part, cnt, stream, ep);
        else if (GS == 4) launch_tiled<DT, SYM, 4>(X, packed, Y, M, L, p, part, cnt, stream, ep);
        else launch_tiled<DT, SYM, 2>(X, packed, Y, M, L, p, part, cnt, stream, ep);
    }
}

}  // namespace

// This object's share of launch_gemm: one activation dtype, with or without
// the epilogue.
#if W4A16_TU_BF16
#if W4A16_TU_EP
#define W4A16_TU_ENTRY launch_gemm_bf16_ep
#else
#define W4A16_TU_ENTRY launch_gemm_bf16
#endif
#else
#if W4A16_TU_EP
#define W4A16_TU_ENTRY launch_gemm_f16_ep
#else
#define W4A16_TU_ENTRY launch_gemm_f16
#endif
#endif

hipError_t W4A16_TU_ENTRY(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                          const Plan& p, void* workspace, const Epilogue& ep,
                          hipStream_t stream) {
    constexpr int DT = W4A16_TU_BF16 ? DT_BF16 : DT_F16;
    uint32_t* cnt = nullptr;
    float* part = nullptr;
    if (p.splits > 1) {
        cnt = (uint32_t*)workspace;
        part = (float*)((uint8_t*)workspace + p.counters_bytes);
    }
    if (L.sym) launch_variant<DT, true>(X, packed, Y, M, L, p, part, cnt, stream, ep);
    else launch_variant<DT, false>(X, packed, Y, M, L, p, part, cnt, stream, ep);
    return hipGetLastError();
}

#if !W4A16_TU_BF16 && !W4A16_TU_EP
// Read-bandwidth probe: the decode kernel's load pattern with no compute.
// The buffer is nchunk 1 KiB chunks, dealt out in balanced contiguous ranges
// to the grid's waves; each lane issues one 16-byte non-temporal load per
// chunk, two batches of two chunks in flight, and XORs what it read (each
// chunk exactly once; clamped duplicate loads past a range are not counted).
// Thread gid writes its XOR to out[gid], so XOR-ing out gives the XOR of the
// whole buffer.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ buf,
                                                                 int64_t nchunk,
                                                                 u32x4* __restrict__ out) {
    constexpr int U = 2;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * (kProbeThreads / 64);
    const int64_t gw = (int64_t)blockIdx.x * (kProbeThreads / 64) + wave;
    const int64_t base = nchunk / nw, rem = nchunk % nw;
    const int64_t s = gw * base + min(gw, rem);
    const int64_t len = base + (gw < rem ? 1 : 0);
    u32x4 acc = {0u, 0u, 0u, 0u};
    if (len > 0) {
        const u32x4* p = buf + s * 64 + lane;
        u32x4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = __builtin_nontemporal_load(p + min((int64_t)u, len - 1) * 64);
        for (int64_t i = 0; i < len; i += 2 * U) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                b[u] = __builtin_nontemporal_load(p + min(i + U + u, len - 1) * 64);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (i + u < len) acc ^= a[u];
#pragma unroll
            for (int u = 0; u < U; ++u)
                a[u] = __builtin_nontemporal_load(p + min(i + 2 * U + u, len - 1) * 64);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (i + U + u < len) acc ^= b[u];
        }
    }
    out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, void* out, hipStream_t stream) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                       (const u32x4*)buf, (int64_t)(bytes / kChunkBytes), (u32x4*)out);
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
#endif

}  // namespace w4a16
