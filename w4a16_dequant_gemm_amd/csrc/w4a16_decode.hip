// w4a16_decode.hip -- the small-M (decode) fused W4A16 dequantize-GEMM kernel
// for gfx950.
//
// Page "W4A16 GEMM 算子浅析" (nxmr.cn), section "硬件性能拐点": at batch 1-8
// the product is bound by the weight stream; page "量化开销对比"
// (laojiahuo2003.github.io), section 6.5: the weights are read exactly once,
// reuse is along N, and the weight bytes divided by the bandwidth are the
// time floor.  Section 6.2: per output tile, walk along k, unpack each weight
// word, apply the group scale and zero before the multiply-accumulate, keep
// the accumulators in registers, with the next loads in flight.
//
// Work decomposition.  An item is TPI tiles (32 columns each) over all of K.
// A workgroup of 8 waves takes items blockIdx.x, blockIdx.x + gridDim.x, ...
// (one workgroup per CU); its waves split K into equal ranges of bodies (256
// of K each), so every wave streams contiguous 4 KiB runs of each tile.  An
// item's partial tiles are added in LDS in wave order and stored by the
// workgroup itself: no partial sum ever leaves the CU, there is no workspace
// and nothing waits on another workgroup.
//
// Streaming.  Each wave keeps PB bodies of weights (4 KiB per tile each) and
// their scale/zero entries in flight in registers while it computes the
// current body, across item boundaries; the loads of a future body are
// issued unconditionally (a clamped address past the wave's last body) so the
// compiler can count exactly how many are outstanding.
//
// Activations.  X (M rows of K) is copied into LDS once per workgroup, rows
// padded by 16 bytes so that the rows a quarter-wave reads at one k sit in
// different banks; the A operand of each k-step is one ds_read_b128 per lane.
//
// MFMA: v_mfma_f32_16x16x32_{f16,bf16}, one per (k-step of 16, tile), half
// the matrix-core cycles of the 32x32x16 form whose B operand the weight
// words are laid out for.  B operand = lane l's dequantized word as it is:
// column c = l % 32 of the tile, k = 8 * (l / 32) .. +7 of the k-step.  In
// the 16x16x32 instruction lane l feeds column l % 16 and reduction slot
// o = l / 16, so slot o carries the columns of half h = o % 2 of the tile
// (c = 16h + l % 16) at k-half o / 2.  The A operand is block diagonal: row
// i of the 16 belongs to half h(i) = (i / 4) % 2 and holds X row
// x(i) = i % 4 + 4 * (i / 8) in the slots of its own half and zeros in the
// other two (and zeros if x(i) >= M), so that D row i, column j sums column
// 16 h(i) + j of the tile only.  With that assignment lane l's accumulator
// register r is column c = l % 32, X row 4 * (l / 32) + r: the lane's own
// column, the same placement as registers 0..3 of the 32x32 form.  Zero
// operands are read from a 512-byte zero strip in LDS.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "w4a16_device.h"
#include "w4a16_epilogue.h"
#include "w4a16_internal.h"

#ifndef W4A16_TU_BF16
#define W4A16_TU_BF16 0
#endif
#ifndef W4A16_TU_EP
#define W4A16_TU_EP 0
#endif

namespace w4a16 {

namespace {

constexpr int DW = kDecodeWaves;   // waves per workgroup

template <int DT, bool SYM, int G, int MB, int TPI, int PB, bool EP>
__global__ __launch_bounds__(DW * 64) void decode_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed, uint16_t* __restrict__ Y,
    int M, int N, int K, int n_items, int tail_items, int tail_parts, uint8_t* __restrict__ ws,
    size_t s_off, size_t z_off, size_t t_off, Epilogue ep) {
    constexpr int EPB = kBodyK / G;          // groups per body: 2, 4, 8
    constexpr int GS = G / kKStep;           // k-steps per group: 8, 4, 2
    constexpr int SE = 2 * EPB;              // scale entry bytes
    constexpr int ZE = EPB / 2;              // zero entry bytes
    constexpr int QMAX = MB / 8;             // 8-row accumulator groups that can hold rows < M
    constexpr int R = PB + 1;                // bodies held per wave (ring)
    constexpr int EARLY = kDecodeEarlyBodies < PB ? kDecodeEarlyBodies : PB;
    // Scale after the product (fp16, at most 8 rows): each group's MFMAs
    // multiply X by the exact (q - z) into a temporary accumulator t (zeroed
    // at the start of each group), then acc += s * t, one fp32 fma per
    // register instead of a v_pk_mul_f16 per weight pair (every register of
    // a lane is its own column, whose scale it holds).  The sum differs from the dequantized-weight product
    // only by the rounding of each weight to fp16 (at most 2^-11 of each
    // term), and stays exact where the pages' result is: q = z gives products
    // of exact zeros, a one-hot row gives s * (q - z) rounded once.
    constexpr bool SA = kDecodeScaleAfter && DT == DT_F16 && MB == 8 && TPI == 1;
    static_assert(MB == 8, "one 8-row group: the 16x16x32 tile holds 2 x 8 rows");
    extern __shared__ __align__(16) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KC = K / kChunkK;
    const int KB = K / kBodyK;
    const int QM = (M + 7) >> 3;
    // this wave's bodies of every item: [b0, b0 + nbw)
    const int bbase = KB / DW, brem = KB % DW;
    const int b0 = wave * bbase + min(wave, brem);
    const int nbw = bbase + (wave < brem ? 1 : 0);
    // This workgroup's items.  Without a tail split (tail_parts == 1) it runs
    // items g, g + W, g + 2W, ... (W workgroups).  With one (S = tail_parts
    // > 1) the last tail_items items are split along K into S parts, so that
    // every workgroup gets the same share of the work: workgroup g <
    // tail_items * S first runs part g % S of item F*W + g / S, then the full
    // items g, g + W, ..., g + (F-1)*W, F = (n_items - tail_items) / W.  Part
    // p of an item is, in every wave, the bodies b0 + p, b0 + p + S, ... of
    // the wave's own range (the plan keeps S <= KB / 8, so each wave has at
    // least one), so X is staged once for both kinds of item.
    const int W = (int)gridDim.x, g = (int)blockIdx.x;
    const int S = tail_parts;
    const int F = S > 1 ? (n_items - tail_items) / W : (n_items - g + W - 1) / W;
    const bool has_tail = S > 1 && g < tail_items * S;
    const int tail_idx = S > 1 ? g / S : 0;          // index among the split items
    const int tail_item = F * W + tail_idx;
    const int tp = g - tail_idx * S;                 // part
    const int ntb = has_tail ? (nbw - tp + S - 1) / S : 0;
    const int n_seq = F + (has_tail ? 1 : 0);        // items in this workgroup's sequence
    const int nsteps = ntb + F * nbw;
    auto is_tail = [&](int j) { return has_tail && j == 0; };
    auto item_of = [&](int j) { return is_tail(j) ? tail_item : (j - (has_tail ? 1 : 0)) * W + g; };
    auto body_of = [&](int j, int i) { return is_tail(j) ? b0 + tp + i * S : b0 + i; };
    auto len_of = [&](int j) { return is_tail(j) ? ntb : nbw; };

    // LDS: X rows (row stride RS bytes), the partial-tile slots of two
    // items, their two arrival counters, two counts of reduced items, the
    // waves' progress counters and the zero strip
    const int RS = 2 * K + 16;
    f32x4* slots = (f32x4*)(lds + (size_t)M * RS);   // [2][DW][TPI][QMAX][64]
    uint32_t* cnt = (uint32_t*)(slots + 2 * DW * TPI * QMAX * 64);
    uint32_t* prog = cnt + 4;                        // [DW] bodies computed per wave
    u32x4* zstrip = (u32x4*)(prog + DW);             // kDecodeZeroBytes of zeros
    auto slot = [&](int par, int w, int tt, int q) -> f32x4& {
        return slots[(((par * DW + w) * TPI + tt) * QMAX + q) * 64 + lane];
    };
    const bool exact = [&] {
        if constexpr (DT == DT_F16) {
            return false;
        } else {
            return (*(const uint32_t*)(packed + t_off + 8) & kFlagExactBf16) != 0;
        }
    }();

    // ---- one body's loads: TPI tiles x 4 chunks, and their scale/zero entries
    struct Bundle {
        u32x4 w[TPI][4];
        SEnt<G> s[TPI];
        uint32_t z[TPI];
    };
    const uint32_t lane16 = (uint32_t)lane * 16;
    const int c32 = lane & 31;
    // issue cursor: item j of this workgroup's sequence, its body ib of this
    // wave; past the last body it stays on the last one (cached, never used).
    // Every call issues the same loads, so the compiler counts them exactly.
    int ij = 0, ib = 0;
    auto issue = [&](Bundle& B) {
        const bool real = ij < n_seq;
        const int j = real ? ij : n_seq - 1;
        const int b = body_of(j, real ? ib : len_of(j) - 1);
        const int item = item_of(j);
#pragma unroll
        for (int tt = 0; tt < TPI; ++tt) {
            const int t = item * TPI + tt;
            const uint8_t* wb = packed + ((size_t)t * KC + 4 * (size_t)b) * kChunkBytes + lane16;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
                B.w[tt][cc] = __builtin_nontemporal_load((const u32x4*)(wb + cc * kChunkBytes));
            const size_t ent = ((size_t)t * KB + b) * 32 + c32;
            B.s[tt] = load_sent<G>(packed + s_off + ent * SE);
            B.z[tt] = SYM ? 0u : load_zent<G>(packed + z_off + ent * ZE);
        }
        if (++ib >= len_of(ij)) {
            ib = 0;
            ++ij;
        }
    };

    // ---- X into LDS, and the first PB bodies' loads.  A wave reads X only in
    // the K range of its own bodies (the same range in every item), so it
    // stages just that slice of every row: no other wave waits for it and no
    // workgroup barrier follows (a wave still issuing its loads, which the
    // memory pipeline throttles at the start, holds nobody back).  The slice's
    // first pieces (16 bytes, NP per lane, NP the power of two that covers
    // them, at most 16) are loaded first, then the first EARLY bodies; each
    // piece is written to LDS as soon as it has arrived, which waits for the
    // X loads only, not for the bodies behind them.  Loads are unconditional
    // at clamped addresses so that the compiler counts exactly how many are
    // outstanding; a piece past the end is the last one again, written back
    // to its own place.  Slices of more than 16 pieces per lane continue 16 at
    // a time, then the remaining bodies are issued.
    Bundle ring[R];
    const int ppr = nbw * (kBodyK / 8);            // pieces per row of this wave's slice
    const int npc = M * ppr;                       // pieces of the slice
    const int xk0 = b0 * kBodyK;                   // first k of the slice
    auto piece_load = [&](int v) {
        v = min(v, npc - 1);
        const int row = v / ppr;
        return *(const u32x4*)(X + (size_t)row * K + xk0 + (v - row * ppr) * 8);
    };
    auto piece_store = [&](int v, const u32x4& x) {
        v = min(v, npc - 1);
        const int row = v / ppr;
        *(u32x4*)(lds + (size_t)row * RS + (size_t)(xk0 + (v - row * ppr) * 8) * 2) = x;
    };
    auto stage = [&](auto np_) {
        constexpr int NP = decltype(np_)::value;
        u32x4 xv[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) xv[i] = piece_load(i * 64 + lane);
        __builtin_amdgcn_sched_barrier(0);   // the X loads, then the early body loads
#pragma unroll
        for (int i = 0; i < EARLY; ++i) issue(ring[i]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NP; ++i) piece_store(i * 64 + lane, xv[i]);
        __builtin_amdgcn_sched_barrier(0);
        for (int v0 = NP * 64; v0 < npc; v0 += 16 * 64) {
            u32x4 xr[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) xr[i] = piece_load(v0 + i * 64 + lane);
#pragma unroll
            for (int i = 0; i < 16; ++i) piece_store(v0 + i * 64 + lane, xr[i]);
        }
        if constexpr (kDecodeRamp) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
#pragma unroll
        for (int i = EARLY; i < PB; ++i) issue(ring[i]);
    };
    // counters zeroed before any wave can reach an item end; no global load
    // has been issued yet, so this barrier costs only the waves' start skew
    if (tid < 4 + DW) cnt[tid] = 0u;
    if (tid < kDecodeZeroBytes / 16) zstrip[tid] = u32x4{};
    __syncthreads();
    if (nbw == 0) return;                          // fewer bodies than waves: no work
    const int npl = (npc + 63) / 64;               // pieces per lane
    if (npl <= 1)
        stage(std::integral_constant<int, 1>{});
    else if (npl <= 2)
        stage(std::integral_constant<int, 2>{});
    else if (npl <= 4)
        stage(std::integral_constant<int, 4>{});
    else if (npl <= 8)
        stage(std::integral_constant<int, 8>{});
    else
        stage(std::integral_constant<int, 16>{});

    // NACC accumulators per tile (k-steps alternate between them), so that
    // consecutive MFMAs do not wait for each other's result: two for a single
    // tile, one each when several tiles interleave
    constexpr int NACC = TPI == 1 ? 2 : 1;
    f32x4 acc[TPI][NACC];
#pragma unroll
    for (int tt = 0; tt < TPI; ++tt)
#pragma unroll
        for (int h = 0; h < NACC; ++h) acc[tt][h] = f32x4{};
    f32x4 acc_sa = f32x4{};                      // scale-after: the tile
    f32x4 t_sa = f32x4{};                        // scale-after: one group's product

    const Magic mg = make_magic();
    const uint32_t zsh = zent_shift<G>(c32);   // this lane's zero entry in its dword
    // A operand of this lane (row i = l % 16, slot o = l / 16): X row x(i) at
    // halves 8 * (o / 2) of each k-step if row i's half is the slot's and
    // x(i) < M, else the zero strip
    const int ai = lane & 15;
    const int axr = (ai & 3) + 4 * (ai >> 3);
    const bool alive = ((ai >> 2) & 1) == ((lane >> 4) & 1) && axr < M;
    const uint32_t arow = (uint32_t)axr * RS + 16 * (lane >> 5);
    const uint32_t azero = (uint32_t)((const uint8_t*)zstrip - lds);

    // One body: the 16 A operands are read from LDS first (all in flight
    // together), then each k-step's words are dequantized and fed to the MFMAs.
    auto compute = [&](const Bundle& B, int b, auto ex) {
        const uint8_t* abase = lds + (alive ? arow + (uint32_t)b * (kBodyK * 2) : azero);
        u32x4 a[16];
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) a[kk] = *(const u32x4*)(abase + kk * (kKStep * 2));
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the body's work
        if constexpr (SA) {
            uint32_t bA = 0, bB = 0;
            float sc = 0.f;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int kk = 4 * cc + u;        // k-step inside the body
                    if (kk % GS == 0) {
                        const int e = kk / GS;
                        const uint32_t sword = B.s[0].word(e >> 1);
                        const uint32_t sbits = (e & 1) ? (sword >> 16) : (sword & 0xFFFFu);
                        const uint32_t z = SYM ? 8u : (((B.z[0] >> zsh) >> (4 * e)) & 0xFu);
                        bA = (0x6400u | z) * 0x00010001u;            // fp16 1024 + z
                        bB = (0x5400u | (z << 4)) * 0x00010001u;     // fp16 64 + z
                        sc = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
                    }
                    const u32x4 bop = unpack_qz(B.w[0][cc][u], bA, bB, mg);
                    if (kk % GS == 0) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) t_sa[r] = opaque_f(0.f);
                    }
                    t_sa = mfma16x16x32<DT>(a[kk], bop, t_sa);
                    if (kk % GS == GS - 1) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc_sa[r] = __builtin_fmaf(sc, t_sa[r], acc_sa[r]);
                    }
                }
            }
            return;
        }
        ColParams<DT> prm[TPI];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int kk = 4 * cc + u;        // k-step inside the body
                if (kk % GS == 0) {
                    const int e = kk / GS;
#pragma unroll
                    for (int tt = 0; tt < TPI; ++tt)
                        prm[tt] = entry_params<DT, SYM>(B.s[tt].word(e >> 1), B.z[tt] >> zsh, e);
                }
#pragma unroll
                for (int tt = 0; tt < TPI; ++tt) {
                    const u32x4 bop = dequant_sel<decltype(ex)::value>(B.w[tt][cc][u], prm[tt], mg);
                    acc[tt][kk % NACC] = mfma16x16x32<DT>(a[kk], bop, acc[tt][kk % NACC]);
                }
            }
        }
    };

    // Part tp of a split item, summed over this workgroup's waves (v), meets
    // the other S - 1 parts, each from another workgroup.  Every part is
    // stored to its slot in the workspace with device-scope stores (sc1: they
    // write through the per-XCD L2, which is not coherent between XCDs); the
    // wave waits until its stores have completed (vmcnt(0)) and only then
    // bumps the item's counter with a device-scope atomic.  The workgroup
    // whose atomic returns S - 1 is the last: every other part's stores
    // completed before that part's atomic, which came before this one, so its
    // device-scope loads (which bypass the L2 as well) read them.  It adds
    // the S parts in part order 0..S-1 (its own from registers, the same
    // values it stored: bitwise reproducible), resets the counter for the
    // next call and stores Y.  Nobody waits for anybody.  The tail part is
    // the first item of the workgroup, so these round trips overlap the full
    // items that follow.  Returns true in the last workgroup.
    const uint32_t part_bytes = (uint32_t)(TPI * QMAX * 64 * 16);
    auto tail_exchange = [&](f32x4 (&v)[TPI][QMAX]) -> bool {
        uint32_t* wcnt = (uint32_t*)ws + tail_idx;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            ws + kCounterBytes + (size_t)tail_idx * S * part_bytes, (short)0, (int)(S * part_bytes),
            kBufferRsrcWord3);
        const uint32_t lane_off = (uint32_t)lane * 16;
        auto off = [&](int part, int tt, int q) {
            return (int)(part * part_bytes + (tt * QMAX + q) * 1024 + lane_off);
        };
#pragma unroll
        for (int tt = 0; tt < TPI; ++tt)
#pragma unroll
            for (int q = 0; q < QMAX; ++q)
                if (q < QM)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[tt][q]), rs,
                                                           off(tp, tt, q), 0, kDeviceScope);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        uint32_t old = 0;
        if (lane == 0)
            old = __hip_atomic_fetch_add(wcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __builtin_amdgcn_readfirstlane(old);
        asm volatile("" ::: "memory");
        if ((int)old != S - 1) return false;
#pragma unroll
        for (int tt = 0; tt < TPI; ++tt)
#pragma unroll
            for (int q = 0; q < QMAX; ++q) {
                if (q >= QM) continue;
                f32x4 sum = tp == 0 ? v[tt][q]
                                    : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                    rs, off(0, tt, q), 0, kDeviceScope));
                for (int sp = 1; sp < S; ++sp)
                    sum += sp == tp ? v[tt][q]
                                    : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                    rs, off(sp, tt, q), 0, kDeviceScope));
                v[tt][q] = sum;
            }
        if (lane == 0) __hip_atomic_store(wcnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    };

    // End of item j (the j-th of this workgroup), without a barrier: each wave
    // writes its partial tiles to the slots of parity j % 2 and bumps that
    // parity's arrival counter; the wave that arrives last adds the slots in
    // wave order (bitwise reproducible), runs the epilogue, stores Y, resets
    // the arrival counter and then bumps that parity's count of reduced items.
    // LDS operations of one wave complete in order, so a wave's slot writes
    // precede its arrival and the reducer's slot reads precede its reset.
    // Before writing the slots of parity j % 2 a wave waits until j / 2 items
    // of that parity have been reduced, i.e. item j - 2 (whose slots and
    // counter it reuses); that reducer is a running wave of this workgroup
    // that waits on nothing, so the wait always ends (and is bounded besides).
    const int nact = min(DW, KB);                 // waves that own bodies
    auto item_end = [&](int j) {
        const int par = j & 1;
        if (j >= 2) {
            for (int spin = 0; spin < (1 << 22); ++spin) {
                const uint32_t d = __builtin_amdgcn_readfirstlane(
                    __hip_atomic_load(&cnt[2 + par], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
                if (d >= (uint32_t)(j >> 1)) break;
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if constexpr (SA) {
            slot(par, wave, 0, 0) = acc_sa;
            acc_sa = f32x4{};
        } else {
#pragma unroll
            for (int tt = 0; tt < TPI; ++tt)
#pragma unroll
                for (int q = 0; q < QMAX; ++q)
                    if (q < QM) {
                        f32x4 v = acc[tt][0];
#pragma unroll
                        for (int h = 1; h < NACC; ++h) v += acc[tt][h];
                        slot(par, wave, tt, q) = v;
                    }
#pragma unroll
            for (int tt = 0; tt < TPI; ++tt)
#pragma unroll
                for (int h = 0; h < NACC; ++h) acc[tt][h] = f32x4{};
        }
        // the slot writes are complete (LDS only: loads in flight stay in flight)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        uint32_t old = 0;
        if (lane == 0)
            old = __hip_atomic_fetch_add(&cnt[par], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        old = __builtin_amdgcn_readfirstlane(old);
        asm volatile("" ::: "memory");
        if ((int)old != nact - 1) return;
        f32x4 v[TPI][QMAX];
#pragma unroll
        for (int tt = 0; tt < TPI; ++tt)
#pragma unroll
            for (int q = 0; q < QMAX; ++q) {
                if (q >= QM) continue;
                v[tt][q] = slot(par, 0, tt, q);
                for (int w = 1; w < nact; ++w) v[tt][q] += slot(par, w, tt, q);
            }
        // the slots are free again once their reads are done
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (lane == 0) {
            __hip_atomic_store(&cnt[par], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_add(&cnt[2 + par], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (is_tail(j) && !tail_exchange(v)) return;
        const int item = item_of(j);
#pragma unroll
        for (int tt = 0; tt < TPI; ++tt)
#pragma unroll
            for (int q = 0; q < QMAX; ++q) {
                if (q >= QM) continue;
                const int64_t col = (int64_t)(item * TPI + tt) * kTileCols + c32;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 8 * q + 4 * (lane >> 5) + i;
                    if (row < M)
                        Y[(int64_t)row * N + col] = out_value<DT, EP>(v[tt][q][i], row, col, N, ep);
                }
            }
    };

    // Waves w and w + 4 share a SIMD, whose issue arbiter favours the older
    // wave when both are ready; left alone the older one runs ahead and
    // finishes first, and the other then runs without a partner to overlap
    // with.  So each wave publishes how many bodies it has computed and takes
    // the lower priority while it is ahead of its partner (a finished wave
    // reports "infinitely far", never holding its partner back).
    auto balance = [&](int done) {
        if constexpr (kDecodeBalance) {
            if (lane == 0)
                __hip_atomic_store(&prog[wave], (uint32_t)done, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            const uint32_t partner = __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                &prog[wave ^ (DW / 2)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
            if ((uint32_t)done > partner)
                __builtin_amdgcn_s_setprio(0);
            else
                __builtin_amdgcn_s_setprio(1);
        }
    };

    auto mainloop = [&](auto ex) {
        int j = 0, bb = 0;                        // item and body of step st
        for (int st = 0; st < nsteps; st += R) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                issue(ring[(r + PB) % R]);
                if (st + r < nsteps) {
                    compute(ring[r], body_of(j, bb), ex);
                    balance(st + r + 1);
                    if (++bb == len_of(j)) {
                        item_end(j);
                        bb = 0;
                        ++j;
                    }
                }
            }
        }
        if constexpr (kDecodeBalance) {
            if (lane == 0)
                __hip_atomic_store(&prog[wave], 0xFFFFFFFFu, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            __builtin_amdgcn_s_setprio(0);
        }
    };
    if (exact)
        mainloop(std::true_type{});
    else
        mainloop(std::false_type{});
}

template <int DT, bool SYM, int G, int MB, int TPI, int PB>
hipError_t launch_decode_t(const void* X, const void* packed, void* Y, int64_t M,
                           const Layout& L, const Plan& p, void* workspace, const Epilogue& ep,
                           hipStream_t stream) {
    constexpr bool EPF = W4A16_TU_EP != 0;
    const size_t lds = decode_lds_bytes(M, L.K, TPI, MB);
    auto kern = decode_kernel<DT, SYM, G, MB, TPI, PB, EPF>;
    hipLaunchKernelGGL(kern, dim3(p.grid_x), dim3(DW * 64), lds, stream, (const uint16_t*)X,
                       (const uint8_t*)packed, (uint16_t*)Y, (int)M, (int)L.N, (int)L.K,
                       p.items, p.tiles, p.splits, (uint8_t*)workspace, L.s_off, L.z_off, L.t_off,
                       ep);
    return hipGetLastError();
}

template <int DT, bool SYM, int G>
hipError_t launch_decode_g(const void* X, const void* packed, void* Y, int64_t M,
                           const Layout& L, const Plan& p, void* workspace, const Epilogue& ep,
                           hipStream_t stream) {
    constexpr int PB = kDecodePrefetch;
    if (M > kDecodeMaxRows) return hipErrorInvalidValue;   // the plan never asks for it
    return launch_decode_t<DT, SYM, G, kDecodeMaxRows, 1, PB>(X, packed, Y, M, L, p, workspace, ep,
                                                              stream);
}

template <int DT, bool SYM>
hipError_t launch_decode_s(const void* X, const void* packed, void* Y, int64_t M,
                           const Layout& L, const Plan& p, void* workspace, const Epilogue& ep,
                           hipStream_t stream) {
    if (L.G == 128) return launch_decode_g<DT, SYM, 128>(X, packed, Y, M, L, p, workspace, ep, stream);
    if (L.G == 64) return launch_decode_g<DT, SYM, 64>(X, packed, Y, M, L, p, workspace, ep, stream);
    return launch_decode_g<DT, SYM, 32>(X, packed, Y, M, L, p, workspace, ep, stream);
}

}  // namespace

#if W4A16_TU_BF16
#if W4A16_TU_EP
#define W4A16_DECODE_ENTRY launch_decode_bf16_ep
#else
#define W4A16_DECODE_ENTRY launch_decode_bf16
#endif
#else
#if W4A16_TU_EP
#define W4A16_DECODE_ENTRY launch_decode_f16_ep
#else
#define W4A16_DECODE_ENTRY launch_decode_f16
#endif
#endif

hipError_t W4A16_DECODE_ENTRY(const void* X, const void* packed, void* Y, int64_t M,
                              const Layout& L, const Plan& p, void* workspace, const Epilogue& ep,
                              hipStream_t stream) {
    constexpr int DT = W4A16_TU_BF16 ? DT_BF16 : DT_F16;
    if (L.sym) return launch_decode_s<DT, true>(X, packed, Y, M, L, p, workspace, ep, stream);
    return launch_decode_s<DT, false>(X, packed, Y, M, L, p, workspace, ep, stream);
}

}  // namespace w4a16
