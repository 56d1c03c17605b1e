// w4a16_wide.hip -- the fused W4A16 dequantize-GEMM for 32 < M <= 128 on
// gfx950 (the batched regime between decode and prefill).
//
// Page "W4A16 GEMM 算子浅析" (nxmr.cn), section "硬件性能拐点": past a batch
// of a few dozen rows the dequantization work starts to matter next to the
// weight stream; page "W4A8量化计算优化" (bjdmk.com.cn), section 3.1: loads
// of the next tile run while the current one is computed, with the
// activations shared through on-chip memory.  Page "量化开销对比", section
// 6.5: each weight is read from HBM once, reuse is along M.
//
// Work decomposition.  An item is one 128-column block (four 32-column
// tiles) over all of K.  The 8 waves of a workgroup are 4 tiles x 2 halves
// of K: wave w computes tile w % 4 on half w / 4 of the item's k range, so
// the workgroup reads every weight byte of the block once and no partial sum
// leaves it (the two halves are added in LDS at the end of the item).  When
// there are fewer blocks than CUs, K is also split across S workgroups per
// block (parts), whose partial tiles meet in the workspace.
//
// Activations.  The k range is walked in steps of SK (256 or 128) per half;
// the X rows of a step, for both halves, are staged into one of two LDS
// slots by all threads while the previous step is computed, and one
// workgroup barrier per step separates the writes of a slot from its reads.
// Rows are padded by 16 bytes so the rows a quarter-wave reads at one k sit
// in different banks.  Weights: one step of a tile (SK/64 chunks plus the
// body's scale and zero entries) in flight per wave while it computes the
// previous one; all loads are unconditional at clamped addresses, so the
// compiler counts exactly what is outstanding.
//
// MFMA: v_mfma_f32_32x32x16_{f16,bf16}; each dequantized word feeds the MR
// row tiles of the block's 32*MR rows (rows >= M read row M-1 and are never
// stored).
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

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

constexpr int WW = kWideWaves;   // waves per workgroup
constexpr int WT = 4;            // tiles per item

// A value the compiler must re-read where it is used (volatile asm): the
// item-end code derives dozens of addresses from M, N and the lane; without
// this they are hoisted out of the step loop and held in registers across it.
__device__ __forceinline__ int at_use(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// f(integral_constant<int, I>) for I = 0..n-1 in order: an unrolled loop whose
// index is a compile-time constant in every copy (arrays of registers indexed
// by it stay in registers, however large the body).
template <class F, int... I>
__device__ __forceinline__ void for_each_index(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}

// The LDS writes of this wave are complete, then the workgroup barrier.
// Global loads in flight stay in flight.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int DT, bool SYM, int G, int MR, int SK, bool EP>
__global__ __launch_bounds__(WW * 64) void wide_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed, uint16_t* __restrict__ Y,
    int M, int N, int K, int n_items, int parts, uint8_t* __restrict__ ws, size_t s_off,
    size_t z_off, size_t t_off, Epilogue ep) {
    constexpr int EPB = kBodyK / G;             // groups per body
    constexpr int GS = G / kKStep;              // k-steps per group
    constexpr int SE = 2 * EPB;                 // scale entry bytes
    constexpr int ZE = EPB / 2;                 // zero entry bytes
    constexpr int KSS = SK / kKStep;            // k-steps per step
    constexpr int CPS = SK / kChunkK;           // chunks per step
    constexpr int RSB = 2 * SK + 16;            // LDS bytes per staged X row
    constexpr int PPR = SK / 8;                 // 16-byte pieces per staged row
    constexpr int NPX = (2 * 32 * MR * PPR + WW * 64 - 1) / (WW * 64);   // pieces per thread
    static_assert(SK == 128 || SK == 256, "steps of half a body or a body");
    extern __shared__ __align__(16) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = wave & (WT - 1);              // tile of the item
    const int h = wave / WT;                    // half of the k range
    const int c32 = lane & 31;
    const int KC = K / kChunkK;
    const int KB = K / kBodyK;
    const int T = K / SK;                       // steps over all of K
    const int W = (int)gridDim.x, g = (int)blockIdx.x;

    // This workgroup's work.  S = 1: items g, g + W, ...  S > 1: part g % S of
    // item g / S.  A part is the steps [P0, P1) of K; its first n0 steps are
    // half 0 and the next n1 half 1.
    const int S = parts;
    const int n_units = S > 1 ? 1 : (n_items - g + W - 1) / W;
    const int p = S > 1 ? g % S : 0;
    const int P0 = p * T / S, P1 = (p + 1) * T / S;
    const int n0 = (P1 - P0 + 1) / 2, n1 = (P1 - P0) / 2;
    const int nh = h == 0 ? n0 : n1;            // steps this wave computes per item
    const int hs = h == 0 ? P0 : P0 + n0;       // its first step
    const int nsteps = n_units * n0;
    auto item_of = [&](int j) __attribute__((always_inline)) { return S > 1 ? g / S : g + j * W; };
    const int slot_bytes = 2 * M * RSB;         // both halves' rows of one step

    const bool exact = [&] {
        if constexpr (DT == DT_F16) {
            return false;
        } else {
            return (*(const uint32_t*)(packed + t_off + 8) & kFlagExactBf16) != 0;
        }
    }();

    // ---- weights of one step of this wave's tile, and the body's entries
    struct Bundle {
        u32x4 w[CPS];
        SEnt<G> s;
        uint32_t z;
    };
    const uint32_t lane16 = (uint32_t)lane * 16;
    auto step_block = [&](int ls) __attribute__((always_inline)) {   // step of K this wave reads at local step ls (clamped)
        return nh > 0 ? hs + min(ls, nh - 1) : P0;
    };
    auto issue = [&](Bundle& B, int j, int ls) __attribute__((always_inline)) {
        const int jj = min(j, n_units - 1);
        const int tile = item_of(jj) * WT + t;
        const int kb = step_block(ls);
        const uint8_t* wb = packed + ((size_t)tile * KC + (size_t)kb * CPS) * kChunkBytes + lane16;
#pragma unroll
        for (int cc = 0; cc < CPS; ++cc)
            B.w[cc] = __builtin_nontemporal_load((const u32x4*)(wb + cc * kChunkBytes));
        const size_t ent = ((size_t)tile * KB + (size_t)kb * SK / kBodyK) * 32 + c32;
        B.s = load_sent<G>(packed + s_off + ent * SE);
        B.z = SYM ? 0u : load_zent<G>(packed + z_off + ent * ZE);
    };

    // ---- X pieces of one step (both halves): piece v = i*512 + tid, half
    // v / (M*PPR), row, 16-byte column; the global offset without the step's
    // k and the LDS offset inside a slot are fixed per thread and piece.
    const int npc = 2 * M * PPR;
    int xg[NPX];          // element offset of the piece in X, half in bit 30
    int xl[NPX];          // byte offset of the piece in a slot
#pragma unroll
    for (int i = 0; i < NPX; ++i) {
        const int v = min(i * WW * 64 + tid, npc - 1);
        const int hh = v / (M * PPR);
        const int rem = v - hh * M * PPR;
        const int row = rem / PPR;
        const int col = rem - row * PPR;
        xg[i] = (row * K + col * 8) | (hh << 30);
        xl[i] = hh * M * RSB + row * RSB + col * 16;
    }
    auto x_load = [&](u32x4 (&xv)[NPX], int ls) {
        const int k0 = min(P0 + ls, T - 1) * SK;                // half 0's k at step ls
        const int k1 = min(P0 + n0 + min(ls, max(n1 - 1, 0)), T - 1) * SK;
#pragma unroll
        for (int i = 0; i < NPX; ++i) {
            const int off = (xg[i] & ~(1 << 30)) + ((xg[i] >> 30) ? k1 : k0);
            xv[i] = *(const u32x4*)(X + off);
        }
    };
    auto x_store = [&](const u32x4 (&xv)[NPX], int slot) {
        uint8_t* base = lds + slot * slot_bytes;
#pragma unroll
        for (int i = 0; i < NPX; ++i) *(u32x4*)(base + xl[i]) = xv[i];
    };

    f32x16 acc[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = f32x16{};
    const Magic mg = make_magic();
    const uint32_t zsh = zent_shift<G>(c32);
    int arow[MR];         // this lane's A row offset (bytes) per row tile: row min(32r + l%32, M-1)
#pragma unroll
    for (int r = 0; r < MR; ++r) arow[r] = min(32 * r + c32, M - 1) * RSB + 16 * (lane >> 5);

    // One step of this wave: KSS k-steps, each one word dequantized and fed
    // to the MR row tiles.  kb: the step of K (for the group entries).
    auto compute = [&](const Bundle& B, int slot, int kb, auto ex) __attribute__((always_inline)) {
        const uint8_t* abase = lds + slot * slot_bytes + h * M * RSB;
        const int kbody = SK == kBodyK ? 0 : (kb & 1) * KSS;   // first k-step of the step in its body
        ColParams<DT> prm;
        // A operands one k-step ahead; the scheduling barrier at the end of a
        // k-step keeps the compiler from hoisting every LDS read of the step
        // (which would hold 4*MR*KSS registers at once)
        u32x4 a_cur[MR], a_nxt[MR];
#pragma unroll
        for (int r = 0; r < MR; ++r) a_cur[r] = *(const u32x4*)(abase + arow[r]);
#pragma unroll
        for (int kk = 0; kk < KSS; ++kk) {
            const int ks = kbody + kk;                           // k-step inside the body
            if (kk + 1 < KSS) {
#pragma unroll
                for (int r = 0; r < MR; ++r)
                    a_nxt[r] = *(const u32x4*)(abase + arow[r] + (kk + 1) * (kKStep * 2));
            }
            if (SK == kBodyK ? (kk % GS == 0) : (kk == 0 || ((kbody + kk) % GS == 0))) {
                const int e = ks / GS;
                prm = entry_params<DT, SYM>(B.s.word(e >> 1), B.z >> zsh, e);
            }
            const u32x4 bop = dequant_sel<decltype(ex)::value>(B.w[kk / 4][kk % 4], prm, mg);
#pragma unroll
            for (int r = 0; r < MR; ++r) acc[r] = mfma32x32x16<DT>(a_cur[r], bop, acc[r]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < MR; ++r) a_cur[r] = a_nxt[r];
        }
    };

    // Parts of an item meet in the workspace (S > 1): every part stores its
    // tiles (half 0's waves, after the halves were added) with device-scope
    // stores, waits for them, and one thread bumps the item's counter with a
    // device-scope atomic after a workgroup barrier.  The workgroup whose
    // atomic returns S - 1 is the last: every other part's stores completed
    // before that part's atomic, so its device-scope loads read them; it adds
    // the S parts in part order (its own from registers) and stores Y.
    // Returns true (in every wave) in the last workgroup.
    constexpr uint32_t wave_part_bytes = (uint32_t)MR * 16 * 64 * 4;   // one tile of one part
    uint32_t* flag = (uint32_t*)(lds + 2 * slot_bytes);
    auto parts_meet = [&](int item) __attribute__((always_inline)) -> bool {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            ws + kCounterBytes + (size_t)item * S * WT * wave_part_bytes, (short)0,
            (int)(S * WT * wave_part_bytes), kBufferRsrcWord3);
        auto off = [&](int part, int r, int q) __attribute__((always_inline)) {
            return (int)(((uint32_t)part * WT + t) * wave_part_bytes + (uint32_t)(r * 4 + q) * 1024 +
                         lane16);
        };
        if (h == 0) {
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4, f32x4{acc[r][4 * q], acc[r][4 * q + 1],
                                                        acc[r][4 * q + 2], acc[r][4 * q + 3]}),
                        rs, off(p, r, q), 0, kDeviceScope);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        barrier_lds();
        if (tid == 0)
            *flag = __hip_atomic_fetch_add((uint32_t*)ws + item, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(S - 1);
        barrier_lds();
        const bool last = __builtin_amdgcn_readfirstlane(*flag) != 0;
        if (!last) return false;
        if (h == 0) {
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 mine = f32x4{acc[r][4 * q], acc[r][4 * q + 1], acc[r][4 * q + 2],
                                             acc[r][4 * q + 3]};
                    f32x4 sum = p == 0 ? mine
                                       : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                       rs, off(0, r, q), 0, kDeviceScope));
                    for (int sp = 1; sp < S; ++sp)
                        sum += sp == p ? mine
                                       : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                       rs, off(sp, r, q), 0, kDeviceScope));
                    acc[r][4 * q] = sum[0];
                    acc[r][4 * q + 1] = sum[1];
                    acc[r][4 * q + 2] = sum[2];
                    acc[r][4 * q + 3] = sum[3];
                }
        }
        if (tid == 0)
            __hip_atomic_store((uint32_t*)ws + item, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    };

    // End of item j, after the barrier of its last step: slot fs is free
    // until the next step's staging writes it.  Half 1's waves write their
    // rows < M to it, half 0's waves add them to their own (h0 + h1, a fixed
    // order), a barrier frees the slot again, and half 0's waves store Y
    // (after the parts meet when K is split across workgroups).
    auto item_end = [&](int j, int fs) __attribute__((always_inline)) {
        const int Mu = at_use(M);                      // computed here, not before the loop
        const int lu = at_use(lane);
        float* red = (float*)(lds + fs * 2 * Mu * RSB);   // [WT][M][32]
        if (h == 1) {
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = 32 * r + acc_row(i, lu);
                    if (row < Mu) red[(t * Mu + row) * 32 + (lu & 31)] = acc[r][i];
                }
        }
        barrier_lds();
        if (h == 0) {
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = 32 * r + acc_row(i, lu);
                    if (row < Mu) acc[r][i] += red[(t * Mu + row) * 32 + (lu & 31)];
                }
        }
        barrier_lds();
        const int item = item_of(j);
        const bool store = S > 1 ? parts_meet(item) : true;
        if (h == 0 && store) {
            const int Nu = at_use(N);
            const int64_t col = (int64_t)item * (WT * kTileCols) + t * kTileCols + (lu & 31);
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = 32 * r + acc_row(i, lu);
                    if (row < Mu)
                        Y[(int64_t)row * Nu + col] = out_value<DT, EP>(acc[r][i], row, col, Nu, ep);
                }
        }
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[r] = f32x16{};
    };

    // ---- the steps.  Step js = local step ls of unit j reads X slot js % 2
    // and ring[js % R]; while it computes, the next step's X and the weights
    // of step js + WPB are in flight (X first, so that staging it waits for
    // the X loads only).
    constexpr int WPB = kWidePrefetch;          // weight steps in flight
    constexpr int R = WPB + 1;
    Bundle ring[R];
    int ij = 0, ils = 0;                        // issue cursor: unit, local step
    auto advance = [&](int& jj, int& ll) __attribute__((always_inline)) {
        if (++ll == n0) {
            ll = 0;
            ++jj;
        }
    };
    {
        u32x4 xv[NPX];
        x_load(xv, 0);
#pragma unroll
        for (int i = 0; i < WPB; ++i) {
            issue(ring[i], ij, ils);
            advance(ij, ils);
        }
        x_store(xv, 0);
        barrier_lds();
    }
    auto mainloop = [&](auto ex) __attribute__((always_inline)) {
        int j = 0, ls = 0;
        for (int js0 = 0; js0 < nsteps; js0 += R) {
            for_each_index([&](auto r_) __attribute__((always_inline)) {
                constexpr int r = decltype(r_)::value;
                const int js = js0 + r;
                if (js < nsteps) {
                    const int lsn = ls + 1 == n0 ? 0 : ls + 1;      // the next step's local step
                    u32x4 xv[NPX];
                    x_load(xv, lsn);
                    issue(ring[(r + WPB) % R], ij, ils);
                    advance(ij, ils);
                    if (ls < nh) compute(ring[r], js & 1, step_block(ls), ex);
                    x_store(xv, (js + 1) & 1);
                    barrier_lds();
                    if (ls + 1 == n0) item_end(j, js & 1);
                    advance(j, ls);
                }
            }, std::make_integer_sequence<int, R>{});
        }
    };
    if (exact)
        mainloop(std::true_type{});
    else
        mainloop(std::false_type{});
}

template <int DT, bool SYM, int G, int MR, int SK>
hipError_t launch_wide_t(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                         const Plan& p, void* workspace, const Epilogue& ep, hipStream_t stream) {
    constexpr bool EPF = W4A16_TU_EP != 0;
    const size_t lds = wide_lds_bytes(M, SK);
    auto kern = wide_kernel<DT, SYM, G, MR, SK, EPF>;
    hipLaunchKernelGGL(kern, dim3(p.grid_x), dim3(WW * 64), lds, stream, (const uint16_t*)X,
                       (const uint8_t*)packed, (uint16_t*)Y, (int)M, (int)L.N, (int)L.K, p.items,
                       p.splits, (uint8_t*)workspace, L.s_off, L.z_off, L.t_off, ep);
    return hipGetLastError();
}

template <int DT, bool SYM, int G>
hipError_t launch_wide_g(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                         const Plan& p, void* workspace, const Epilogue& ep, hipStream_t stream) {
    if (M <= 64) return launch_wide_t<DT, SYM, G, 2, 256>(X, packed, Y, M, L, p, workspace, ep, stream);
    if (M <= 96) return launch_wide_t<DT, SYM, G, 3, 128>(X, packed, Y, M, L, p, workspace, ep, stream);
    if (M <= 128) return launch_wide_t<DT, SYM, G, 4, 128>(X, packed, Y, M, L, p, workspace, ep, stream);
    return hipErrorInvalidValue;   // the plan never asks for it
}

template <int DT, bool SYM>
hipError_t launch_wide_s(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                         const Plan& p, void* workspace, const Epilogue& ep, hipStream_t stream) {
    if (L.G == 128) return launch_wide_g<DT, SYM, 128>(X, packed, Y, M, L, p, workspace, ep, stream);
    if (L.G == 64) return launch_wide_g<DT, SYM, 64>(X, packed, Y, M, L, p, workspace, ep, stream);
    return launch_wide_g<DT, SYM, 32>(X, packed, Y, M, L, p, workspace, ep, stream);
}

}  // namespace

#if W4A16_TU_BF16
#if W4A16_TU_EP
#define W4A16_WIDE_ENTRY launch_wide_bf16_ep
#else
#define W4A16_WIDE_ENTRY launch_wide_bf16
#endif
#else
#if W4A16_TU_EP
#define W4A16_WIDE_ENTRY launch_wide_f16_ep
#else
#define W4A16_WIDE_ENTRY launch_wide_f16
#endif
#endif

hipError_t W4A16_WIDE_ENTRY(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                            const Plan& p, void* workspace, const Epilogue& ep, hipStream_t stream) {
    constexpr int DT = W4A16_TU_BF16 ? DT_BF16 : DT_F16;
    if (L.sym) return launch_wide_s<DT, true>(X, packed, Y, M, L, p, workspace, ep, stream);
    return launch_wide_s<DT, false>(X, packed, Y, M, L, p, workspace, ep, stream);
}

}  // namespace w4a16
