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

constexpr int SK_WAVES = 8;   // waves per split-K workgroup
constexpr int SK_U = 8;       // k-steps per load batch
constexpr int MAX_SPLITS = 16;

__device__ __forceinline__ u32x4 load_weights(const u32x4* p) {
    return __builtin_nontemporal_load(p);   // streamed once: do not keep in cache
}

// ---------------------------------------------------------------------------
// Split-K streaming kernel, M <= 32.
// ---------------------------------------------------------------------------
template <int DT, bool SYM, int GS>
__global__ __launch_bounds__(SK_WAVES * 64) void splitk_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed, uint16_t* __restrict__ Y,
    float* __restrict__ part, uint32_t* __restrict__ cnt, int M, int N, int K,
    int steps_per_wave, int S, size_t s_off, size_t z_off) {
    constexpr int NGB = SK_U / GS;   // whole groups per batch (GS divides SK_U)
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nb = blockIdx.x;
    const int split = blockIdx.y;
    const int KS = K / kKStep;
    const int NG = K / (kKStep * GS);
    const int s_beg = (split * SK_WAVES + wave) * steps_per_wave;
    const int s_end = min(s_beg + steps_per_wave, KS);

    const u32x4* wchunk = (const u32x4*)packed + (size_t)nb * KS * 64 + lane;
    const uint8_t* srec = packed + s_off + (size_t)nb * NG * kScaleRecBytes + (lane & 31) * 8;
    const uint8_t* zrec = packed + z_off + (size_t)nb * NG * kZeroRecBytes + (lane & 31) * 2;
    const int row = lane & 31;
    const bool row_ok = row < M;
    const uint16_t* xrow = X + (size_t)(row_ok ? row : 0) * K + 8 * (lane >> 5);

    f32x16 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x16{};

    struct Batch {
        u32x4 w[SK_U];
        u32x4 x[SK_U];
        u32x2 sc[NGB];
        uint32_t zw[NGB];
    };

    auto load = [&](Batch& b, int sb) {
#pragma unroll
        for (int u = 0; u < SK_U; ++u) {
            const int s = sb + u;
            if (s < s_end) {
                b.w[u] = load_weights(wchunk + (size_t)s * 64);
                b.x[u] = row_ok ? *(const u32x4*)(xrow + kKStep * s) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int j = 0; j < NGB; ++j) {
            const int g = sb / GS + j;
            if (g * GS < s_end) {
                b.sc[j] = *(const u32x2*)(srec + (size_t)g * kScaleRecBytes);
                b.zw[j] = SYM ? 0u : (uint32_t)*(const uint16_t*)(zrec + (size_t)g * kZeroRecBytes);
            }
        }
    };

    auto compute = [&](const Batch& b, int sb) {
#pragma unroll
        for (int j = 0; j < NGB; ++j) {
            if (sb + j * GS >= s_end) break;
            ColParams<DT> prm[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) prm[t] = tile_params<DT, SYM>(b.sc[j], b.zw[j], t);
            auto steps = [&](auto exact) {
#pragma unroll
                for (int uu = 0; uu < GS; ++uu) {
                    const int u = j * GS + uu;
                    if (sb + u >= s_end) break;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const u32x4 bop = dequant_sel<decltype(exact)::value>(b.w[u][t], prm[t]);
                        acc[t] = mfma32x32x16<DT>(b.x[u], bop, acc[t]);
                    }
                }
            };
            if (wave_needs_exact<DT>(prm))
                steps(std::true_type{});
            else
                steps(std::false_type{});
        }
    };

    if (s_beg < s_end) {
        Batch b0, b1;
        load(b0, s_beg);
        for (int sb = s_beg; sb < s_end; sb += 2 * SK_U) {
            if (sb + SK_U < s_end) load(b1, sb + SK_U);
            compute(b0, sb);
            if (sb + SK_U >= s_end) break;
            if (sb + 2 * SK_U < s_end) load(b0, sb + 2 * SK_U);
            compute(b1, sb + SK_U);
        }
    }

    // Reduce the 8 waves' partial tiles through LDS: halve the active waves
    // each round, always adding slot w into wave w (a fixed order).
    __shared__ f32x4 red[SK_WAVES / 2][4][4][64];
    __shared__ uint32_t s_last;
#pragma unroll
    for (int h = SK_WAVES / 2; h >= 1; h >>= 1) {
        if (wave >= h && wave < 2 * h) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    red[wave - h][t][q][lane] =
                        f32x4{acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]};
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

    const int64_t col0 = (int64_t)nb * kColBlock + (lane & 31);
    if (S == 1) {
        if (wave == 0) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = acc_row(r, lane);
                    if (rr < M) Y[(int64_t)rr * N + col0 + 32 * t] = round_out<DT>(acc[t][r]);
                }
        }
        return;
    }

    // Cross-workgroup reduction.  Only row quads that hold rows < M are kept:
    // quad q of lane l covers rows 8q + 4*(l/32) + 0..3.
    const int nq = (M + 7) / 8;
    f32x4* slot_base = (f32x4*)part + (size_t)nb * S * 4 * nq * 64;
    if (wave == 0) {
        f32x4* mine = slot_base + (size_t)split * 4 * nq * 64;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q < nq)
                    mine[(t * nq + q) * 64 + lane] =
                        f32x4{acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]};
    }
    __threadfence();   // release: partials visible device-wide before the count
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(&cnt[nb], 1u) == (uint32_t)(S - 1)) ? 1u : 0u;
    __syncthreads();
    if (!s_last) return;
    __threadfence();   // acquire: see every other workgroup's partials

    for (int f = threadIdx.x; f < 4 * nq * 64; f += SK_WAVES * 64) {
        const int t = f / (nq * 64);
        const int q = (f / 64) % nq;
        const int ln = f & 63;
        f32x4 v[MAX_SPLITS];
#pragma unroll
        for (int s = 0; s < MAX_SPLITS; ++s)
            if (s < S) v[s] = slot_base[(size_t)s * 4 * nq * 64 + f];
        f32x4 sum = v[0];
#pragma unroll
        for (int s = 1; s < MAX_SPLITS; ++s)
            if (s < S) sum += v[s];
        const int64_t col = (int64_t)nb * kColBlock + 32 * t + (ln & 31);
        const float sv[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = 8 * q + 4 * (ln >> 5) + i;
            if (rr < M) Y[(int64_t)rr * N + col] = round_out<DT>(sv[i]);
        }
    }
    if (threadIdx.x == 0) cnt[nb] = 0u;   // leave the counter zero for the next call
}

// ---------------------------------------------------------------------------
// LDS-tiled kernel, M > 32.
// ---------------------------------------------------------------------------
template <int DT, bool SYM, int GS, int MT>
__global__ __launch_bounds__(256) void tiled_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed, uint16_t* __restrict__ Y,
    float* __restrict__ part, uint32_t* __restrict__ cnt, int M, int N, int K,
    int steps_per_split, int S, size_t s_off, size_t z_off) {
    constexpr int KT = 8;                       // k-steps per stage (128 reduction indices)
    constexpr int ROWS = 32 * MT;
    constexpr int LDX = KT * kKStep + 8;        // LDS row pitch in halves (272 B)
    constexpr int SPG = GS < KT ? GS : KT;      // k-steps per group inside a stage
    constexpr int NGST = KT / SPG;              // groups per stage
    constexpr int XCH = ROWS * KT * kKStep / 8 / 256;   // 16-byte X chunks per thread per stage
    __shared__ __align__(16) uint16_t xs[2][ROWS * LDX];
    __shared__ uint32_t s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int NB = N / kColBlock;
    const int KS = K / kKStep;
    const int NG = K / (kKStep * GS);
    const int nb = blockIdx.x * 4 + wave;
    const bool nb_ok = nb < NB;
    const int nbc = nb_ok ? nb : NB - 1;
    const int m0 = blockIdx.y * ROWS;
    const int split = blockIdx.z;
    const int s_beg = split * steps_per_split;
    const int s_end = min(KS, s_beg + steps_per_split);

    const u32x4* wchunk = (const u32x4*)packed + (size_t)nbc * KS * 64 + lane;
    const uint8_t* srec = packed + s_off + (size_t)nbc * NG * kScaleRecBytes + (lane & 31) * 8;
    const uint8_t* zrec = packed + z_off + (size_t)nbc * NG * kZeroRecBytes + (lane & 31) * 2;

    struct Stage {
        u32x4 w[KT];
        u32x2 sc[NGST];
        uint32_t zw[NGST];
    };

    // X stage copy: chunk c = tid + 256*i covers row c / (KT*2), 8 halves at
    // column 8 * (c % (KT*2)).
    auto load_x = [&](u32x4 (&xr)[XCH], int st) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + 256 * i;
            const int r = c / (KT * 2);
            const int kk = kKStep * st + 8 * (c % (KT * 2));
            const int row = m0 + r;
            xr[i] = (row < M && kk < K) ? *(const u32x4*)(X + (size_t)row * K + kk)
                                        : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_x = [&](int buf, const u32x4 (&xr)[XCH]) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + 256 * i;
            const int r = c / (KT * 2);
            *(u32x4*)&xs[buf][r * LDX + 8 * (c % (KT * 2))] = xr[i];
        }
    };
    auto load_w = [&](Stage& b, int st) {
#pragma unroll
        for (int u = 0; u < KT; ++u) {
            const int s = st + u;
            if (s < s_end) b.w[u] = load_weights(wchunk + (size_t)s * 64);
        }
#pragma unroll
        for (int j = 0; j < NGST; ++j) {
            const int s = st + j * SPG;
            if (s < s_end) {
                const int g = s / GS;
                b.sc[j] = *(const u32x2*)(srec + (size_t)g * kScaleRecBytes);
                b.zw[j] = SYM ? 0u : (uint32_t)*(const uint16_t*)(zrec + (size_t)g * kZeroRecBytes);
            }
        }
    };

    f32x16 acc[MT][4];
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[r][t] = f32x16{};

    auto compute = [&](const Stage& b, int buf, int st) {
        const uint16_t* xb = &xs[buf][(lane & 31) * LDX + 8 * (lane >> 5)];
#pragma unroll
        for (int j = 0; j < NGST; ++j) {
            if (st + j * SPG >= s_end) break;
            ColParams<DT> prm[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) prm[t] = tile_params<DT, SYM>(b.sc[j], b.zw[j], t);
            auto steps = [&](auto exact) {
#pragma unroll
                for (int uu = 0; uu < SPG; ++uu) {
                    const int u = j * SPG + uu;
                    if (st + u >= s_end) break;
                    u32x4 a[MT];
#pragma unroll
                    for (int r = 0; r < MT; ++r)
                        a[r] = *(const u32x4*)(xb + 32 * r * LDX + kKStep * u);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const u32x4 bop = dequant_sel<decltype(exact)::value>(b.w[u][t], prm[t]);
#pragma unroll
                        for (int r = 0; r < MT; ++r)
                            acc[r][t] = mfma32x32x16<DT>(a[r], bop, acc[r][t]);
                    }
                }
            };
            if (wave_needs_exact<DT>(prm))
                steps(std::true_type{});
            else
                steps(std::false_type{});
        }
    };

    if (s_beg < s_end) {
        Stage A, B;
        u32x4 xr[XCH];
        load_x(xr, s_beg);
        load_w(A, s_beg);
        store_x(0, xr);
        __syncthreads();
        int buf = 0;
        for (int st = s_beg; st < s_end; st += 2 * KT) {
            const bool n1 = st + KT < s_end;
            if (n1) {
                load_x(xr, st + KT);
                load_w(B, st + KT);
            }
            compute(A, buf, st);
            if (n1) store_x(buf ^ 1, xr);
            __syncthreads();
            if (!n1) break;
            buf ^= 1;
            const bool n2 = st + 2 * KT < s_end;
            if (n2) {
                load_x(xr, st + 2 * KT);
                load_w(A, st + 2 * KT);
            }
            compute(B, buf, st + KT);
            if (n2) store_x(buf ^ 1, xr);
            __syncthreads();
            buf ^= 1;
        }
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

    // Cross-workgroup reduction in register order: per (tile, split) slot,
    // float4 index ((wave*MT + r)*4 + t)*4 + q, times 64 lanes.
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;
    constexpr int QPW = MT * 4 * 4;   // float4 quads per lane per wave
    const size_t slot_f4 = (size_t)4 * QPW * 64;
    f32x4* base = (f32x4*)part + (size_t)tile * S * slot_f4 + (size_t)wave * QPW * 64 + lane;
    {
        f32x4* mine = base + (size_t)split * slot_f4;
#pragma unroll
        for (int r = 0; r < MT; ++r)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    mine[((r * 4 + t) * 4 + q) * 64] = f32x4{acc[r][t][4 * q], acc[r][t][4 * q + 1],
                                                             acc[r][t][4 * q + 2], acc[r][t][4 * q + 3]};
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&cnt[tile], 1u) == (uint32_t)(S - 1)) ? 1u : 0u;
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // Sum the S slots in split order 0..S-1 (this workgroup's own slot is
    // taken from registers at its position in that order).
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 sum[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) sum[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < S; ++s) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = (s == split)
                                        ? f32x4{acc[r][t][4 * q], acc[r][t][4 * q + 1],
                                                acc[r][t][4 * q + 2], acc[r][t][4 * q + 3]}
                                        : base[(size_t)s * slot_f4 + ((r * 4 + t) * 4 + q) * 64];
                    sum[q] = (s == 0) ? v : sum[q] + v;
                }
            }
            if (nb_ok) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float sv[4] = {sum[q].x, sum[q].y, sum[q].z, sum[q].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = m0 + 32 * r + 8 * q + 4 * (lane >> 5) + i;
                        if (rr < M) Y[(int64_t)rr * N + colw + 32 * t] = round_out<DT>(sv[i]);
                    }
                }
            }
        }
    if (tid == 0) cnt[tile] = 0u;
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

template <int DT, bool SYM, int GS>
void launch_splitk(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                   const Plan& p, float* part, uint32_t* cnt, hipStream_t stream) {
    hipLaunchKernelGGL((splitk_kernel<DT, SYM, GS>), dim3(p.grid_x, p.grid_y, p.grid_z),
                       dim3(SK_WAVES * 64), 0, stream, (const uint16_t*)X, (const uint8_t*)packed,
                       (uint16_t*)Y, part, cnt, (int)M, (int)L.N, (int)L.K, p.steps_per_split,
                       p.splits, L.s_off, L.z_off);
}

template <int DT, bool SYM, int GS>
void launch_tiled(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                  const Plan& p, float* part, uint32_t* cnt, hipStream_t stream) {
    const dim3 grid(p.grid_x, p.grid_y, p.grid_z), block(256);
    if (p.mt == 2)
        hipLaunchKernelGGL((tiled_kernel<DT, SYM, GS, 2>), grid, block, 0, stream,
                           (const uint16_t*)X, (const uint8_t*)packed, (uint16_t*)Y, part, cnt,
                           (int)M, (int)L.N, (int)L.K, p.steps_per_split, p.splits, L.s_off,
                           L.z_off);
    else
        hipLaunchKernelGGL((tiled_kernel<DT, SYM, GS, 4>), grid, block, 0, stream,
                           (const uint16_t*)X, (const uint8_t*)packed, (uint16_t*)Y, part, cnt,
                           (int)M, (int)L.N, (int)L.K, p.steps_per_split, p.splits, L.s_off,
                           L.z_off);
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
