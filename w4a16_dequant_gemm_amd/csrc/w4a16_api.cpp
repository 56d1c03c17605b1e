// w4a16_api.cpp -- the extern "C" entry points declared in include/w4a16.h:
// host-side validation (always before any HIP call), the kernel plan, and
// the launches.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "../../include/w4a16.h"
#include "w4a16_internal.h"

namespace w4a16 {

namespace {

constexpr int kDefaultCUs = 256;    // MI355X compute units (when no device answers)
constexpr int kMaxDevices = 64;
constexpr int kMaxSplits = 16;
// One uint32 counter per output tile in the workspace's counter area, which
// has the same size (kCounterBytes) for every shape, so the partial sums of
// one call never land where another call's counters live when calls share a
// workspace.
constexpr int kMaxTilesSplit = (int)(kCounterBytes / 4);
constexpr int64_t kMaxDim = (int64_t)1 << 31;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Shape checks shared by every entry point: 0 = ok, else a status.  Plan
// hints (W4A16_PLAN_*) are accepted only where a plan is made.
w4a16_status_t check_shape(int64_t K, int64_t N, int group_size, uint32_t flags,
                           bool plan_hints = false) {
    const uint32_t allowed = W4A16_FLAGS_MASK | (plan_hints ? W4A16_PLAN_BITS : 0u);
    if (flags & ~allowed) return W4A16_ERR_INVALID_ARG;
    if (K < 1 || N < 1 || K >= kMaxDim || N >= kMaxDim) return W4A16_ERR_INVALID_ARG;
    if (group_size != 32 && group_size != 64 && group_size != 128) {
        // a group size that cannot divide K is an invalid request whatever the build
        if (group_size < 1 || K % group_size != 0) return W4A16_ERR_INVALID_ARG;
        return W4A16_ERR_UNSUPPORTED;
    }
    if (K % group_size != 0) return W4A16_ERR_INVALID_ARG;
    if ((double)K * (double)N >= (double)((int64_t)1 << 40)) return W4A16_ERR_INVALID_ARG;
    if (K % kKAlign != 0 || N % kColBlock != 0) return W4A16_ERR_UNSUPPORTED;
    return W4A16_OK;
}

w4a16_status_t from_hip(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP; }

// Compute units of the current device, asked once per device (kDefaultCUs when
// no device answers, e.g. a host without a GPU asking for workspace sizes).
int num_cus() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCUs;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = kDefaultCUs;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace

Plan make_plan(int64_t M, int64_t N, int64_t K, int G, uint32_t flags) {
    Plan p;
    memset(&p, 0, sizeof(p));
    const int cus = num_cus();
    const int64_t KS = K / kKStep;
    const int64_t NB = N / kColBlock;
    const int64_t NT = N / kTileCols;
    const uint32_t hint = flags & W4A16_PLAN_MASK;
    const int param = (int)((flags >> W4A16_PLAN_PARAM_SHIFT) & 0xFFu);
    (void)G;

    // The decode kernel holds X in LDS: it serves M <= 8 whenever X fits.
    auto decode_fits = [&](int tpi) {
        return M <= kDecodeMaxRows && decode_lds_bytes(M, K, tpi, kDecodeMaxRows) <= kDecodeLdsMax;
    };
    // The wide kernel serves 32 < M <= 128 (its steps need K to hold at least
    // one step per half).  Measured on MI355X (K = 8192, fp16): faster than
    // the tiled kernel for M <= 96 (N = 28672 M = 96: 74-77 vs 83 us), and
    // for every M up to 128 when the 128-column blocks cover at most half
    // of the CUs (N = 8192: 31-49 vs 41-77 us); at N = 28672 M = 128 the
    // tiled kernel is faster (85 vs 90-95 us).
    const bool wide_fits = M >= kWideMinRows && M <= kWideMaxRows && K >= 2 * wide_step_k(M);
    const bool wide_default = wide_fits && (M <= 96 || NB * 2 <= cus);
    Variant v;
    if (hint == W4A16_PLAN_DECODE && decode_fits(1))
        v = VARIANT_DECODE;
    else if (hint == W4A16_PLAN_SPLITK && M <= 32)
        v = VARIANT_SPLITK;
    else if (hint == W4A16_PLAN_TILED)
        v = VARIANT_TILED;
    else if (hint == W4A16_PLAN_WIDE && wide_fits)
        v = VARIANT_WIDE;
    else if (decode_fits(1))
        v = VARIANT_DECODE;
    else if (M <= 32)
        v = VARIANT_SPLITK;
    else if (wide_default)
        v = VARIANT_WIDE;
    else
        v = VARIANT_TILED;

    if (v == VARIANT_DECODE) {
        // Items of one tile over all of K, one workgroup per CU (or the forced
        // count).  F = items / W whole rounds are dealt round-robin; the R =
        // items % W left over are split along K into S = W / R parts (at most
        // KB / 8, so that every wave has a body of each part, and at most 8),
        // one per workgroup, so that every workgroup gets the same share.
        // Split parts meet in the workspace (one counter per split item).
        p.variant = VARIANT_DECODE;
        p.tpi = 1;
        p.items = (int)NT;
        p.waves = kDecodeWaves;
        int64_t W = cus;
        const bool forced = hint == W4A16_PLAN_DECODE && param > 0;
        if (forced) W = param;   // forced workgroup count
        const int64_t F = NT / W, R = NT % W;
        int64_t S = R > 0 ? std::min<int64_t>({W / R, K / kBodyK / kDecodeWaves, 8}) : 1;
        if (S < 2 || R > kMaxTilesSplit) S = 1;
        // Fewer tiles than workgroups (F = 0): every tile would be split, and
        // every workgroup would end with a cross-workgroup meeting.  Measured
        // on MI355X (us per call, graph replay): K = N = 4096 M = 1 6.2
        // unsplit vs 7.35 in halves, M = 4 6.55 vs 7.8; K = 8192 N = 4096
        // 7.9 vs 8.7.  So tiles stay whole there unless K is larger.
        if (F == 0 && K <= kDecodeWholeTileMaxK && !forced) S = 1;
        p.grid_x = (int)(S > 1 ? (F > 0 ? W : R * S) : std::min<int64_t>(NT, W));
        p.grid_y = 1;
        p.grid_z = 1;
        p.splits = (int)S;
        p.tiles = S > 1 ? (int)R : 0;
        p.tile_floats = (size_t)64 * 4;   // one part: 8 rows x 32 columns (64 lanes x 4)
    } else if (v == VARIANT_WIDE) {
        // Items of one 128-column block over all of K, one workgroup per CU
        // (or the forced count), round-robin; with fewer blocks than
        // workgroups each block's K is split into S parts (at most 8, and at
        // most one per two steps of K), one workgroup per (block, part).
        p.variant = VARIANT_WIDE;
        p.items = (int)NB;
        p.waves = kWideWaves;
        int64_t W = cus;
        if (hint == W4A16_PLAN_WIDE && param > 0) W = param;   // forced workgroup count
        const int64_t T = K / wide_step_k(M);
        int64_t S = NB < W ? std::min<int64_t>({W / NB, T / 2, 8}) : 1;
        if (S < 2 || NB > kMaxTilesSplit) S = 1;
        p.grid_x = (int)(S > 1 ? NB * S : std::min<int64_t>(NB, W));
        p.grid_y = 1;
        p.grid_z = 1;
        p.splits = (int)S;
        p.tiles = S > 1 ? (int)NB : 0;
        // one part of a block: 4 tiles x (32-row tiles) x 16 registers x 64 lanes
        p.tile_floats = (size_t)4 * ((M + 31) / 32) * 16 * 64;
    } else if (v == VARIANT_SPLITK) {
        // Balanced contiguous ranges of batches for every wave of one
        // workgroup per CU (fewer workgroups when there are fewer batches).
        p.variant = VARIANT_SPLITK;
        p.mt = 1;
        p.waves = kSplitKWaves;
        p.nbat = (int)ceil_div(KS, kSplitKBatch);
        const int64_t TB = NB * p.nbat;
        // Measured on MI355X: whole column blocks per workgroup (no partial
        // tiles shared between workgroups) when that still occupies at least
        // 3/4 of the CUs; otherwise one workgroup per CU, but at least two
        // batches per wave (small problems pay more for shared tiles than
        // they gain from more CUs).
        const int64_t per_wg = ceil_div(NB, cus);               // blocks per workgroup
        int64_t W = ceil_div(NB, per_wg);
        if (W * 4 < (int64_t)cus * 3) W = cus;
        if (W > TB / (2 * p.waves)) W = TB / (2 * p.waves);
        if (W < 1) W = 1;
        if (hint == W4A16_PLAN_SPLITK && param > 0) W = (int64_t)param * 8;  // forced: 8*param
        if (W > ceil_div(TB, p.waves)) W = ceil_div(TB, p.waves);   // every workgroup has work
        if (W > kMaxTilesSplit) W = kMaxTilesSplit;                  // counters fit their area
        const int64_t TW = W * p.waves;
        p.base = (int)(TB / TW);
        p.rem = (int)(TB % TW);
        p.grid_x = (int)W;
        p.grid_y = 1;
        p.grid_z = 1;
        // A column block is shared by workgroups when a workgroup boundary
        // falls inside it; each workgroup then has at most two partial tiles
        // (its first and its last column block) and the counter of a shared
        // block is indexed by the first workgroup that touches it.
        bool shared = false;
        for (int64_t g = 1; g < W && !shared; ++g) {
            const int64_t gw = g * p.waves;
            const int64_t b = gw * p.base + (gw < p.rem ? gw : p.rem);
            shared = b % p.nbat != 0;
        }
        p.tiles = (int)W;
        p.tile_floats = (size_t)4 * M * 32;
        p.splits = shared ? 2 : 1;                              // partial tiles per workgroup
    } else {
        p.variant = VARIANT_TILED;
        p.mt = M <= 64 ? 2 : 4;
        p.waves = 8;
        const int64_t CG = ceil_div(NB, 4);
        const int64_t RB = ceil_div(M, 32 * p.mt);
        const int64_t tiles = CG * RB;
        // Split K over workgroups when there are fewer tiles than CUs, as far
        // as one round of workgroups (one per CU) goes: measured on MI355X, a
        // second round or more partial tiles cost more than they gain.
        int64_t s = 1;
        if (tiles < cus) s = cus / tiles;
        if (s > kMaxSplits) s = kMaxSplits;
        if (hint == W4A16_PLAN_TILED && param > 0) s = param < kMaxSplits ? param : kMaxSplits;
        // at least 4 stages per split, and whole bodies (two stages) per split
        int64_t sps = round_up(ceil_div(KS, s), 2 * kTiledStage);
        if (sps < 4 * kTiledStage) sps = 4 * kTiledStage;
        p.steps_per_split = (int)sps;
        p.splits = (int)ceil_div(KS, sps);
        p.grid_x = (int)CG;
        p.grid_y = (int)RB;
        p.grid_z = p.splits;
        p.tiles = (int)tiles;
        p.tile_floats = (size_t)4 * p.mt * 4 * 16 * 64;
    }
    if (p.variant == VARIANT_TILED && p.splits > 1 && p.tiles > kMaxTilesSplit) {
        // enough tiles to fill the machine without splitting K
        p.splits = 1;
        p.steps_per_split = (int)round_up(KS, 2 * kTiledStage);
        p.grid_z = 1;
    }
    if (p.splits > 1) {
        p.counters_bytes = kCounterBytes;
        p.workspace = p.counters_bytes + (size_t)p.tiles * p.splits * p.tile_floats * 4;
    } else {
        p.tiles = 0;
        p.counters_bytes = 0;
        p.workspace = 0;
    }
    return p;
}

}  // namespace w4a16

namespace w4a16 {

hipError_t launch_gemm(const void* X, const void* packed, void* Y, int64_t M, const Layout& L,
                       bool bf16, const Plan& plan, void* workspace, const Epilogue& ep,
                       hipStream_t stream) {
    if (plan.variant == VARIANT_DECODE) {
        if (bf16)
            return ep.any ? launch_decode_bf16_ep(X, packed, Y, M, L, plan, workspace, ep, stream)
                          : launch_decode_bf16(X, packed, Y, M, L, plan, workspace, ep, stream);
        return ep.any ? launch_decode_f16_ep(X, packed, Y, M, L, plan, workspace, ep, stream)
                      : launch_decode_f16(X, packed, Y, M, L, plan, workspace, ep, stream);
    }
    if (plan.variant == VARIANT_WIDE) {
        if (bf16)
            return ep.any ? launch_wide_bf16_ep(X, packed, Y, M, L, plan, workspace, ep, stream)
                          : launch_wide_bf16(X, packed, Y, M, L, plan, workspace, ep, stream);
        return ep.any ? launch_wide_f16_ep(X, packed, Y, M, L, plan, workspace, ep, stream)
                      : launch_wide_f16(X, packed, Y, M, L, plan, workspace, ep, stream);
    }
    if (bf16)
        return ep.any ? launch_gemm_bf16_ep(X, packed, Y, M, L, plan, workspace, ep, stream)
                      : launch_gemm_bf16(X, packed, Y, M, L, plan, workspace, ep, stream);
    return ep.any ? launch_gemm_f16_ep(X, packed, Y, M, L, plan, workspace, ep, stream)
                  : launch_gemm_f16(X, packed, Y, M, L, plan, workspace, ep, stream);
}

w4a16_status_t prepare_gemm(const void* X, const void* packed, size_t packed_bytes, void* Y,
                            int64_t M, int64_t N, int64_t K, int group_size, uint32_t flags,
                            const w4a16_epilogue_t* epilogue, GemmCall* out) {
    if (M < 1 || M >= kMaxDim) return W4A16_ERR_INVALID_ARG;
    w4a16_status_t st = check_shape(K, N, group_size, flags, true);
    if (st != W4A16_OK) return st;
    if (!X || !packed || !Y) return W4A16_ERR_INVALID_ARG;
    if (!aligned16(X) || !aligned16(packed) || !aligned16(Y)) return W4A16_ERR_INVALID_ARG;
    if ((double)M * (double)K >= (double)((int64_t)1 << 40) ||
        (double)M * (double)N >= (double)((int64_t)1 << 40))
        return W4A16_ERR_INVALID_ARG;
    Epilogue& ep = out->ep;
    memset(&ep, 0, sizeof(ep));
    if (epilogue) {
        const w4a16_epilogue_t& e = *epilogue;
        if (e.activation < W4A16_ACT_NONE || e.activation > W4A16_ACT_SILU) return W4A16_ERR_INVALID_ARG;
        if (e.aux_op != W4A16_AUX_ADD && e.aux_op != W4A16_AUX_MUL) return W4A16_ERR_INVALID_ARG;
        if (((uintptr_t)e.col_scale & 3) || ((uintptr_t)e.bias & 1) || ((uintptr_t)e.aux & 1))
            return W4A16_ERR_INVALID_ARG;
        if (e.aux && e.aux != Y) {   // aux is Y itself (in place) or disjoint from it
            const uintptr_t a0 = (uintptr_t)e.aux, y0 = (uintptr_t)Y;
            const uintptr_t bytes = (uintptr_t)(M * N * 2);
            if (a0 < y0 + bytes && y0 < a0 + bytes) return W4A16_ERR_INVALID_ARG;
        }
        // absent operands read harmless memory of at least their size: the
        // blob (>= K*N/2 >= 16*N bytes) for [N] operands, Y for [M][N]
        ep.has_scale = e.col_scale != nullptr;
        ep.has_bias = e.bias != nullptr;
        ep.has_aux = e.aux != nullptr;
        ep.col_scale = e.col_scale ? e.col_scale : (const float*)packed;
        ep.bias = (const uint16_t*)(e.bias ? e.bias : packed);
        ep.aux = (const uint16_t*)(e.aux ? e.aux : Y);
        ep.act = e.activation;
        ep.aux_mul = e.aux_op == W4A16_AUX_MUL;
        ep.any = ep.has_scale || ep.has_bias || ep.has_aux || e.activation != W4A16_ACT_NONE;
    }
    out->layout = make_layout(K, N, group_size, (flags & W4A16_SYM) != 0);
    if (packed_bytes < out->layout.total) return W4A16_ERR_INVALID_ARG;
    out->plan = make_plan(M, N, K, group_size, flags);
    out->bf16 = (flags & W4A16_BF16) != 0;
    return W4A16_OK;
}

w4a16_status_t run_gemm(const GemmCall& c, const void* X, const void* packed, void* Y, int64_t M,
                        void* workspace, hipStream_t stream) {
    return from_hip(launch_gemm(X, packed, Y, M, c.layout, c.bf16, c.plan, workspace, c.ep,
                                stream));
}

}  // namespace w4a16

using namespace w4a16;

extern "C" {

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

int w4a16_layout_version(void) { return W4A16_LAYOUT_VERSION; }

const char* w4a16_status_string(w4a16_status_t s) {
    switch (s) {
        case W4A16_OK: return "ok";
        case W4A16_ERR_INVALID_ARG: return "invalid argument";
        case W4A16_ERR_UNSUPPORTED: return "unsupported shape or group size";
        case W4A16_ERR_WORKSPACE: return "workspace missing or too small";
        case W4A16_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t w4a16_packed_bytes(int64_t K, int64_t N, int group_size, uint32_t flags) {
    if (check_shape(K, N, group_size, flags) != W4A16_OK) return 0;
    return make_layout(K, N, group_size, (flags & W4A16_SYM) != 0).total;
}

w4a16_status_t w4a16_repack(const uint32_t* qweight, const void* scales, const uint8_t* zeros,
                            int64_t K, int64_t N, int group_size, uint32_t flags, void* packed,
                            size_t packed_bytes, void* stream) {
    w4a16_status_t st = check_shape(K, N, group_size, flags);
    if (st != W4A16_OK) return st;
    const bool sym = (flags & W4A16_SYM) != 0;
    if (sym != (zeros == nullptr)) return W4A16_ERR_INVALID_ARG;
    if (!qweight || !scales || !packed) return W4A16_ERR_INVALID_ARG;
    if (!aligned16(qweight) || !aligned16(scales) || !aligned16(packed) ||
        (zeros && !aligned16(zeros)))
        return W4A16_ERR_INVALID_ARG;
    const Layout L = make_layout(K, N, group_size, sym);
    if (packed_bytes < L.total) return W4A16_ERR_INVALID_ARG;
    return from_hip(launch_repack(qweight, scales, zeros, L, (flags & W4A16_BF16) != 0, packed,
                                  (hipStream_t)stream));
}

w4a16_status_t w4a16_unrepack(const void* packed, size_t packed_bytes, uint32_t* qweight,
                              void* scales, uint8_t* zeros, int64_t K, int64_t N, int group_size,
                              uint32_t flags, void* stream) {
    w4a16_status_t st = check_shape(K, N, group_size, flags);
    if (st != W4A16_OK) return st;
    const bool sym = (flags & W4A16_SYM) != 0;
    if (sym != (zeros == nullptr)) return W4A16_ERR_INVALID_ARG;
    if (!qweight || !scales || !packed) return W4A16_ERR_INVALID_ARG;
    if (!aligned16(qweight) || !aligned16(scales) || !aligned16(packed) ||
        (zeros && !aligned16(zeros)))
        return W4A16_ERR_INVALID_ARG;
    const Layout L = make_layout(K, N, group_size, sym);
    if (packed_bytes < L.total) return W4A16_ERR_INVALID_ARG;
    return from_hip(launch_unrepack(packed, L, (flags & W4A16_BF16) != 0, qweight, scales, zeros,
                                    (hipStream_t)stream));
}

size_t w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int group_size, uint32_t flags) {
    if (M < 1 || M >= kMaxDim || check_shape(K, N, group_size, flags, true) != W4A16_OK) return 0;
    return make_plan(M, N, K, group_size, flags).workspace;
}

w4a16_status_t w4a16_gemm_ex(const void* X, const void* packed, size_t packed_bytes, void* Y,
                             int64_t M, int64_t N, int64_t K, int group_size, uint32_t flags,
                             const w4a16_epilogue_t* epilogue, void* workspace,
                             size_t workspace_bytes, void* stream) {
    GemmCall c;
    const w4a16_status_t st =
        prepare_gemm(X, packed, packed_bytes, Y, M, N, K, group_size, flags, epilogue, &c);
    if (st != W4A16_OK) return st;
    if (c.plan.workspace > 0) {
        if (!workspace || workspace_bytes < c.plan.workspace || !aligned16(workspace))
            return W4A16_ERR_WORKSPACE;
    }
    return run_gemm(c, X, packed, Y, M, workspace, (hipStream_t)stream);
}

w4a16_status_t w4a16_gemm(const void* X, const void* packed, size_t packed_bytes, void* Y,
                          int64_t M, int64_t N, int64_t K, int group_size, uint32_t flags,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return w4a16_gemm_ex(X, packed, packed_bytes, Y, M, N, K, group_size, flags, nullptr,
                         workspace, workspace_bytes, stream);
}

w4a16_status_t w4a16_dequant(const void* packed, size_t packed_bytes, void* W_out, int64_t K,
                             int64_t N, int group_size, uint32_t flags, void* stream) {
    w4a16_status_t st = check_shape(K, N, group_size, flags);
    if (st != W4A16_OK) return st;
    if (!packed || !W_out || !aligned16(packed) || !aligned16(W_out)) return W4A16_ERR_INVALID_ARG;
    const Layout L = make_layout(K, N, group_size, (flags & W4A16_SYM) != 0);
    if (packed_bytes < L.total) return W4A16_ERR_INVALID_ARG;
    return from_hip(launch_dequant(packed, L, (flags & W4A16_BF16) != 0, W_out,
                                   (hipStream_t)stream));
}

size_t w4a16_read_probe_out_bytes(void) { return (size_t)kProbeBlocks * kProbeThreads * 16; }

w4a16_status_t w4a16_read_probe(const void* buf, size_t bytes, void* out, size_t out_bytes,
                                void* stream) {
    if (!buf || !out || !aligned16(buf) || !aligned16(out)) return W4A16_ERR_INVALID_ARG;
    if (bytes == 0 || bytes % kChunkBytes != 0) return W4A16_ERR_INVALID_ARG;
    if (out_bytes < w4a16_read_probe_out_bytes()) return W4A16_ERR_INVALID_ARG;
    return from_hip(launch_read_probe(buf, bytes, out, (hipStream_t)stream));
}

w4a16_status_t w4a16_mfma_layout_probe(const void* A, const void* B, float* D, uint32_t flags,
                                       void* stream) {
    if (flags & ~W4A16_BF16) return W4A16_ERR_INVALID_ARG;
    if (!A || !B || !D || !aligned16(A) || !aligned16(B) || !aligned16(D))
        return W4A16_ERR_INVALID_ARG;
    return from_hip(launch_mfma_probe(A, B, D, (flags & W4A16_BF16) != 0, (hipStream_t)stream));
}

}  // extern "C"
