// w4a16_device.h -- gfx950 device helpers: in-register unpack + group dequant,
// MFMA operand types, output rounding.
//
// Page "W4A16 GEMM 算子浅析" (nxmr.cn), sections "计算流水线的核心哲学" and
// "Marlin 与 CUTLASS 中的寄存器解包黑魔法": split a 32-bit word into its eight
// nibbles with masks and shifts, turn each nibble into a 16-bit float by
// placing it in the fraction field of a float whose spacing is 1 (no
// integer-to-float convert instruction), then subtract the zero point and
// multiply by the group scale before the values enter the matrix unit.
// Page "量化开销对比", section 6.3: the unpacked values must land directly in
// the operand registers the matrix instruction expects.
//
// Rounding: each dequantized weight is RNE((q - z) * s) in the activation
// dtype, the single rounding of the exact product.
//   fp16: (1024+q) - (1024+z) and (64+q) - (64+z) are exact small integers in
//         fp16, so v_pk_add_f16 is exact and v_pk_mul_f16 rounds once.  (A
//         fused multiply-add against a pre-multiplied zero would round the
//         addend first and is not exact.)
//   bf16: there is no packed bf16 arithmetic on gfx950, so each value goes
//         through fp32.  The nibbles are unpacked with the same fp16 trick as
//         above (1024+q or 64+q, exact), and one v_fma_mix_f32 per value reads
//         that fp16 half straight from the packed register: fma(B+q, s,
//         -(B+z)*s) is (q - z) * s exactly (B+z has at most 11 significant
//         bits and s 8, so -(B+z)*s is exact in fp32, and so is the result),
//         then v_cvt_pk_bf16_f32 rounds once per value.  When -(1024+z)*s
//         overflows fp32 (scales above about 3.2e35) the launch uses
//         (q - z) * s instead, also exact before the one rounding (a flag in
//         the blob trailer).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

// Buffer resource word 3 for raw (untyped) buffer accesses, and the cache
// policy bit of device-scope accesses (sc1: they bypass the per-XCD L2, the
// same policy the device-scope atomics use), for partial sums exchanged
// between workgroups.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kDeviceScope = 16;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { DT_F16 = 0, DT_BF16 = 1 };

// Per-column dequantization constants for one group.
template <int DT>
struct ColParams;

template <>
struct ColParams<DT_F16> {
    uint32_t s2;   // (s, s) as two fp16
    uint32_t bA;   // (1024+z, 1024+z): bias of pairs taken with mask 0x000F000F
    uint32_t bB;   // (64+z, 64+z): bias of pairs taken with mask 0x00F000F0
};

template <>
struct ColParams<DT_BF16> {
    float s;       // the scale, exactly
    float cA;      // -(1024+z)*s, exact in fp32 unless it overflows (then infinite)
    float cB;      // -(64+z)*s, exact in fp32 when cA is finite
    float zneg;    // -z (used only by the exact form)
};

__device__ __forceinline__ ColParams<DT_F16> make_params(uint32_t sbits, uint32_t z,
                                                         ColParams<DT_F16>*) {
    ColParams<DT_F16> p;
    p.s2 = sbits * 0x00010001u;
    p.bA = (0x6400u | z) * 0x00010001u;          // fp16 1024 + z
    p.bB = (0x5400u | (z << 4)) * 0x00010001u;   // fp16 64 + z (spacing 1/16 at 64)
    return p;
}

__device__ __forceinline__ ColParams<DT_BF16> make_params(uint32_t sbits, uint32_t z,
                                                          ColParams<DT_BF16>*) {
    ColParams<DT_BF16> p;
    p.s = __uint_as_float(sbits << 16);
    p.cA = -((float)(1024u + z) * p.s);
    p.cB = -((float)(64u + z) * p.s);
    p.zneg = -(float)z;
    return p;
}

template <int DT>
__device__ __forceinline__ ColParams<DT> col_params(uint32_t sbits, uint32_t z) {
    return make_params(sbits, z, (ColParams<DT>*)nullptr);
}

// A value the compiler must treat as unknown (kept in a VGPR): stops it from
// re-deriving bit ranges and picking longer instruction sequences.
__device__ __forceinline__ uint32_t opaque_v(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

__device__ __forceinline__ float opaque_f(float v) {
    asm("" : "+v"(v));
    return v;
}

// (x & m) | g in one VALU instruction.  The backend splits it into v_and +
// v_or when both constants are literals (gfx9 VOP3 takes no literal and one
// scalar operand), so it is written out: mask in an SGPR, g in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t g) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(g));
    return r;
}

// The two fp16 exponent-bias patterns of the unpack (1024 and 64 in both
// halves), held in VGPRs the compiler treats as unknown values: made once per
// kernel and passed to every dequant_word, so they are not re-materialised
// for each word.
struct Magic {
    uint32_t a;   // 0x64006400: fp16 1024, spacing 1
    uint32_t b;   // 0x54005400: fp16 64, spacing 1/16
};
__device__ __forceinline__ Magic make_magic() { return Magic{opaque_v(0x64006400u), opaque_v(0x54005400u)}; }

// Eight dequantized weights of one repacked word as the four dwords of an
// MFMA operand: dword i holds (j = 2i, j = 2i+1) in its (low, high) halves.
// 13 VALU instructions: 1 shift, 4 v_and_or_b32, 4 v_pk_add_f16, 4 v_pk_mul_f16.
__device__ __forceinline__ u32x4 dequant_word(uint32_t w, const ColParams<DT_F16>& p,
                                              const Magic& mg) {
    const uint32_t w8 = w >> 8;
    const f16x2 s2 = __builtin_bit_cast(f16x2, p.s2);
    const f16x2 bA = __builtin_bit_cast(f16x2, p.bA);
    const f16x2 bB = __builtin_bit_cast(f16x2, p.bB);
    const uint32_t gA = mg.a;   // fp16 1024 in both halves
    const uint32_t gB = mg.b;   // fp16 64 in both halves
    // nibble positions (0,4) -> j (0,1); (1,5) -> (2,3); (2,6) -> (4,5); (3,7) -> (6,7)
    const f16x2 v0 = __builtin_bit_cast(f16x2, and_or(w, 0x000F000Fu, gA));    // 1024 + q
    const f16x2 v1 = __builtin_bit_cast(f16x2, and_or(w, 0x00F000F0u, gB));    // 64 + q
    const f16x2 v2 = __builtin_bit_cast(f16x2, and_or(w8, 0x000F000Fu, gA));
    const f16x2 v3 = __builtin_bit_cast(f16x2, and_or(w8, 0x00F000F0u, gB));
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, (f16x2)((v0 - bA) * s2));
    r.y = __builtin_bit_cast(uint32_t, (f16x2)((v1 - bB) * s2));
    r.z = __builtin_bit_cast(uint32_t, (f16x2)((v2 - bA) * s2));
    r.w = __builtin_bit_cast(uint32_t, (f16x2)((v3 - bB) * s2));
    return r;
}

// (q - z) of the eight weights of one repacked word, exact small integers in
// fp16, as the four dwords of an MFMA operand (the group scale is applied to
// the product later).  bA = (1024+z, 1024+z), bB = (64+z, 64+z) as fp16.
// 9 VALU instructions: 1 shift, 4 v_and_or_b32, 4 v_pk_add_f16.
__device__ __forceinline__ u32x4 unpack_qz(uint32_t w, uint32_t bA_bits, uint32_t bB_bits,
                                           const Magic& mg) {
    const uint32_t w8 = w >> 8;
    const f16x2 bA = __builtin_bit_cast(f16x2, bA_bits);
    const f16x2 bB = __builtin_bit_cast(f16x2, bB_bits);
    const f16x2 v0 = __builtin_bit_cast(f16x2, and_or(w, 0x000F000Fu, mg.a));    // 1024 + q
    const f16x2 v1 = __builtin_bit_cast(f16x2, and_or(w, 0x00F000F0u, mg.b));    // 64 + q
    const f16x2 v2 = __builtin_bit_cast(f16x2, and_or(w8, 0x000F000Fu, mg.a));
    const f16x2 v3 = __builtin_bit_cast(f16x2, and_or(w8, 0x00F000F0u, mg.b));
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, (f16x2)(v0 - bA));
    r.y = __builtin_bit_cast(uint32_t, (f16x2)(v1 - bB));
    r.z = __builtin_bit_cast(uint32_t, (f16x2)(v2 - bA));
    r.w = __builtin_bit_cast(uint32_t, (f16x2)(v3 - bB));
    return r;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    // one v_cvt_pk_bf16_f32: both values rounded to nearest even
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ u32x4 dequant_word(uint32_t w, const ColParams<DT_BF16>& p,
                                              const Magic& mg) {
    // The same four (j, j+1) pairs as the fp16 form, each half widened inside
    // the fma (v_fma_mix_f32): 1 shift, 4 v_and_or_b32, 8 fma, 4 cvt.
    const uint32_t w8 = w >> 8;
    const uint32_t gA = mg.a;   // fp16 1024 in both halves
    const uint32_t gB = mg.b;   // fp16 64 in both halves
    const f16x2 v0 = __builtin_bit_cast(f16x2, and_or(w, 0x000F000Fu, gA));    // 1024 + q
    const f16x2 v1 = __builtin_bit_cast(f16x2, and_or(w, 0x00F000F0u, gB));    // 64 + q
    const f16x2 v2 = __builtin_bit_cast(f16x2, and_or(w8, 0x000F000Fu, gA));
    const f16x2 v3 = __builtin_bit_cast(f16x2, and_or(w8, 0x00F000F0u, gB));
    u32x4 r;
    r.x = pack_bf16x2(__builtin_fmaf((float)v0.x, p.s, p.cA), __builtin_fmaf((float)v0.y, p.s, p.cA));
    r.y = pack_bf16x2(__builtin_fmaf((float)v1.x, p.s, p.cB), __builtin_fmaf((float)v1.y, p.s, p.cB));
    r.z = pack_bf16x2(__builtin_fmaf((float)v2.x, p.s, p.cA), __builtin_fmaf((float)v2.y, p.s, p.cA));
    r.w = pack_bf16x2(__builtin_fmaf((float)v3.x, p.s, p.cB), __builtin_fmaf((float)v3.y, p.s, p.cB));
    return r;
}

// The fma form above needs -(1024+z)*s to be exact; it overflows fp32 only
// for scales beyond fp32_max/1039 (about 3.2e35).  For such columns this form is
// used instead: (q - z) exactly, then one product, then one RNE.
__device__ __forceinline__ bool needs_exact_path(const ColParams<DT_F16>&) { return false; }
__device__ __forceinline__ bool needs_exact_path(const ColParams<DT_BF16>& p) {
    return __builtin_isinf(p.cA);
}

__device__ __forceinline__ u32x4 dequant_word_exact(uint32_t w, const ColParams<DT_F16>& p,
                                                    const Magic& mg) {
    return dequant_word(w, p, mg);   // the fp16 form is exact for every scale
}

__device__ __forceinline__ u32x4 dequant_word_exact(uint32_t w, const ColParams<DT_BF16>& p,
                                                    const Magic&) {
    float v[8];
#pragma unroll
    for (int p_ = 0; p_ < 8; ++p_) {
        const int j = 2 * (p_ & 3) + (p_ >> 2);
        v[j] = ((float)((w >> (4 * p_)) & 0xFu) + p.zneg) * p.s;
    }
    u32x4 r;
    r.x = pack_bf16x2(v[0], v[1]);
    r.y = pack_bf16x2(v[2], v[3]);
    r.z = pack_bf16x2(v[4], v[5]);
    r.w = pack_bf16x2(v[6], v[7]);
    return r;
}

template <bool EXACT, int DT>
__device__ __forceinline__ u32x4 dequant_sel(uint32_t w, const ColParams<DT>& p, const Magic& mg) {
    if constexpr (EXACT)
        return dequant_word_exact(w, p, mg);
    else
        return dequant_word(w, p, mg);
}

// Constants of group entry e of a lane's scale / zero record entries: the
// scale is 16-bit field e % 2 of `sword` (the record dword that holds entry e)
// and the zero point is nibble e of `zword` (8 for the symmetric format).
template <int DT, bool SYM>
__device__ __forceinline__ ColParams<DT> entry_params(uint32_t sword, uint32_t zword, int e) {
    const uint32_t sbits = (e & 1) ? (sword >> 16) : (sword & 0xFFFFu);
    const uint32_t z = SYM ? 8u : ((zword >> (4 * e)) & 0xFu);
    return col_params<DT>(sbits, z);
}

// Scale entry of a lane for one body: 256/G scales (4, 8 or 16 bytes).
template <int G>
struct SEnt;
template <>
struct SEnt<128> {
    uint32_t v;
    __device__ uint32_t word(int) const { return v; }
};
// word(i) selects with comparisons rather than indexing the vector: an index
// known only at run time (the split-K kernel's batch phase) would otherwise
// send the vector to scratch memory.
template <>
struct SEnt<64> {
    u32x2 v;
    __device__ uint32_t word(int i) const { return i ? v[1] : v[0]; }
};
template <>
struct SEnt<32> {
    u32x4 v;
    __device__ uint32_t word(int i) const {
        const uint32_t lo = (i & 1) ? v[1] : v[0];
        const uint32_t hi = (i & 1) ? v[3] : v[2];
        return (i & 2) ? hi : lo;
    }
};

template <int G>
__device__ __forceinline__ SEnt<G> load_sent(const uint8_t* p) {
    SEnt<G> s;
    if constexpr (G == 128)
        s.v = *(const uint32_t*)p;
    else if constexpr (G == 64)
        s.v = *(const u32x2*)p;
    else
        s.v = *(const u32x4*)p;
    return s;
}

// Zero entry of a lane for one body: 256/G nibbles (1, 2 or 4 bytes), read as
// the aligned dword that holds it (sub-dword loads make the compiler insert
// zero-extensions that wait for every load in flight).  The entry sits at bit
// zent_shift<G>(c32) of that dword.
template <int G>
__device__ __forceinline__ uint32_t load_zent(const uint8_t* p) {
    // pointer arithmetic (not an integer round trip) keeps the global address
    // space, so this stays a global load (a flat load is waited for with
    // vmcnt(0), i.e. after every load in flight)
    return *(const uint32_t*)(p - ((uintptr_t)p & 3));
}
template <int G>
__device__ __forceinline__ uint32_t zent_shift(int c32) {
    if constexpr (G == 128)
        return 8u * (uint32_t)(c32 & 3);
    else if constexpr (G == 64)
        return 16u * (uint32_t)(c32 & 1);
    else
        return 0u;
}

// D = A.B + C on one 32x32x16 tile.  A: lane l holds row l%32, reduction
// indices 8*(l/32)..+7; B: lane l holds column l%32, the same indices; C/D:
// lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mfma32x32x16<DT_F16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mfma32x32x16<DT_BF16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D = A.B + C on one 16x16x32 tile.  A: lane l holds row l%16, reduction
// indices 8*(l/16)..+7; B: lane l holds column l%16, the same indices; C/D:
// lane l, register r holds row 4*(l/16) + r, column l%16.  As for the 32x32
// form, only the lane groups matter: lanes 16o..16o+15 of A and of B supply
// the same eight reduction indices.
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c);

template <>
__device__ __forceinline__ f32x4 mfma16x16x32<DT_F16>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mfma16x16x32<DT_BF16>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 -> activation dtype, round to nearest even.
template <int DT>
__device__ __forceinline__ uint16_t round_out(float v);

template <>
__device__ __forceinline__ uint16_t round_out<DT_F16>(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

template <>
__device__ __forceinline__ uint16_t round_out<DT_BF16>(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Accumulator register r of lane l -> row offset inside a 32x32 tile.
__device__ __forceinline__ int acc_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

}  // namespace w4a16
