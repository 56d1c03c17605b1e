// w4a8_device.h -- gfx950 device helpers of the W4A8 route: the in-register
// u4 -> i8 step and the int8 MFMA operand types.
//
// Page "W4A8量化计算优化：提升LLM推理效率的关键技术", section 2.1: the int8
// weight is the byte q*s8 + a with its top bit flipped.  With s8 <= 16 and
// a + 15*s8 <= 255 no byte carries into its neighbour, so four weights are
// made at once: the four codes sit one per byte of a register (a mask), one
// v_pk_mad_u16 multiplies each byte by s8 and adds a (each 16-bit half holds
// two bytes and no product or sum passes 255), and one v_xor_b32 flips the
// four top bits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Per-(group, column) constants: S = s8 in both 16-bit halves, A = a in every
// byte.
struct GroupW8 {
    uint32_t S, A;
};

__device__ __forceinline__ GroupW8 group_w8(uint32_t meta) {
    GroupW8 g;
    g.S = (meta & 0xFFu) * 0x00010001u;
    g.A = ((meta >> 8) & 0xFFu) * 0x01010101u;
    return g;
}

// x * s + a on two 16-bit halves (v_pk_mad_u16).
__device__ __forceinline__ uint32_t mad_u16x2(uint32_t x, uint32_t s, uint32_t a) {
    const u16x2 r = __builtin_bit_cast(u16x2, x) * __builtin_bit_cast(u16x2, s) +
                    __builtin_bit_cast(u16x2, a);
    return __builtin_bit_cast(uint32_t, r);
}

// One repacked word (codes i = 0..3 at nibbles 0, 2, 4, 6 and i = 4..7 at
// nibbles 1, 3, 5, 7) -> eight int8 weights in k order: lo holds i = 0..3,
// hi holds i = 4..7, one byte each.
__device__ __forceinline__ void word_to_i8(uint32_t w, GroupW8 g, uint32_t& lo, uint32_t& hi) {
    lo = mad_u16x2(w & 0x0F0F0F0Fu, g.S, g.A) ^ 0x80808080u;
    hi = mad_u16x2((w >> 4) & 0x0F0F0F0Fu, g.S, g.A) ^ 0x80808080u;
}

// The 16-byte B operand of one k-step from two words of a chunk.
__device__ __forceinline__ i32x4 operand_b(uint32_t w0, uint32_t w1, GroupW8 g) {
    uint32_t b0, b1, b2, b3;
    word_to_i8(w0, g, b0, b1);
    word_to_i8(w1, g, b2, b3);
    i32x4 r;
    r[0] = (int)b0;
    r[1] = (int)b1;
    r[2] = (int)b2;
    r[3] = (int)b3;
    return r;
}

// Buffer resource word 3 of a raw (unstrided) buffer with range checking:
// a load at an offset past num_records returns zeros.
constexpr int kRawBufferWord3 = 0x00020000;

// Accumulator register r of lane l -> row offset inside a 32x32 tile.
__device__ __forceinline__ int acc_row_w8(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

}  // namespace w4a8
