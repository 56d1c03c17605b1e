// w4a16_epilogue.h -- the fused output epilogue, run on an fp32 accumulator
// just before its one store, shared by the GEMM kernels.
//
// Page "量化开销对比" (laojiahuo2003.github.io), sections 6.2, 6.6 and 6.7:
// after the k loop the result is scaled per output channel, the bias added,
// and a residual or activation applied inside the same kernel, so no further
// launch re-reads Y.  Each step is optional; the order is t = v*c[n] + b[n],
// u = act(t), then u + a[m][n] or u * a[m][n].  All in fp32, one rounding into
// the output dtype.
#pragma once
#include <hip/hip_runtime.h>

#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {

template <int DT>
__device__ __forceinline__ float act_in(uint16_t b) {
    if constexpr (DT == DT_F16)
        return (float)__builtin_bit_cast(_Float16, b);
    else
        return __uint_as_float((uint32_t)b << 16);
}

// EP = false: the plain store value.  EP = true: every pointer of ep is valid
// (the host substitutes a harmless source for an absent operand), so each
// element runs the same straight-line code: unconditional loads, then
// selects.
template <int DT, bool EP>
__device__ __forceinline__ __attribute__((always_inline)) uint16_t
out_value(float v, int64_t row, int64_t col, int N, const Epilogue& ep) {
    if constexpr (EP) {
        const float c = ep.has_scale ? ep.col_scale[col] : 1.0f;
        const float b = ep.has_bias ? act_in<DT>(ep.bias[col]) : 0.0f;
        const float a = act_in<DT>(ep.aux[row * N + col]);
        const float t = v * c + b;
        // SiLU as t * 1/(1 + 2^(-t*log2 e)) with the hardware exp2 and reciprocal
        const float sg =
            t * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-t * 1.4426950408889634f));
        const float u = ep.act == kActSilu ? sg : (ep.act == kActRelu ? (t > 0.0f ? t : 0.0f) : t);
        v = ep.has_aux ? (ep.aux_mul ? u * a : u + a) : u;
    }
    return round_out<DT>(v);
}

}  // namespace w4a16
