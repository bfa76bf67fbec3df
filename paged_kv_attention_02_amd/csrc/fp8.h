// OCP e4m3fn conversions shared by the kernels (gfx950 device code): the
// encoder of the cache writers and the exact decoder of the readers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pka {

// fp32 -> e4m3fn code, saturating at +-448, round to nearest even.  Written
// on the bit pattern: the fp32 exponent is rebiased (127 -> 7) and the 23-bit
// mantissa rounded to 3 bits; below 2^-6 the value is a multiple of 2^-9.
__device__ __forceinline__ uint32_t e4m3fn_from_f32(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;             // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;     // |y| >= 448 (and inf): saturate
    if (a < 0x3c800000u) {                         // |y| < 2^-6: subnormal codes 0..8
        const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
        return sign | (uint32_t)m;
    }
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);  // RNE on the 20 dropped bits
    return sign | ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, float inv) {
    return e4m3fn_from_f32(bf16_lo(w0) * inv) | (e4m3fn_from_f32(bf16_hi(w0) * inv) << 8) |
           (e4m3fn_from_f32(bf16_lo(w1) * inv) << 16) | (e4m3fn_from_f32(bf16_hi(w1) * inv) << 24);
}

// Two e4m3fn codes (bytes 0,1 or, with HI, bytes 2,3 of w) -> two bf16, exact
// (every e4m3fn value has a bf16 representation).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

}  // namespace pka
