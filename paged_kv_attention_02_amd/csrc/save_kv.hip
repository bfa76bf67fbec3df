// save_kv: write the new tokens' K/V rows into the page pools.
//
// The backend's forward runs with save_kv_cache=True, so the new K/V go into
// the cache before attention reads it ("[SGLang] Hybrid Attention", forward
// delegation).  Each thread moves 8 elements of one row; grid.y picks K or V.
// An fp8 e4m3fn cache stores round-to-nearest-even(sat(x * fp32(1/scale))).
#include "pka_internal.h"

namespace pka {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> e4m3fn code, saturating at +-448, round to nearest even.  Written
// on the bit pattern: the fp32 exponent is rebiased (127 -> 7) and the 23-bit
// mantissa rounded to 3 bits; below 2^-6 the value is a multiple of 2^-9.
__device__ inline uint32_t e4m3fn_from_f32(float y) {
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

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline uint32_t quant4(uint32_t w0, uint32_t w1, float inv) {
    return e4m3fn_from_f32(bf16_lo(w0) * inv) | (e4m3fn_from_f32(bf16_hi(w0) * inv) << 8) |
           (e4m3fn_from_f32(bf16_lo(w1) * inv) << 16) | (e4m3fn_from_f32(bf16_hi(w1) * inv) << 24);
}

// ELEM_SRC / ELEM_DST: bytes per element of the source rows and the pool.
template <int SRC_B, int DST_B>
__global__ __launch_bounds__(256) void save_kv_kernel(SaveArgs a) {
    const int per_row = a.row_elems / 8;  // 8 elements per thread
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)a.N * per_row) return;
    const int32_t j = (int32_t)(idx / per_row);
    const int32_t e = (int32_t)(idx % per_row) * 8;
    const bool is_v = blockIdx.y == 1;
    const int32_t slot = a.out_cache_loc[j];
    if (slot < 0 || slot >= a.pool_slots) {
        if (e == 0) atomicOr(a.plan + PLAN_STATUS, PKA_DEV_BAD_PAGE);
        return;
    }
    const uint8_t* src = (const uint8_t*)(is_v ? a.v_new : a.k_new) +
                         ((int64_t)j * a.row_elems + e) * SRC_B;
    uint8_t* dst = (uint8_t*)(is_v ? a.v_pool : a.k_pool) +
                   ((int64_t)slot * a.row_elems + e) * DST_B;
    if constexpr (SRC_B == DST_B) {
        #pragma unroll
        for (int i = 0; i < SRC_B / 2; ++i)
            ((u32x4_t*)dst)[i] = ((const u32x4_t*)src)[i];
    } else {
        static_assert(SRC_B == 2 && DST_B == 1, "bf16 -> fp8 only");
        const u32x4_t w = *(const u32x4_t*)src;
        const float inv = is_v ? a.v_inv : a.k_inv;
        u32x2_t o;
        o.x = quant4(w.x, w.y, inv);
        o.y = quant4(w.z, w.w, inv);
        *(u32x2_t*)dst = o;
    }
}

}  // namespace

hipError_t launch_save_kv(pka_dtype src, pka_dtype kv, int /*D*/, const SaveArgs& a,
                          hipStream_t s) {
    const int64_t threads = (int64_t)a.N * (a.row_elems / 8);
    if (threads == 0) return hipSuccess;
    const dim3 grid((unsigned)((threads + 255) / 256), 2);
    if (src == PKA_F32 && kv == PKA_F32)
        hipLaunchKernelGGL((save_kv_kernel<4, 4>), grid, dim3(256), 0, s, a);
    else if (src == PKA_BF16 && kv == PKA_BF16)
        hipLaunchKernelGGL((save_kv_kernel<2, 2>), grid, dim3(256), 0, s, a);
    else if (src == PKA_BF16 && kv == PKA_FP8_E4M3FN)
        hipLaunchKernelGGL((save_kv_kernel<2, 1>), grid, dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pka
