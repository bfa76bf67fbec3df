// save_kv: write the new tokens' K/V rows into the page pools.
//
// The backend's forward runs with save_kv_cache=True, so the new K/V go into
// the cache before attention reads it ("[SGLang] Hybrid Attention", forward
// delegation).  Each thread moves 8 elements of one row; grid.y picks K or V.
// An fp8 e4m3fn cache stores round-to-nearest-even(sat(x * fp32(1/scale))).
#include <algorithm>

#include "fp8.h"
#include "pka_internal.h"

namespace pka {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// SRC_B / DST_B: bytes per element of the source rows and the pool.  K and
// V rows may differ in width; the grid covers the wider one.
template <int SRC_B, int DST_B>
__global__ __launch_bounds__(256) void save_kv_kernel(SaveArgs a) {
    const bool is_v = blockIdx.y == 1;
    const int row_elems = is_v ? a.v_row_elems : a.k_row_elems;
    const int per_row = row_elems / 8;  // 8 elements per thread
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)a.N * per_row) return;
    const int32_t j = (int32_t)(idx / per_row);
    const int32_t e = (int32_t)(idx % per_row) * 8;
    const int32_t slot = a.out_cache_loc[j];
    if (slot < 0 || slot >= a.pool_slots) {
        if (e == 0) atomicOr(a.plan + PLAN_STATUS, PKA_DEV_BAD_PAGE);
        return;
    }
    const uint8_t* src = (const uint8_t*)(is_v ? a.v_new : a.k_new) +
                         ((int64_t)j * row_elems + e) * SRC_B;
    uint8_t* dst = (uint8_t*)(is_v ? a.v_pool : a.k_pool) +
                   ((int64_t)slot * row_elems + e) * DST_B;
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

hipError_t launch_save_kv(pka_dtype src, pka_dtype kv, const SaveArgs& a, hipStream_t s) {
    const int64_t threads = (int64_t)a.N * (std::max(a.k_row_elems, a.v_row_elems) / 8);
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
