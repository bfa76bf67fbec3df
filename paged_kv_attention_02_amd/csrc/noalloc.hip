// pka_forward_with_metadata for callers that cannot allocate device memory.
//
// Code under HIP graph capture, tight serving loops and harnesses that forbid
// hipMalloc cannot hand the decode path a workspace of their own.  This entry
// point gives the decode launch's split partials a file-scope device array
// instead: every GPU the library runs on holds one copy of it, of
// PKA_NOALLOC_SCRATCH_BYTES, until the process ends.  Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address reaches kernels; the array's name in host code is a
// host-side stand-in, not a device address.
//
// The decode kernel writes every partial row the merge reads within the same
// call, so nothing in the array needs clearing between calls.  Calls on one
// GPU share the array: calls that overlap in time on one GPU (different
// streams, or graphs replayed concurrently) race on it.
#include <mutex>

#include "pka_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[PKA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_scratch[MAX_DEVICES];  // device address of `scratch`, per device

// The current device's copy of the array (looked up on its first use there).
pka_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return pka::set_error(PKA_ERR_HIP, "querying the current device: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES)
        return pka::set_error(PKA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return pka::set_error(PKA_ERR_HIP, "device address of the scratch array on device %d: %s", dev,
                                  hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return PKA_OK;
}

}  // namespace

extern "C" pka_status pka_forward_with_metadata_noalloc(
    const pka_ctx* ctx, pka_forward_mode mode, pka_spec_attn_mode spec_mode, const int32_t* seq_lens,
    const int32_t* extend_lens, const int32_t* page_table, int32_t page_table_stride,
    int32_t page_table_cols, pka_batch* md, const void* q, const void* k_new, const void* v_new, int save_kv,
    void* k_pool, void* v_pool, void* out, float* lse, void* stream) {
    int64_t need = 0;
    pka_status s = pka::forward_workspace_need(ctx, mode, spec_mode, md, &need);
    if (s != PKA_OK) return s;
    if (need > (int64_t)PKA_NOALLOC_SCRATCH_BYTES)
        return pka::set_error(PKA_ERR_WORKSPACE,
                              "this batch needs %lld bytes of decode scratch and the no-allocation entry point "
                              "holds %lld (PKA_NOALLOC_SCRATCH_BYTES); pass a workspace to "
                              "pka_forward_with_metadata instead",
                              (long long)need, (long long)PKA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (need > 0) {
        if ((s = scratch_address(&ws)) != PKA_OK) return s;
        ws_bytes = PKA_NOALLOC_SCRATCH_BYTES;
    }
    return pka_forward_with_metadata(ctx, mode, spec_mode, seq_lens, extend_lens, page_table, page_table_stride,
                                     page_table_cols, md, q, k_new, v_new, save_kv, k_pool, v_pool, out, lse, ws,
                                     ws_bytes, stream);
}
