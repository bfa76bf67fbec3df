// Internal declarations shared by the libpka translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pka.h"

namespace pka {

// ----------------------------------------------------------------- plan --
// Layout of the int32 `plan` array of a pka_batch.
enum : int32_t {
    PLAN_STATUS = 0,     // sticky PKA_DEV_* flags of save_kv / attention (atomic OR)
    PLAN_SHARE = 1,      // decode: tiles per workgroup (q; the first PLAN_SHARE_REM take q + 1)
    PLAN_TOTAL = 2,      // decode: sum over requests of ceil(L_b / DEC_TILE)
    PLAN_NWG = 3,        // decode: workgroups the partition was made for
    PLAN_EXT_COUNT = 4,  // extend: number of (request, query tile) items
    PLAN_EXT_TQ = 5,     // extend: query tokens per item
    PLAN_SHARE_REM = 6,  // decode: workgroups whose share is one tile longer
    PLAN_MDST = 16,      // PKA_DEV_* flags of each metadata workgroup (MD_SLOTS words)
    PLAN_HDR = 80,
};
constexpr int MD_SLOTS = 64;  // most metadata workgroups per launch

// Batches up to this size (and page plus new-token counts up to
// FUSE_MAX_ITEMS) build all metadata in one launch: every workgroup scans
// the batch itself and gathers its slice of kv_indices / out_cache_loc.
constexpr int FUSE_MAX_B = 1024;
constexpr int FUSE_PER_THREAD = 4;  // lookups in flight per thread
constexpr int64_t FUSE_MAX_ITEMS = (int64_t)MD_SLOTS * 1024 * FUSE_PER_THREAD;

// Tokens per decode tile (two MFMA row blocks of 16 tokens).
constexpr int DEC_TILE = 32;
// Smallest share of the flattened tile range given to one workgroup (tiles).
// A small batch leaves some workgroups idle rather than give every share a
// tile or two: each share pays a start-up chain of dependent round trips
// (lengths, page ids, first tile) and a partial for the merge.
constexpr int DEC_MIN_SHARE = 4;
// Decode shares: share w is tiles [share_start(w), share_start(w + 1)) of the
// requests' tiles laid end to end, q tiles each and one more for the first r
// shares.
__host__ __device__ inline int64_t share_start(int64_t w, int64_t q, int64_t r) {
    return w * q + (w < r ? w : r);
}
// the share that holds tile t
__host__ __device__ inline int64_t share_of(int64_t t, int64_t q, int64_t r) {
    const int64_t big = r * (q + 1);
    return t < big ? t / (q + 1) : r + (t - big) / q;
}
// Upper bound of decode shares (persistent grid).
constexpr int DEC_MAX_WG = 2048;
// Most query tokens per request on the decode path (speculative verify).
constexpr int DEC_MAX_Q = 16;
// Most waves that share one head group's column passes (speculative verify).
constexpr int DEC_MAX_CSPLIT = 4;
// Most key-range chunks per extend item (batches of few query rows per request).
constexpr int EXT_MAX_SPLIT = 8;

// plan offsets that depend on the batch size: the token prefix F[b] = sum of
// L over requests before b, the tile prefix T[b] = sum of ceil(L / DEC_TILE)
// (the decode partition cuts it), the first request of each decode share,
// then one PKA_DEV_* word per decode share (written by the decode kernel that
// builds its own metadata; zeroed by the metadata kernel)
__host__ __device__ inline int64_t plan_seg_prefix(int32_t /*B*/) { return PLAN_HDR; }
__host__ __device__ inline int64_t plan_tile_prefix(int32_t B) { return PLAN_HDR + (int64_t)B + 1; }
__host__ __device__ inline int64_t plan_wg_seg(int32_t B) { return PLAN_HDR + 2 * ((int64_t)B + 1); }
__host__ __device__ inline int64_t plan_share_flags(int32_t B) { return plan_wg_seg(B) + DEC_MAX_WG; }
__host__ __device__ inline int64_t plan_ext_items(int32_t B) {
    return plan_share_flags(B) + DEC_MAX_WG;
}
// extend items (request, query tile of tq tokens): at most ceil(N / tq) + B
__host__ __device__ inline int64_t plan_ext_capacity(int32_t B, int32_t N, int32_t tq) {
    return ((int64_t)N + tq - 1) / tq + B;
}
__host__ __device__ inline int64_t plan_elems(int32_t B, int32_t N, int32_t tq) {
    return plan_ext_items(B) + 2 * plan_ext_capacity(B, N, tq);
}

// Decode batches up to this size may build their metadata inside the decode
// kernel (every workgroup scans the lengths into LDS).
constexpr int DEC_MD_MAX_B = 512;

// Clamp one request's lengths the way every metadata builder does: L >= 1,
// 0 <= n <= L, and no more pages than the page table has columns.  Returns the
// PKA_DEV_* flags of what was clamped; `pages` = ceil(L / page size).
__host__ __device__ inline int32_t md_clamp_request(int64_t& L, int64_t& n, int64_t& pages,
                                                    int32_t page_shift, int32_t pt_cols) {
    int32_t flags = 0;
    if (L < 1) { flags |= PKA_DEV_BAD_LENGTH; L = 1; }
    if (n < 0) { flags |= PKA_DEV_BAD_LENGTH; n = 0; }
    if (n > L) { flags |= PKA_DEV_BAD_LENGTH; n = L; }
    pages = (L + (1 << page_shift) - 1) >> page_shift;
    if (pages > pt_cols) {
        flags |= PKA_DEV_TABLE_SHORT;
        pages = pt_cols;
        L = (int64_t)pt_cols << page_shift;
        if (n > L) n = L;
    }
    return flags;
}

// Decode shares of W tiles over nwg workgroups: q tiles each (at least
// DEC_MIN_SHARE) and one more for the first r.
__host__ __device__ inline void decode_shares(int64_t W, int32_t nwg, int64_t& q, int64_t& r) {
    q = W / nwg;
    r = W % nwg;
    if (q < DEC_MIN_SHARE) {
        q = DEC_MIN_SHARE;
        r = 0;
    }
}

// --------------------------------------------------------------- launch --
struct MetaArgs {
    const int32_t* seq_lens;
    const int32_t* extend_lens;  // null: decode (n_b = 1)
    const int32_t* page_table;
    int64_t pt_stride;
    int32_t pt_cols;
    int32_t B;
    int32_t N;
    int64_t max_kv_pages;
    int32_t page_shift;
    int32_t num_pages;
    int32_t nwg;       // decode shares
    int32_t ext_tq;    // extend query tokens per item
    int32_t is_decode;
    int32_t fuse_gather;  // B <= FUSE_MAX_B: md_scan also writes kv_indices / out_cache_loc
    int32_t* kv_indptr;
    int32_t* kv_indices;
    int32_t* kv_last_page_len;
    int32_t* qo_indptr;
    int32_t* out_cache_loc;
    int32_t* plan;
};

struct SaveArgs {
    const void* k_new;
    const void* v_new;
    void* k_pool;
    void* v_pool;
    const int32_t* out_cache_loc;
    int32_t* plan;
    int32_t N;
    int32_t k_row_elems;  // Hkv * key width
    int32_t v_row_elems;  // Hkv * value width
    int64_t pool_slots;
    float k_inv;  // fp32(1 / k_scale)
    float v_inv;
};

struct AttnArgs {
    const void* q;
    const void* k_pool;
    const void* v_pool;
    void* out;
    float* lse;
    // decode split partials [(B + nwg) * qslots, Hq, value width] in the
    // output's type (bf16 rows with bf16 queries, fp32 with fp32); extend
    // key-range partials [N, Hq, chunks, value width] bf16
    void* ws_o;
    float* ws_lse;  // their log-sum-exps (natural log), one per row
    const int32_t* kv_indptr;
    const int32_t* kv_indices;
    const int32_t* kv_last_page_len;
    const int32_t* qo_indptr;
    const int32_t* plan;
    int64_t kv_cap;  // capacity of kv_indices (reads are clamped below it)
    int32_t B;
    int32_t N;
    int32_t Hq;
    int32_t Hkv;
    int32_t G;
    int32_t qgroups;  // ceil(G / 16): head groups per KV head
    int32_t csplit;   // decode waves per head group (MQ: they take its column passes in turn)
    int32_t cb;       // decode column blocks of 16 per wave and pass (MQ: 1 or 2)
    int32_t ext_split;  // extend: key-range chunks per item (1: none; partials in ws_o / ws_lse)
    int32_t page_shift;
    int32_t num_pages;
    int32_t nwg;       // decode shares (the partition's workgroup count)
    int32_t spw;       // decode shares per workgroup (its waves = spw * units per share)
    float scale_log2;  // scale * log2(e) * k_scale
    float v_scale;
    // decode partial slots per (request, workgroup): 1, or up to DEC_MAX_Q
    // when requests carry several query tokens (their rows are then the
    // request's qo_indptr range and each is causal over the new tokens)
    int32_t qslots;
    // cache write fused into decode (null k_new: none): the new token's K/V
    // row of each request is written by the wave that later reads it
    const void* k_new;
    const void* v_new;
    const int32_t* out_cache_loc;
    int64_t pool_slots;
    float k_inv;  // fp32(1 / k_scale) for an fp8 cache, else 1
    float v_inv;
};

hipError_t launch_metadata(const MetaArgs& a, hipStream_t s);

// Record a failure for pka_last_error() and return s.
pka_status set_error(pka_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Workspace bytes a pka_forward_with_metadata call on this batch uses (0 when
// its path takes none); checks the mode arguments and the batch sizes.
pka_status forward_workspace_need(const pka_ctx* ctx, pka_forward_mode mode, pka_spec_attn_mode spec_mode,
                                  const pka_batch* md, int64_t* need);
// DK: key (and query) head width; DV: value (and output) head width.
hipError_t launch_save_kv(pka_dtype src, pka_dtype kv, const SaveArgs& a, hipStream_t s);
// wpb: waves per share (KV-head units of one share in a workgroup); a
// workgroup holds a.spw shares, 64 * wpb * a.spw threads.
hipError_t launch_decode(pka_dtype q, pka_dtype kv, int DK, int DV, const AttnArgs& a, int wpb,
                         hipStream_t s);
// Decode (one query per request, bf16 / fp8 cache) that builds the batch's
// metadata itself from m.seq_lens and m.page_table, then the merge.
hipError_t launch_decode_md(pka_dtype q, pka_dtype kv, int DK, int DV, const AttnArgs& a,
                            const MetaArgs& m, int wpb, hipStream_t s);
// Whether that kernel keeps the occupancy of the plain decode kernel.
bool decode_md_fits(pka_dtype kv, int DK, int DV, int waves);
hipError_t launch_extend(pka_dtype q, pka_dtype kv, int DK, int DV, const AttnArgs& a, hipStream_t s);

// Decode workgroups of `waves` waves that fit on one compute unit at once.
int decode_blocks_per_cu(pka_dtype kv, int DK, int DV, int waves);

// Query tokens per extend item for a dtype pair.
int extend_tq(pka_dtype q, pka_dtype kv, int G, int page_size);
// largest query-head group (Hq / Hkv) the extend kernels cover
int extend_max_group(pka_dtype q, int page_size);

}  // namespace pka
