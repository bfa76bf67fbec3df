// C ABI of libpka: validation, the ForwardMode dispatch and kernel launches.
//
// Every entry point checks what the host can see before anything is
// enqueued and returns a pka_status; on error nothing is launched, after the
// pages' rule that a backend refuses to start on what it cannot run
// ("sglang-101 s4.2 --attention-backend", section "The obvious fix, and why it
// fails").  The library holds no device memory: buffers come from the caller.
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>

#include "pka_internal.h"

struct pka_ctx {
    pka_config cfg;
    int32_t dk;          // key (and query) head width
    int32_t dv;          // value (and output) head width
    int32_t G;
    int32_t qgroups;     // ceil(G / 16): decode waves per KV head
    int32_t page_shift;
    int32_t wpb;         // decode waves per share (KV-head units of one share in a workgroup)
    int32_t ext_tq;      // extend query tokens per work item
    int32_t max_q;       // most query rows per request on the decode path (1 .. DEC_MAX_Q)
    std::atomic<int32_t> nwg{0};  // decode shares (from the device's CU count)
    std::atomic<int32_t> spw{0};  // decode shares per workgroup
    std::atomic<int32_t> packed8{0};  // 8-wave decode workgroups resident per CU
    std::atomic<int32_t> md_fits{-1};  // decode with in-kernel metadata keeps the occupancy (-1: unknown)
};

namespace {

thread_local std::string g_last_error;

pka_status fail(pka_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pka_status fail(pka_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

pka_status hip_fail(hipError_t e, const char* what) {
    return fail(PKA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t elem_bytes(pka_dtype t) { return t == PKA_F32 ? 4 : t == PKA_BF16 ? 2 : 1; }

// Decode shares: exactly one resident round (every workgroup on the device
// at once, so the equal tile shares finish together), from the device's CU
// count and the kernel's occupancy.  With fewer than 8 waves per share, the
// MFMA kernel packs 8 / wpb shares into one 8-wave workgroup when that keeps
// as many waves resident (the two waves on each SIMD are then balanced
// against each other).  Queried once per context.
int32_t decode_wpb(const pka_ctx* ctx) {
    // the fp32 kernel is built for workgroups of at most 4 waves
    return ctx->cfg.kv_dtype == PKA_F32 ? std::min(ctx->wpb, 4) : ctx->wpb;
}

pka_status decode_wgs(const pka_ctx* ctx, int32_t* out, int32_t* spw_out = nullptr) {
    int32_t v = ctx->nwg.load(std::memory_order_acquire);
    int32_t spw = ctx->spw.load(std::memory_order_relaxed);
    if (v <= 0) {
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "querying the device");
        const pka_dtype kv = ctx->cfg.kv_dtype;
        const int wpb = decode_wpb(ctx);
        int per_cu = pka::decode_blocks_per_cu(kv, ctx->dk, ctx->dv, wpb);  // shares per CU
        spw = 1;
        if (kv != PKA_F32 && wpb < 8) {
            const int packed = pka::decode_blocks_per_cu(kv, ctx->dk, ctx->dv, 8);
            if (packed >= 1 && packed * 8 >= per_cu * wpb) {
                spw = 8 / wpb;
                per_cu = packed * spw;
            }
        }
        if (per_cu < 1) per_cu = 1;
        v = std::min<int32_t>(pka::DEC_MAX_WG, std::max(1, cus * per_cu));
        pka_ctx* c = const_cast<pka_ctx*>(ctx);
        c->packed8.store(kv != PKA_F32 ? pka::decode_blocks_per_cu(kv, ctx->dk, ctx->dv, 8) : 0,
                         std::memory_order_relaxed);
        c->spw.store(spw, std::memory_order_relaxed);
        c->nwg.store(v, std::memory_order_release);
    }
    *out = v;
    if (spw_out) *spw_out = spw;
    return PKA_OK;
}

bool is_extend_like(pka_forward_mode m) {
    return m == PKA_MODE_EXTEND || m == PKA_MODE_TARGET_VERIFY || m == PKA_MODE_DRAFT_EXTEND;
}

// Decode partial slots per (request, workgroup): a decode batch has one query
// row per request; an extend-like batch sent down the decode path
// (speculative verify) may carry up to ctx->max_q rows per request.
int32_t decode_qslots(const pka_ctx* ctx, pka_forward_mode m, int32_t num_q_tokens) {
    if (m == PKA_MODE_DECODE) return 1;
    return std::max(1, std::min<int32_t>(ctx->max_q, num_q_tokens));
}

// 16-column passes a verify batch's query columns (tokens x heads of a
// group) need on the decode path, from the average tokens per request; 1
// for a decode batch or an fp32 cache.
int32_t decode_passes(const pka_ctx* ctx, const pka_batch* md) {
    if (ctx->cfg.kv_dtype == PKA_F32 || md->batch <= 0) return 1;
    const int32_t qslots = decode_qslots(ctx, md->mode, md->num_q_tokens);
    if (qslots <= 1) return 1;
    const int32_t nq = std::min<int32_t>(qslots, (md->num_q_tokens + md->batch - 1) / md->batch);
    return std::max<int32_t>(1, (nq * std::min<int32_t>(ctx->G, 16) + 15) / 16);
}

// Column blocks of 16 per decode wave: with several passes each wave takes
// two adjacent blocks, so one tile stream serves 32 columns (keys of at most
// 128; the 192-wide kernel has no registers left for a second block).
int32_t decode_cb(const pka_ctx* ctx, const pka_batch* md) {
    return ctx->dk <= 128 && decode_passes(ctx, md) >= 2 ? 2 : 1;
}

// Waves per head group on the decode path.  Passes beyond a wave's column
// blocks go to up to DEC_MAX_CSPLIT waves of one workgroup that read the
// same tiles side by side, instead of one wave reading them once per pass.
// The split follows the average tokens per request; a request with fewer
// leaves the surplus waves idle over its tiles.
int32_t decode_csplit(const pka_ctx* ctx, const pka_batch* md) {
    const int32_t cb = decode_cb(ctx, md);
    return std::min<int32_t>((decode_passes(ctx, md) + cb - 1) / cb, pka::DEC_MAX_CSPLIT);
}

// Launch shape of a decode call with column split cs: waves per share in a
// workgroup (wpb) and shares per workgroup (spw).  A share then needs cs
// times the waves, so the partition is cut into nwg / cs shares
// (batch_shares) and all of them stay resident at once.
void decode_shape(const pka_ctx* ctx, int32_t cs, int32_t base_spw, int* wpb, int* spw) {
    if (cs <= 1) {
        *wpb = decode_wpb(ctx);
        *spw = base_spw;
        return;
    }
    const int units = ctx->cfg.num_kv_heads * ctx->qgroups * cs;
    int w = 8;
    while (units % w) w >>= 1;
    *wpb = w;
    *spw = w < 8 && ctx->packed8.load(std::memory_order_relaxed) >= 1 ? 8 / w : 1;
}

// Decode shares of a batch's partition (one resident round of the launch that
// will serve it) and, for the plain launch shape, shares per workgroup.  The
// metadata and the decode call derive it from the same batch sizes.
pka_status batch_shares(const pka_ctx* ctx, const pka_batch* md, int32_t* nwg, int32_t* spw = nullptr) {
    pka_status s = decode_wgs(ctx, nwg, spw);
    if (s == PKA_OK) *nwg = std::max<int32_t>(1, *nwg / decode_csplit(ctx, md));
    return s;
}

// Key-range chunks per extend item.  A batch of few query rows per request
// (at most 16 on average: speculative verify, short continuations) has about
// one item per request and KV head; when those are too few to fill the chip,
// a long request's item would stream its keys alone while most workgroup
// slots idle.  Its key range is then cut into chunks whose partials a merge
// kernel combines: enough chunks for about EXT_SPLIT_WGS workgroups (two
// rounds of two resident extend workgroups on each of 256 CUs), at most
// EXT_MAX_SPLIT, and none below three (two chunks of a batch that nearly
// fills the chip cost more in partials than they balance).  A function of
// the batch sizes only, so the workspace and the launch agree.  bf16
// queries (the MFMA kernel) only.
constexpr int64_t EXT_SPLIT_WGS = 1024;
int32_t ext_split(const pka_ctx* ctx, int32_t batch, int32_t num_q_tokens) {
    if (ctx->cfg.q_dtype != PKA_BF16 || batch <= 0 || num_q_tokens <= 0) return 1;
    if ((int64_t)num_q_tokens > 16LL * batch) return 1;
    const int64_t c = EXT_SPLIT_WGS / ((int64_t)batch * ctx->cfg.num_kv_heads);
    return c < 3 ? 1 : (int32_t)std::min<int64_t>(c, pka::EXT_MAX_SPLIT);
}
// Workspace of a split extend call: a bf16 partial row and an fp32 lse per
// (query row, head, chunk).
int64_t ext_ws_bytes(const pka_ctx* ctx, int32_t num_q_tokens, int32_t C) {
    return C > 1 ? (int64_t)num_q_tokens * ctx->cfg.num_q_heads * C * ((int64_t)ctx->dv * 2 + 4) : 0;
}

// Workspace of a decode call: a partial row in the output's type (bf16 or
// fp32, that of the queries) and an fp32 lse per (request or share, query
// slot, head).
int64_t decode_ws_bytes(const pka_ctx* ctx, int32_t B, int32_t nwg, int32_t qslots) {
    const int64_t row = (int64_t)ctx->dv * elem_bytes(ctx->cfg.q_dtype) + 4;
    return ((int64_t)B + nwg) * qslots * ctx->cfg.num_q_heads * row;
}

pka_status check_batch(const pka_ctx* ctx, const pka_batch* md) {
    if (!ctx || !md) return fail(PKA_ERR_INVALID_ARG, "null context or batch");
    if (md->batch < 0 || md->num_q_tokens < 0 || md->max_kv_pages < 0)
        return fail(PKA_ERR_INVALID_ARG, "negative batch sizes");
    if (md->mode < PKA_MODE_EXTEND || md->mode > PKA_MODE_DRAFT_EXTEND)
        return fail(PKA_ERR_INVALID_ARG, "unknown forward mode %d", (int)md->mode);
    if (md->mode == PKA_MODE_DECODE && md->num_q_tokens != md->batch)
        return fail(PKA_ERR_INVALID_ARG, "decode batch needs num_q_tokens == batch (%d vs %d)",
                    md->num_q_tokens, md->batch);
    if (md->batch > 0 && (!md->kv_indptr || !md->kv_indices || !md->kv_last_page_len ||
                          !md->qo_indptr || !md->plan))
        return fail(PKA_ERR_INVALID_ARG, "null metadata array");
    if (md->batch > 0 && md->max_kv_pages < 1)
        return fail(PKA_ERR_INVALID_ARG, "max_kv_pages must be positive");
    if (md->num_q_tokens > 0 && !md->out_cache_loc)
        return fail(PKA_ERR_INVALID_ARG, "null out_cache_loc");
    return PKA_OK;
}

pka::AttnArgs attn_args(const pka_ctx* ctx, const pka_batch* md, const void* q, const void* kp,
                        const void* vp, void* out, float* lse) {
    pka::AttnArgs a{};
    const pka_config& c = ctx->cfg;
    a.q = q;
    a.k_pool = kp;
    a.v_pool = vp;
    a.out = out;
    a.lse = lse;
    a.kv_indptr = md->kv_indptr;
    a.kv_indices = md->kv_indices;
    a.kv_last_page_len = md->kv_last_page_len;
    a.qo_indptr = md->qo_indptr;
    a.plan = md->plan;
    a.kv_cap = md->max_kv_pages;
    a.B = md->batch;
    a.N = md->num_q_tokens;
    a.Hq = c.num_q_heads;
    a.Hkv = c.num_kv_heads;
    a.G = ctx->G;
    a.qgroups = ctx->qgroups;
    a.page_shift = ctx->page_shift;
    a.num_pages = c.num_pages;
    a.pool_slots = (int64_t)c.num_pages * c.page_size;
    a.spw = 1;
    a.csplit = 1;
    a.cb = 1;
    a.ext_split = 1;
    const float k_scale = c.kv_dtype == PKA_FP8_E4M3FN ? c.k_scale : 1.0f;
    a.scale_log2 = c.scale * 1.4426950408889634f * k_scale;
    a.v_scale = c.kv_dtype == PKA_FP8_E4M3FN ? c.v_scale : 1.0f;
    return a;
}

pka_status check_attn(const pka_ctx* ctx, const pka_batch* md, const void* q, const void* kp,
                      const void* vp, void* out) {
    pka_status s = check_batch(ctx, md);
    if (s != PKA_OK) return s;
    if (md->num_q_tokens > 0 && (!q || !kp || !vp || !out))
        return fail(PKA_ERR_INVALID_ARG, "null q, pool or output pointer");
    if (!aligned16(q) || !aligned16(kp) || !aligned16(vp) || !aligned16(out))
        return fail(PKA_ERR_INVALID_ARG, "q, pools and output must be 16-byte aligned");
    return PKA_OK;
}


// Validated arguments of a decode launch (nothing is enqueued); with
// write_new the new tokens k_new / v_new are written by the decode kernel
// itself (bf16 and fp8 caches).  The caller skips idle and empty batches.
pka_status decode_args(const pka_ctx* ctx, const pka_batch* md, const void* q, const void* k_pool,
                       const void* v_pool, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, bool write_new, const void* k_new, const void* v_new,
                       pka::AttnArgs* args, int* wpb_out) {
    pka_status s = check_attn(ctx, md, q, k_pool, v_pool, out);
    if (s != PKA_OK) return s;
    if (write_new && (!k_new || !v_new)) return fail(PKA_ERR_INVALID_ARG, "null K/V pointer");
    if (write_new && (!aligned16(k_new) || !aligned16(v_new)))
        return fail(PKA_ERR_INVALID_ARG, "K/V rows must be 16-byte aligned");
    const int32_t qslots = decode_qslots(ctx, md->mode, md->num_q_tokens);
    if (write_new && qslots != 1)
        return fail(PKA_ERR_INVALID_ARG, "the fused cache write serves decode batches only");
    if (qslots > 1 && (int64_t)md->num_q_tokens > (int64_t)qslots * md->batch)
        return fail(PKA_ERR_UNSUPPORTED,
                    "verify batch of %d query tokens over %d requests: the decode path takes at most %d "
                    "per request (max_q_per_request / 16)", md->num_q_tokens, md->batch, qslots);
    int32_t nwg = 0, spw = 1;
    if ((s = batch_shares(ctx, md, &nwg, &spw)) != PKA_OK) return s;
    const int64_t need = decode_ws_bytes(ctx, md->batch, nwg, qslots);
    if (!workspace || (int64_t)workspace_bytes < need || !aligned16(workspace))
        return fail(PKA_ERR_WORKSPACE, "decode needs %lld workspace bytes (16-byte aligned), got %zu",
                    (long long)need, workspace_bytes);
    pka::AttnArgs a = attn_args(ctx, md, q, k_pool, v_pool, out, lse);
    int wpb = 1, sp = 1;
    a.csplit = decode_csplit(ctx, md);  // 1 unless several query rows per request
    a.cb = decode_cb(ctx, md);
    decode_shape(ctx, a.csplit, spw, &wpb, &sp);
    a.nwg = nwg;
    a.spw = sp;
    a.qslots = qslots;
    a.ws_o = workspace;
    a.ws_lse = (float*)((uint8_t*)workspace + ((int64_t)md->batch + nwg) * qslots * ctx->cfg.num_q_heads *
                                                  ctx->dv * (int64_t)elem_bytes(ctx->cfg.q_dtype));
    if (write_new) {
        const pka_config& c = ctx->cfg;
        a.k_new = k_new;
        a.v_new = v_new;
        a.out_cache_loc = md->out_cache_loc;
        a.pool_slots = (int64_t)c.num_pages * c.page_size;
        a.k_inv = 1.0f / (c.kv_dtype == PKA_FP8_E4M3FN ? c.k_scale : 1.0f);
        a.v_inv = 1.0f / (c.kv_dtype == PKA_FP8_E4M3FN ? c.v_scale : 1.0f);
    }
    *args = a;
    *wpb_out = wpb;
    return PKA_OK;
}

pka_status decode_call(const pka_ctx* ctx, const pka_batch* md, const void* q, const void* k_pool,
                       const void* v_pool, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream, bool write_new, const void* k_new,
                       const void* v_new) {
    pka_status s = check_attn(ctx, md, q, k_pool, v_pool, out);
    if (s != PKA_OK) return s;
    if (md->mode == PKA_MODE_IDLE || md->batch == 0) return PKA_OK;
    pka::AttnArgs a;
    int wpb = 1;
    if ((s = decode_args(ctx, md, q, k_pool, v_pool, out, lse, workspace, workspace_bytes, write_new,
                         k_new, v_new, &a, &wpb)) != PKA_OK)
        return s;
    hipError_t e = pka::launch_decode(ctx->cfg.q_dtype, ctx->cfg.kv_dtype, ctx->dk, ctx->dv, a, wpb,
                                      (hipStream_t)stream);
    return e == hipSuccess ? PKA_OK : hip_fail(e, "decode launch");
}

// Validated metadata arguments (nothing is enqueued); the caller skips idle
// and empty batches.
pka_status meta_args(const pka_ctx* ctx, const int32_t* seq_lens, const int32_t* extend_lens,
                     const int32_t* page_table, int32_t page_table_stride, int32_t page_table_cols,
                     const pka_batch* md, pka::MetaArgs* out) {
    pka_status s = check_batch(ctx, md);
    if (s != PKA_OK) return s;
    if (!seq_lens || !page_table) return fail(PKA_ERR_INVALID_ARG, "null seq_lens or page_table");
    if (md->mode != PKA_MODE_DECODE && !extend_lens)
        return fail(PKA_ERR_INVALID_ARG, "extend-like batches need extend_lens");
    if (page_table_cols < 1 || page_table_stride < page_table_cols)
        return fail(PKA_ERR_INVALID_ARG, "page table stride %d / cols %d", page_table_stride, page_table_cols);
    pka::MetaArgs a{};
    a.seq_lens = seq_lens;
    a.extend_lens = md->mode == PKA_MODE_DECODE ? nullptr : extend_lens;
    a.page_table = page_table;
    a.pt_stride = page_table_stride;
    a.pt_cols = page_table_cols;
    a.B = md->batch;
    a.N = md->num_q_tokens;
    a.max_kv_pages = md->max_kv_pages;
    a.page_shift = ctx->page_shift;
    a.num_pages = ctx->cfg.num_pages;
    int32_t nwg = 0;
    if ((s = batch_shares(ctx, md, &nwg)) != PKA_OK) return s;
    a.nwg = nwg;
    a.ext_tq = ctx->ext_tq;
    a.is_decode = md->mode == PKA_MODE_DECODE;
    a.fuse_gather = md->batch <= pka::FUSE_MAX_B && md->max_kv_pages <= pka::FUSE_MAX_ITEMS &&
                    md->num_q_tokens <= pka::FUSE_MAX_ITEMS;
    a.kv_indptr = md->kv_indptr;
    a.kv_indices = md->kv_indices;
    a.kv_last_page_len = md->kv_last_page_len;
    a.qo_indptr = md->qo_indptr;
    a.out_cache_loc = md->out_cache_loc;
    a.plan = md->plan;
    *out = a;
    return PKA_OK;
}

// Checks of pka_forward that need no launch: modes, buffers, the metadata's
// mode, the decode workspace and the new K/V rows.  Sets *path.
pka_status forward_checks(const pka_ctx* ctx, pka_forward_mode mode, pka_spec_attn_mode spec_mode,
                          const pka_batch* md, const void* q, const void* k_new, const void* v_new,
                          int save_kv, void* k_pool, void* v_pool, void* out, void* workspace,
                          size_t workspace_bytes, pka_path* path) {
    if (mode < PKA_MODE_EXTEND || mode > PKA_MODE_DRAFT_EXTEND)
        return fail(PKA_ERR_INVALID_ARG, "unknown forward mode %d", (int)mode);
    if (spec_mode != PKA_SPEC_PREFILL && spec_mode != PKA_SPEC_DECODE)
        return fail(PKA_ERR_INVALID_ARG, "unknown speculative attention mode %d", (int)spec_mode);
    *path = pka_select_path(mode, spec_mode);
    if (*path == PKA_PATH_NONE) return PKA_OK;
    pka_status s = check_attn(ctx, md, q, k_pool, v_pool, out);
    if (s != PKA_OK) return s;
    if (md->mode != mode)
        return fail(PKA_ERR_INVALID_ARG, "metadata was built for mode %d, forward called with %d",
                    (int)md->mode, (int)mode);
    if (*path == PKA_PATH_DECODE) {
        int32_t nwg = 0;
        if ((s = batch_shares(ctx, md, &nwg)) != PKA_OK) return s;
        if (!workspace ||
            (int64_t)workspace_bytes < decode_ws_bytes(ctx, md->batch, nwg, decode_qslots(ctx, md->mode, md->num_q_tokens)))
            return fail(PKA_ERR_WORKSPACE, "decode workspace too small");
    }
    if (save_kv && md->num_q_tokens > 0) {
        if (!k_new || !v_new) return fail(PKA_ERR_INVALID_ARG, "null K/V pointer");
        if (!aligned16(k_new) || !aligned16(v_new))
            return fail(PKA_ERR_INVALID_ARG, "K/V rows must be 16-byte aligned");
    }
    return PKA_OK;
}

// Whether a decode batch can build its metadata inside the decode kernel:
// bf16 / fp8 cache, at most DEC_MD_MAX_B requests, and the kernel keeps the
// plain decode kernel's occupancy (the partition assumes one resident round).
bool decode_md_ok(const pka_ctx* ctx, const pka_batch* md) {
    if (ctx->cfg.kv_dtype == PKA_F32 || md->mode != PKA_MODE_DECODE || md->batch > pka::DEC_MD_MAX_B)
        return false;
    int32_t v = ctx->md_fits.load(std::memory_order_acquire);
    if (v < 0) {
        int32_t nwg = 0, spw = 1;
        if (decode_wgs(ctx, &nwg, &spw) != PKA_OK) return false;
        v = pka::decode_md_fits(ctx->cfg.kv_dtype, ctx->dk, ctx->dv, decode_wpb(ctx) * spw) ? 1 : 0;
        const_cast<pka_ctx*>(ctx)->md_fits.store(v, std::memory_order_release);
    }
    return v == 1;
}

const char* dtype_name(pka_dtype t) { return t == PKA_F32 ? "f32" : t == PKA_BF16 ? "bf16" : "fp8 e4m3fn"; }

}  // namespace

namespace pka {

pka_status set_error(pka_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

pka_status forward_workspace_need(const pka_ctx* ctx, pka_forward_mode mode, pka_spec_attn_mode spec_mode,
                                  const pka_batch* md, int64_t* need) {
    *need = 0;
    if (mode < PKA_MODE_EXTEND || mode > PKA_MODE_DRAFT_EXTEND)
        return fail(PKA_ERR_INVALID_ARG, "unknown forward mode %d", (int)mode);
    if (spec_mode != PKA_SPEC_PREFILL && spec_mode != PKA_SPEC_DECODE)
        return fail(PKA_ERR_INVALID_ARG, "unknown speculative attention mode %d", (int)spec_mode);
    if (pka_select_path(mode, spec_mode) != PKA_PATH_DECODE) return PKA_OK;
    pka_status s = check_batch(ctx, md);
    if (s != PKA_OK || md->batch == 0) return s;
    int32_t nwg = 0;
    if ((s = batch_shares(ctx, md, &nwg)) != PKA_OK) return s;
    *need = decode_ws_bytes(ctx, md->batch, nwg, decode_qslots(ctx, md->mode, md->num_q_tokens));
    return PKA_OK;
}

}  // namespace pka

extern "C" {

pka_status pka_describe(const pka_ctx* ctx, pka_forward_mode mode, pka_spec_attn_mode spec_mode,
                        int32_t batch, int32_t num_q_tokens, int with_metadata, char* buf, size_t len) {
    if (!ctx || !buf || len == 0) return fail(PKA_ERR_INVALID_ARG, "null context or buffer");
    if (mode < PKA_MODE_EXTEND || mode > PKA_MODE_DRAFT_EXTEND)
        return fail(PKA_ERR_INVALID_ARG, "unknown forward mode %d", (int)mode);
    if (spec_mode != PKA_SPEC_PREFILL && spec_mode != PKA_SPEC_DECODE)
        return fail(PKA_ERR_INVALID_ARG, "unknown speculative attention mode %d", (int)spec_mode);
    if (batch < 0 || num_q_tokens < 0 || (mode == PKA_MODE_DECODE && num_q_tokens != batch))
        return fail(PKA_ERR_INVALID_ARG, "batch %d / num_q_tokens %d", batch, num_q_tokens);
    const pka_config& c = ctx->cfg;
    const pka_path path = pka_select_path(mode, spec_mode);
    pka_batch md{};
    md.mode = mode;
    md.batch = batch;
    md.num_q_tokens = num_q_tokens;
    std::string d;
    char tmp[512];
    if (path == PKA_PATH_NONE) {
        d = "path none (idle batch: nothing is launched)";
    } else if (path == PKA_PATH_DECODE) {
        int32_t nwg = 0, base_spw = 1;
        pka_status s = batch_shares(ctx, &md, &nwg, &base_spw);
        if (s != PKA_OK) return s;
        const int32_t cs = decode_csplit(ctx, &md), cb = decode_cb(ctx, &md);
        int wpb = 1, spw = 1;
        decode_shape(ctx, cs, base_spw, &wpb, &spw);
        const int32_t qslots = decode_qslots(ctx, mode, num_q_tokens);
        const bool md_in = with_metadata && decode_md_ok(ctx, &md);
        const char* kern = c.kv_dtype == PKA_F32 ? "decode_f32_kernel" : "decode_mfma_kernel";
        snprintf(tmp, sizeof tmp,
                 "path decode: %s<Dk %d, Dv %d, %s cache%s%s>, page size %d, %d query heads per KV head "
                 "(%d head group(s) of <= 16), %d shares (one resident round), %d wave(s) per share, "
                 "%d share(s) per workgroup, %d workgroups, %d column block(s) of 16 per wave, column split %d, "
                 "%d partial row(s) per share; "
                 "then decode_merge_kernel<Dv %d>%s",
                 kern, ctx->dk, ctx->dv, dtype_name(c.kv_dtype), qslots > 1 ? ", several query rows" : "",
                 md_in ? ", metadata built in-kernel" : "", c.page_size, ctx->G, ctx->qgroups, nwg, wpb, spw,
                 (nwg + spw - 1) / spw, cb, cs, qslots, ctx->dv,
                 with_metadata && !md_in ? "; metadata by md_scan_kernel first" : "");
        d = tmp;
    } else {
        if (c.q_dtype == PKA_F32) {
            snprintf(tmp, sizeof tmp, "path extend: extend_f32_kernel<Dk %d, Dv %d>, %d query tokens per item",
                     ctx->dk, ctx->dv, ctx->ext_tq);
        } else {
            const bool big = c.page_size >= 64;
            const int64_t row = (int64_t)c.num_kv_heads * std::max(ctx->dk, ctx->dv) * (int64_t)elem_bytes(c.kv_dtype);
            const bool wide = !big && (int64_t)c.num_pages * c.page_size * row > (int64_t)UINT32_MAX;
            const int32_t C = ext_split(ctx, batch, num_q_tokens);
            char split[160] = "";
            if (C > 1)
                snprintf(split, sizeof split,
                         ", key range cut into %d chunks per item (with a workspace of pka_batch_sizes' size), "
                         "then extend_split_merge_kernel<Dv %d>", C, ctx->dv);
            snprintf(tmp, sizeof tmp,
                     "path extend: extend_mfma_kernel<Dk %d, Dv %d, scale %s 0, %s, %s cache>, %d query tokens "
                     "x %d heads per workgroup item, 64-key tiles%s",
                     ctx->dk, ctx->dv, c.scale > 0.f ? ">" : "<=",
                     big ? "one page per key tile" : (wide ? "per-row slots, 64-bit addresses" : "per-row slots"),
                     dtype_name(c.kv_dtype), ctx->ext_tq, ctx->G, split);
        }
        d = tmp;
        if (with_metadata) d = "md_scan_kernel, then " + d;
    }
    if (d.size() + 1 > len) return fail(PKA_ERR_INVALID_ARG, "description needs %zu bytes", d.size() + 1);
    memcpy(buf, d.c_str(), d.size() + 1);
    return PKA_OK;
}

const char* pka_status_string(pka_status s) {
    switch (s) {
    case PKA_OK: return "ok";
    case PKA_ERR_INVALID_ARG: return "invalid argument";
    case PKA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKA_ERR_WORKSPACE: return "workspace too small";
    case PKA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* pka_last_error(void) { return g_last_error.c_str(); }

const char* pka_version(void) { return "pka 0.1 gfx950"; }

pka_status pka_create(const pka_config* cfg, pka_ctx** out) {
    if (!cfg || !out) return fail(PKA_ERR_INVALID_ARG, "null config or output handle");
    *out = nullptr;
    const pka_config& c = *cfg;
    if (c.num_q_heads < 1 || c.num_kv_heads < 1 || c.num_q_heads % c.num_kv_heads != 0)
        return fail(PKA_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                    c.num_q_heads, c.num_kv_heads);
    const int32_t dv = c.v_head_dim == 0 ? c.head_dim : c.v_head_dim;
    const bool widths_ok = (c.head_dim == 64 && dv == 64) || (c.head_dim == 128 && dv == 128) ||
                           (c.head_dim == 192 && dv == 128);
    if (!widths_ok)
        return fail(PKA_ERR_UNSUPPORTED, "head widths K %d / V %d (supported: 64/64, 128/128, 192/128)",
                    c.head_dim, dv);
    if (c.page_size < 1 || c.page_size > 256 || (c.page_size & (c.page_size - 1)))
        return fail(PKA_ERR_UNSUPPORTED, "page_size %d (supported: powers of two up to 256)", c.page_size);
    if (c.num_pages < 1 || (int64_t)c.num_pages * c.page_size > INT32_MAX)
        return fail(PKA_ERR_INVALID_ARG, "num_pages %d: pool slots must fit in int32", c.num_pages);
    const bool pair_ok = (c.q_dtype == PKA_F32 && c.kv_dtype == PKA_F32) ||
                         (c.q_dtype == PKA_BF16 && c.kv_dtype == PKA_BF16) ||
                         (c.q_dtype == PKA_BF16 && c.kv_dtype == PKA_FP8_E4M3FN);
    if (!pair_ok)
        return fail(PKA_ERR_UNSUPPORTED, "dtype pair q=%d kv=%d (supported: f32/f32, bf16/bf16, bf16/fp8)",
                    (int)c.q_dtype, (int)c.kv_dtype);
    if (!std::isfinite(c.scale)) return fail(PKA_ERR_INVALID_ARG, "scale must be finite");
    if (c.kv_dtype == PKA_FP8_E4M3FN) {
        if (!(c.k_scale > 0.f) || !(c.v_scale > 0.f) || !std::isfinite(c.k_scale) ||
            !std::isfinite(c.v_scale) || !std::isfinite(1.0f / c.k_scale) || !std::isfinite(1.0f / c.v_scale))
            return fail(PKA_ERR_INVALID_ARG, "fp8 k_scale / v_scale must be positive and finite");
    } else if (c.k_scale != 1.f || c.v_scale != 1.f) {
        return fail(PKA_ERR_INVALID_ARG, "k_scale / v_scale apply to fp8 caches only (must be 1)");
    }
    if (c.max_q_per_request < 0)
        return fail(PKA_ERR_INVALID_ARG, "max_q_per_request must be >= 0 (0: 16)");
    const int G = c.num_q_heads / c.num_kv_heads;
    if (G > pka::extend_max_group(c.q_dtype, c.page_size))
        return fail(PKA_ERR_UNSUPPORTED, "%d query heads per KV head (extend supports up to %d at page size %d)",
                    G, pka::extend_max_group(c.q_dtype, c.page_size), c.page_size);
    pka_ctx* ctx = new (std::nothrow) pka_ctx;
    if (!ctx) return fail(PKA_ERR_INVALID_ARG, "out of host memory");
    ctx->cfg = c;
    ctx->cfg.v_head_dim = dv;
    ctx->dk = c.head_dim;
    ctx->dv = dv;
    ctx->G = c.num_q_heads / c.num_kv_heads;
    ctx->qgroups = (ctx->G + 15) / 16;
    int shift = 0;
    while ((1 << shift) < c.page_size) ++shift;
    ctx->page_shift = shift;
    const int units = c.num_kv_heads * ctx->qgroups;
    int wpb = 8;
    while (units % wpb) wpb >>= 1;
    ctx->wpb = wpb;
    ctx->ext_tq = pka::extend_tq(c.q_dtype, c.kv_dtype, ctx->G, c.page_size);
    ctx->max_q = c.max_q_per_request == 0 ? pka::DEC_MAX_Q : std::min<int32_t>(c.max_q_per_request, pka::DEC_MAX_Q);
    *out = ctx;
    return PKA_OK;
}

void pka_destroy(pka_ctx* ctx) { delete ctx; }

pka_status pka_batch_sizes(const pka_ctx* ctx, pka_forward_mode mode, int32_t batch,
                           int32_t num_q_tokens, int64_t max_kv_pages, pka_sizes* out) {
    if (!ctx || !out) return fail(PKA_ERR_INVALID_ARG, "null context or output");
    if (batch < 0 || num_q_tokens < 0 || max_kv_pages < 0)
        return fail(PKA_ERR_INVALID_ARG, "negative sizes");
    if (mode < PKA_MODE_EXTEND || mode > PKA_MODE_DRAFT_EXTEND)
        return fail(PKA_ERR_INVALID_ARG, "unknown forward mode %d", (int)mode);
    if (mode == PKA_MODE_DECODE && num_q_tokens != batch)
        return fail(PKA_ERR_INVALID_ARG, "decode batch needs num_q_tokens == batch");
    out->kv_indptr = (int64_t)batch + 1;
    out->kv_indices = std::max<int64_t>(max_kv_pages, 1);
    out->kv_last_page_len = std::max<int32_t>(batch, 1);
    out->qo_indptr = (int64_t)batch + 1;
    out->out_cache_loc = std::max<int32_t>(num_q_tokens, 1);
    out->plan = pka::plan_elems(batch, num_q_tokens, ctx->ext_tq);
    // split partials.  Decode path (a verify batch may be routed to it by
    // the speculative-attention dispatch): one resident round of the
    // device's decode launch (without a column split: the most shares any
    // batch of this mode can use), else the library's bound when no device
    // answers.  Extend path: the key-range chunks of a batch of few rows per
    // request.
    out->workspace_bytes = 0;
    if (mode != PKA_MODE_EXTEND && mode != PKA_MODE_IDLE) {
        int32_t nwg = 0;
        if (decode_wgs(ctx, &nwg) != PKA_OK) nwg = pka::DEC_MAX_WG;
        out->workspace_bytes = decode_ws_bytes(ctx, batch, nwg, decode_qslots(ctx, mode, num_q_tokens));
    }
    if (mode != PKA_MODE_DECODE && mode != PKA_MODE_IDLE)
        out->workspace_bytes = std::max<int64_t>(
            out->workspace_bytes, ext_ws_bytes(ctx, num_q_tokens, ext_split(ctx, batch, num_q_tokens)));
    return PKA_OK;
}

pka_status pka_init_metadata(const pka_ctx* ctx, const int32_t* seq_lens,
                             const int32_t* extend_lens, const int32_t* page_table,
                             int32_t page_table_stride, int32_t page_table_cols, pka_batch* md,
                             void* stream) {
    pka_status s = check_batch(ctx, md);
    if (s != PKA_OK) return s;
    if (md->mode == PKA_MODE_IDLE || md->batch == 0) return PKA_OK;
    pka::MetaArgs a;
    if ((s = meta_args(ctx, seq_lens, extend_lens, page_table, page_table_stride, page_table_cols, md,
                       &a)) != PKA_OK)
        return s;
    hipError_t e = pka::launch_metadata(a, (hipStream_t)stream);
    return e == hipSuccess ? PKA_OK : hip_fail(e, "metadata launch");
}

pka_status pka_save_kv(const pka_ctx* ctx, const pka_batch* md, const void* k_new,
                       const void* v_new, void* k_pool, void* v_pool, void* stream) {
    pka_status s = check_batch(ctx, md);
    if (s != PKA_OK) return s;
    if (md->mode == PKA_MODE_IDLE || md->num_q_tokens == 0) return PKA_OK;
    if (!k_new || !v_new || !k_pool || !v_pool)
        return fail(PKA_ERR_INVALID_ARG, "null K/V or pool pointer");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return fail(PKA_ERR_INVALID_ARG, "K/V rows and pools must be 16-byte aligned");
    const pka_config& c = ctx->cfg;
    pka::SaveArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.out_cache_loc = md->out_cache_loc;
    a.plan = md->plan;
    a.N = md->num_q_tokens;
    a.k_row_elems = c.num_kv_heads * ctx->dk;
    a.v_row_elems = c.num_kv_heads * ctx->dv;
    a.pool_slots = (int64_t)c.num_pages * c.page_size;
    a.k_inv = 1.0f / (c.kv_dtype == PKA_FP8_E4M3FN ? c.k_scale : 1.0f);
    a.v_inv = 1.0f / (c.kv_dtype == PKA_FP8_E4M3FN ? c.v_scale : 1.0f);
    hipError_t e = pka::launch_save_kv(c.q_dtype, c.kv_dtype, a, (hipStream_t)stream);
    return e == hipSuccess ? PKA_OK : hip_fail(e, "save_kv launch");
}

pka_status pka_attn_decode(const pka_ctx* ctx, const pka_batch* md, const void* q,
                           const void* k_pool, const void* v_pool, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return decode_call(ctx, md, q, k_pool, v_pool, out, lse, workspace, workspace_bytes, stream,
                       false, nullptr, nullptr);
}

pka_status pka_attn_extend(const pka_ctx* ctx, const pka_batch* md, const void* q,
                           const void* k_pool, const void* v_pool, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
    pka_status s = check_attn(ctx, md, q, k_pool, v_pool, out);
    if (s != PKA_OK) return s;
    if (md->mode == PKA_MODE_IDLE || md->batch == 0 || md->num_q_tokens == 0) return PKA_OK;
    if (!is_extend_like(md->mode))
        return fail(PKA_ERR_INVALID_ARG, "metadata was built for a decode batch; extend needs extend metadata");
    pka::AttnArgs a = attn_args(ctx, md, q, k_pool, v_pool, out, lse);
    // a batch of few rows per request splits its key ranges when the
    // workspace holds the partials (else it runs unsplit)
    const int32_t C = ext_split(ctx, md->batch, md->num_q_tokens);
    if (C > 1 && workspace && aligned16(workspace) &&
        (int64_t)workspace_bytes >= ext_ws_bytes(ctx, md->num_q_tokens, C)) {
        a.ext_split = C;
        a.ws_o = workspace;
        a.ws_lse = (float*)((uint8_t*)workspace + (int64_t)md->num_q_tokens * ctx->cfg.num_q_heads * C * ctx->dv * 2);
    }
    hipError_t e = pka::launch_extend(ctx->cfg.q_dtype, ctx->cfg.kv_dtype, ctx->dk, ctx->dv, a,
                                      (hipStream_t)stream);
    return e == hipSuccess ? PKA_OK : hip_fail(e, "extend launch");
}

pka_path pka_select_path(pka_forward_mode mode, pka_spec_attn_mode spec_mode) {
    switch (mode) {
    case PKA_MODE_IDLE: return PKA_PATH_NONE;
    case PKA_MODE_DECODE: return PKA_PATH_DECODE;
    case PKA_MODE_TARGET_VERIFY:
    case PKA_MODE_DRAFT_EXTEND:
        return spec_mode == PKA_SPEC_DECODE ? PKA_PATH_DECODE : PKA_PATH_EXTEND;
    default: return PKA_PATH_EXTEND;
    }
}

pka_status pka_forward(const pka_ctx* ctx, pka_forward_mode mode, pka_spec_attn_mode spec_mode,
                       const pka_batch* md, const void* q, const void* k_new, const void* v_new,
                       int save_kv, void* k_pool, void* v_pool, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
    // everything is checked before anything is enqueued
    pka_path path;
    pka_status s = forward_checks(ctx, mode, spec_mode, md, q, k_new, v_new, save_kv, k_pool, v_pool,
                                  out, workspace, workspace_bytes, &path);
    if (s != PKA_OK || path == PKA_PATH_NONE) return s;
    // bf16 / fp8 decode writes the new tokens inside the decode kernel (one
    // launch less); other paths (and verify batches on the decode path) write
    // them first with the save_kv kernel
    const bool fused = path == PKA_PATH_DECODE && save_kv && ctx->cfg.kv_dtype != PKA_F32 &&
                       md->mode == PKA_MODE_DECODE;
    if (save_kv && !fused && (s = pka_save_kv(ctx, md, k_new, v_new, k_pool, v_pool, stream)) != PKA_OK)
        return s;
    if (fused)
        return decode_call(ctx, md, q, k_pool, v_pool, out, lse, workspace, workspace_bytes, stream,
                           true, k_new, v_new);
    if (path == PKA_PATH_DECODE)
        return pka_attn_decode(ctx, md, q, k_pool, v_pool, out, lse, workspace, workspace_bytes, stream);
    return pka_attn_extend(ctx, md, q, k_pool, v_pool, out, lse, workspace, workspace_bytes, stream);
}

pka_status pka_forward_with_metadata(const pka_ctx* ctx, pka_forward_mode mode,
                                     pka_spec_attn_mode spec_mode, const int32_t* seq_lens,
                                     const int32_t* extend_lens, const int32_t* page_table,
                                     int32_t page_table_stride, int32_t page_table_cols,
                                     pka_batch* md, const void* q, const void* k_new,
                                     const void* v_new, int save_kv, void* k_pool, void* v_pool,
                                     void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    pka_path path;
    pka_status s = forward_checks(ctx, mode, spec_mode, md, q, k_new, v_new, save_kv, k_pool, v_pool,
                                  out, workspace, workspace_bytes, &path);
    if (s != PKA_OK || path == PKA_PATH_NONE) return s;
    if (md->batch == 0) return PKA_OK;
    pka::MetaArgs m;
    if ((s = meta_args(ctx, seq_lens, extend_lens, page_table, page_table_stride, page_table_cols, md,
                       &m)) != PKA_OK)
        return s;
    if (path == PKA_PATH_DECODE && decode_md_ok(ctx, md)) {
        // one decode launch builds the metadata, writes the new tokens and
        // attends; then the merge
        pka::AttnArgs a;
        int wpb = 1;
        if ((s = decode_args(ctx, md, q, k_pool, v_pool, out, lse, workspace, workspace_bytes, save_kv != 0,
                             k_new, v_new, &a, &wpb)) != PKA_OK)
            return s;
        hipError_t e = pka::launch_decode_md(ctx->cfg.q_dtype, ctx->cfg.kv_dtype, ctx->dk, ctx->dv, a, m,
                                             wpb, (hipStream_t)stream);
        return e == hipSuccess ? PKA_OK : hip_fail(e, "decode launch");
    }
    hipError_t e = pka::launch_metadata(m, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "metadata launch");
    return pka_forward(ctx, mode, spec_mode, md, q, k_new, v_new, save_kv, k_pool, v_pool, out, lse,
                       workspace, workspace_bytes, stream);
}

pka_status pka_read_status(const pka_batch* md, int32_t* status, void* stream) {
    if (!md || !status || !md->plan) return fail(PKA_ERR_INVALID_ARG, "null batch or status");
    if (md->batch < 0) return fail(PKA_ERR_INVALID_ARG, "negative batch size");
    int32_t words[pka::PLAN_MDST + pka::MD_SLOTS];
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess) e = hipMemcpy(words, md->plan, sizeof words, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "reading the status words");
    int32_t v = words[pka::PLAN_STATUS];
    for (int i = 0; i < pka::MD_SLOTS; ++i) v |= words[pka::PLAN_MDST + i];
    // the per-share page flags of the partition the plan was last built for
    const int32_t nwg = std::min<int32_t>(std::max<int32_t>(words[pka::PLAN_NWG], 0), pka::DEC_MAX_WG);
    if (nwg > 0 && md->batch > 0) {
        int32_t share[pka::DEC_MAX_WG];
        e = hipMemcpy(share, md->plan + pka::plan_share_flags(md->batch), nwg * sizeof(int32_t),
                      hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "reading the status words");
        for (int i = 0; i < nwg; ++i) v |= share[i];
    }
    *status = v;
    return PKA_OK;
}

}  // extern "C"
