/*
 * pka.h -- paged KV attention for one batch on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpka.so.  An attention backend, as the pages define it, builds
 * per-batch metadata (page tables and index buffers), and runs forward_extend
 * for prefill and forward_decode for decode over the paged KV cache of one
 * batch ("sglang-101 s4.2 --attention-backend", section "What an attention
 * backend is").  This library exposes those steps as plain C calls:
 *
 *   pka_init_metadata  seq_lens + page table -> kv_indptr / kv_indices / ...
 *   pka_save_kv        scatter new K/V rows into the page pool
 *   pka_attn_decode    one query token per request (split-K flash decoding;
 *                      up to 16 causal query tokens for speculative verify)
 *   pka_attn_extend    a causal block of new tokens against prefix + itself
 *   pka_forward        ForwardMode-keyed dispatch between the two paths
 *   pka_forward_with_metadata  metadata + forward in one call (one decode
 *                      launch builds both for bf16 / fp8 decode batches)
 *
 * Conventions shared by every call
 * --------------------------------
 * - All device buffers are owned by the caller and passed as plain device
 *   pointers; the library never allocates, frees or synchronises on these
 *   paths.  Work is enqueued on the caller's HIP stream (a hipStream_t passed
 *   as void*; NULL is the default stream).
 * - Layouts are row-major and contiguous:
 *     q                 [num_q_tokens, num_q_heads, head_dim]     (q dtype)
 *     out               [num_q_tokens, num_q_heads, v_head_dim]   (q dtype)
 *     k_new             [num_q_tokens, num_kv_heads, head_dim]    (q dtype)
 *     v_new             [num_q_tokens, num_kv_heads, v_head_dim]  (q dtype)
 *     k_pool            [num_pages * page_size, num_kv_heads, head_dim]
 *     v_pool            [num_pages * page_size, num_kv_heads, v_head_dim]
 *                       (kv dtype; separate K and V pools, token-major)
 *     lse               [num_q_tokens, num_q_heads] fp32, natural log
 *   Page p holds slots p*page_size .. p*page_size + page_size - 1.  Query
 *   head h reads KV head h / (num_q_heads / num_kv_heads).
 * - seq_lens[b] (L_b) counts every token request b attends to, including its
 *   new tokens; the new tokens sit at positions L_b - n_b .. L_b - 1 and new
 *   token i attends to positions 0 .. L_b - n_b + i (bottom-right causal).
 *   Decode has n_b = 1 for every request.
 * - Every call validates its host-visible arguments first and returns a
 *   pka_status; on any error nothing is launched, and pka_last_error()
 *   returns a description (thread-local).  No C++ exception crosses the ABI.
 *   Device-side data (lengths, page ids) is checked by the kernels: out of
 *   range values are clamped so no access leaves its buffer, and a sticky
 *   flag is set that pka_read_status reports.
 */
#ifndef PKA_H
#define PKA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Forward modes of a batch, after the pages' ForwardMode ("[SGLang] Hybrid
 * Attention", section on _select_backend: decode_or_idle, target_verify,
 * draft_extend, and prefill/extend). */
typedef enum {
    PKA_MODE_EXTEND = 0,
    PKA_MODE_DECODE = 1,
    PKA_MODE_IDLE = 2,
    PKA_MODE_TARGET_VERIFY = 3,
    PKA_MODE_DRAFT_EXTEND = 4
} pka_forward_mode;

/* Which path runs the speculative verify pass; the pages give "prefill" as
 * the default ("sglang-101 s4.2", section "Two backends in one server"). */
typedef enum { PKA_SPEC_PREFILL = 0, PKA_SPEC_DECODE = 1 } pka_spec_attn_mode;

typedef enum { PKA_F32 = 0, PKA_BF16 = 1, PKA_FP8_E4M3FN = 2 } pka_dtype;

typedef enum {
    PKA_OK = 0,
    PKA_ERR_INVALID_ARG = -1,
    PKA_ERR_UNSUPPORTED = -2,
    PKA_ERR_WORKSPACE = -3,
    PKA_ERR_HIP = -4
} pka_status;

typedef enum { PKA_PATH_NONE = 0, PKA_PATH_DECODE = 1, PKA_PATH_EXTEND = 2 } pka_path;

/* Per-layer attention parameters (the analogue of one attention layer's
 * handle).  Supported:
 *   (head_dim, v_head_dim) in {(64, 64), (128, 128), (192, 128)}: head_dim
 *   is the width of query and key heads, v_head_dim that of value and output
 *   heads (0 means equal to head_dim).  The pages have one backend picked
 *   for models whose K and V heads differ in width ("sglang-101 s4.2
 *   --attention-backend", backend table and "How SGLang picks a default");
 *   192 / 128 is the query-key width with a rotary part against a narrower
 *   value, as in MLA models run as plain multi-head attention for prefill.
 *   page_size in {1, 2, 4, ..., 256} (a power of two);
 *   num_q_heads a positive multiple of num_kv_heads;
 *   (q, kv) dtypes: (F32, F32), (BF16, BF16), (BF16, FP8_E4M3FN), on both
 *   the decode and the extend path.
 * scale multiplies q.k; k_scale / v_scale are the per-tensor fp8 scales (the
 * cached code c stands for c * scale); they must be 1 for non-fp8 caches.
 * max_q_per_request: the most query tokens one request carries in a
 * target-verify / draft-extend batch sent down the decode path (the
 * server's speculative draft-token count); it sizes the decode workspace's
 * partial rows.  0 means 16, the most the decode path takes per request.
 * v_head_dim and max_q_per_request come last so a zero-initialised tail
 * keeps the equal-width, 16-row behaviour. */
typedef struct {
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t num_pages; /* pool capacity in pages */
    pka_dtype q_dtype;
    pka_dtype kv_dtype;
    float scale;
    float k_scale;
    float v_scale;
    int32_t v_head_dim; /* 0: same as head_dim */
    int32_t max_q_per_request; /* 0: 16 */
} pka_config;

typedef struct pka_ctx pka_ctx;

/* Caller-owned device int32 arrays describing one batch, sized by
 * pka_batch_sizes.  pka_init_metadata fills them; the attention calls read
 * them.  mode records which kind of batch they were built for. */
typedef struct {
    pka_forward_mode mode;
    int32_t batch;            /* B */
    int32_t num_q_tokens;     /* N = sum of n_b (decode: B) */
    int64_t max_kv_pages;     /* capacity of kv_indices */
    int32_t* kv_indptr;       /* [B+1]  page offsets per request */
    int32_t* kv_indices;      /* [max_kv_pages] page ids, request-major */
    int32_t* kv_last_page_len;/* [B]    tokens in each request's last page */
    int32_t* qo_indptr;       /* [B+1]  query-token offsets per request */
    int32_t* out_cache_loc;   /* [N]    pool slot of each new token */
    int32_t* plan;            /* [plan elems] work partition + status word */
} pka_batch;

/* Element counts of the pka_batch arrays and workspace bytes for a batch. */
typedef struct {
    int64_t kv_indptr;
    int64_t kv_indices;
    int64_t kv_last_page_len;
    int64_t qo_indptr;
    int64_t out_cache_loc;
    int64_t plan;
    int64_t workspace_bytes;
} pka_sizes;

/* Validate a configuration and create a host-only context (no device memory,
 * no device calls).  Refuses unsupported combinations with
 * PKA_ERR_UNSUPPORTED, after the pages' rule that a backend refuses to start
 * on what it cannot run ("sglang-101 s4.2", section "The obvious fix, and why
 * it fails").  *out must be released with pka_destroy. */
pka_status pka_create(const pka_config* cfg, pka_ctx** out);
void pka_destroy(pka_ctx* ctx);

/* Sizes for a batch of `batch` requests, `num_q_tokens` new tokens and at
 * most `max_kv_pages` pages in total (sum of ceil(L_b / page_size)).  The
 * decode workspace holds partial rows in the output's type (bf16 rows for
 * bf16 queries, fp32 for fp32), each with an fp32 log-sum-exp, for one
 * resident round of the decode launch on the current device (its compute units times the
 * kernel's occupancy; the most the library allows, 2048 shares, if no
 * device can be queried) and up to min(16, max_q_per_request, num_q_tokens)
 * query rows per request for verify batches; it also covers any smaller
 * batch of the same mode on the same device.  For an extend-like batch of
 * bf16 queries with at most 16 rows per request on average, it also covers
 * the extend path's key-range partials (pka_attn_extend): a bf16 row and
 * an fp32 lse per (query row, query head, chunk), with C = min(8, 1024 /
 * (batch * num_kv_heads)) chunks when C >= 3 (no split, and none of these
 * bytes, otherwise). */
pka_status pka_batch_sizes(const pka_ctx* ctx, pka_forward_mode mode, int32_t batch,
                           int32_t num_q_tokens, int64_t max_kv_pages, pka_sizes* out);

/* Build the per-batch index buffers on the device ("What an attention backend
 * is": per-batch metadata such as page tables and index buffers):
 *   kv_indptr[b+1] = kv_indptr[b] + ceil(L_b / P); kv_indices = the first
 *   ceil(L_b / P) ids of page-table row b; kv_last_page_len[b] =
 *   L_b - (ceil(L_b/P) - 1) * P; qo_indptr = prefix sum of n_b;
 *   out_cache_loc = slot (page * P + offset) of each new token;
 *   plan = the work partition for the attention kernels.
 * seq_lens [B] and extend_lens [B] (n_b; NULL for decode) are device int32;
 * page_table is device int32 [B, page_table_stride] whose first
 * page_table_cols entries per row may be read.  md->mode, batch,
 * num_q_tokens, max_kv_pages and the array pointers must be set by the
 * caller.  One kernel launch. */
pka_status pka_init_metadata(const pka_ctx* ctx, const int32_t* seq_lens,
                             const int32_t* extend_lens, const int32_t* page_table,
                             int32_t page_table_stride, int32_t page_table_cols, pka_batch* md,
                             void* stream);

/* Write the new tokens' K and V rows into the pools at out_cache_loc (the
 * backend's save_kv_cache=True step, "[SGLang] Hybrid Attention", forward
 * delegation).  Same dtype: copy.  bf16 -> fp8 e4m3fn: y = x * fp32(1/scale),
 * saturated at +-448 and rounded to nearest even. */
pka_status pka_save_kv(const pka_ctx* ctx, const pka_batch* md, const void* k_new,
                       const void* v_new, void* k_pool, void* v_pool, void* stream);

/* forward_decode: one query per request against its whole cache, split-K
 * flash decoding (split partials + log-sum-exp merge).  workspace: device
 * bytes >= pka_sizes.workspace_bytes.  lse may be NULL.
 * With metadata built for TARGET_VERIFY / DRAFT_EXTEND (the speculative
 * verify pass sent down the decode path, "[SGLang] Hybrid Attention",
 * section on _select_backend), each request carries n_b = extend_lens[b]
 * query rows (0 <= n_b <= R, R = min(16, max_q_per_request)); row i sits at
 * position L_b - n_b + i and sees keys 0 .. L_b - n_b + i, the cache being
 * read once per 16 (row, query head) pairs of a KV head (once for all rows
 * when n_b * G <= 16).  A batch with num_q_tokens > R * batch is refused
 * (PKA_ERR_UNSUPPORTED: some request certainly has more than R rows); rows
 * of a request beyond the R-th are not computed and PKA_DEV_BAD_LENGTH is
 * raised.  The workspace then holds R partial rows per (request, share of
 * the split): pka_batch_sizes sizes it by mode. */
pka_status pka_attn_decode(const pka_ctx* ctx, const pka_batch* md, const void* q,
                           const void* k_pool, const void* v_pool, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/* forward_extend: each new token attends causally to its request's prefix and
 * to the new tokens up to itself.  Same buffers as decode.  A batch of few
 * rows per request has about one work item per request and KV head; when
 * those are too few to fill the chip (the C >= 3 of pka_batch_sizes) and
 * the workspace holds that many partials, each item's key range is cut into
 * C chunks computed by workgroups of their own and merged by a second
 * kernel (the same attention up to rounding); with a smaller workspace, or
 * none, the batch runs unsplit.  bf16 and fp8 e4m3fn caches run on MFMA (fp8 tiles are widened
 * to bf16 exactly on their way into LDS; k_scale and v_scale are applied to
 * the scores and the output), fp32 on the vector ALUs.  bf16 queries cover
 * up to 128 query heads per KV head (checked by pka_create). */
pka_status pka_attn_extend(const pka_ctx* ctx, const pka_batch* md, const void* q,
                           const void* k_pool, const void* v_pool, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/* The pages' backend selection by ForwardMode ("[SGLang] Hybrid Attention",
 * section on _select_backend): decode/idle -> decode; target_verify and
 * draft_extend -> decode if the speculative attention mode is decode, else
 * prefill; everything else -> prefill (extend).  IDLE maps to PKA_PATH_NONE
 * (nothing to compute).  Pure host function. */
pka_path pka_select_path(pka_forward_mode mode, pka_spec_attn_mode spec_mode);

/* One attention layer's forward: optional save_kv, then the path chosen by
 * pka_select_path.  A verify batch routed to the decode path is computed as
 * described at pka_attn_decode (several causal query rows per request).  On
 * a bf16 / fp8 DECODE batch the cache write happens inside the decode kernel
 * (one launch); otherwise save_kv runs first as its own kernel. */
pka_status pka_forward(const pka_ctx* ctx, pka_forward_mode mode, pka_spec_attn_mode spec_mode,
                       const pka_batch* md, const void* q, const void* k_new, const void* v_new,
                       int save_kv, void* k_pool, void* v_pool, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/* pka_init_metadata followed by pka_forward, as one call: builds the batch's
 * metadata into md from seq_lens / extend_lens / page_table (same arguments
 * and results as pka_init_metadata) and runs the forward pass on it (same
 * arguments and results as pka_forward).  The pages build the metadata once
 * per batch and then run the forward ("sglang-101 s4.2 --attention-backend",
 * section "What an attention backend is"); for a DECODE batch with a bf16 or
 * fp8 cache and at most 512 requests both happen in the decode launch
 * itself: every workgroup scans seq_lens and reads page ids straight from
 * the page table, and the metadata arrays are written on the side, bit-equal
 * to what pka_init_metadata writes (two launches: decode, merge).  Other
 * batches launch pka_init_metadata's kernels, then pka_forward's.  All
 * arguments are checked before anything is enqueued; on error nothing is. */
pka_status pka_forward_with_metadata(const pka_ctx* ctx, pka_forward_mode mode,
                                     pka_spec_attn_mode spec_mode, const int32_t* seq_lens,
                                     const int32_t* extend_lens, const int32_t* page_table,
                                     int32_t page_table_stride, int32_t page_table_cols,
                                     pka_batch* md, const void* q, const void* k_new,
                                     const void* v_new, int save_kv, void* k_pool, void* v_pool,
                                     void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* pka_forward_with_metadata without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The extend path runs
 * without its key-range split here.  The decode path's split
 * partials go to a file-scope device array of PKA_NOALLOC_SCRATCH_BYTES that
 * every GPU the library runs on holds until the process ends (its address
 * is looked up on the first call on each device); nothing is allocated, and
 * nothing in it needs clearing between calls.  A batch whose decode
 * partials need more (pka_batch_sizes' workspace_bytes is an upper bound)
 * is refused with PKA_ERR_WORKSPACE and nothing is launched.  All calls on
 * one GPU share the array: calls that overlap in time on one GPU (other
 * streams, concurrent graph replays) race on it.  Otherwise the same
 * arguments, results and errors as pka_forward_with_metadata. */
#define PKA_NOALLOC_SCRATCH_BYTES (64u << 20)
pka_status pka_forward_with_metadata_noalloc(const pka_ctx* ctx, pka_forward_mode mode,
                                             pka_spec_attn_mode spec_mode, const int32_t* seq_lens,
                                             const int32_t* extend_lens, const int32_t* page_table,
                                             int32_t page_table_stride, int32_t page_table_cols,
                                             pka_batch* md, const void* q, const void* k_new,
                                             const void* v_new, int save_kv, void* k_pool,
                                             void* v_pool, void* out, float* lse, void* stream);

/* Synchronise `stream` and read the sticky device status word of a batch:
 * 0 = clean, else a bitwise OR of PKA_DEV_* flags. */
pka_status pka_read_status(const pka_batch* md, int32_t* status, void* stream);
#define PKA_DEV_BAD_LENGTH 1    /* L_b < 1, n_b < 0 or n_b > L_b (clamped) */
#define PKA_DEV_BAD_PAGE 2      /* page id outside [0, num_pages) (clamped) */
#define PKA_DEV_TABLE_SHORT 4   /* ceil(L_b/P) > page_table_cols (clamped) */
#define PKA_DEV_CAPACITY 8      /* pages or tokens beyond the batch capacities */

/* Name the kernels and launch shape a call would resolve to for a batch of
 * `batch` requests and `num_q_tokens` query tokens, as text in buf (len
 * bytes, NUL-terminated); with_metadata: the batch goes through
 * pka_forward_with_metadata.  The pages ask to read which backend was
 * actually resolved before measuring anything ("sglang-101 s4.2
 * --attention-backend", section "What to measure"); this is that read-out
 * for the kernels.  Host-only: it launches nothing (it may query the current
 * device's compute-unit count and the kernels' occupancy).  Returns
 * PKA_ERR_INVALID_ARG if the text does not fit. */
pka_status pka_describe(const pka_ctx* ctx, pka_forward_mode mode, pka_spec_attn_mode spec_mode,
                        int32_t batch, int32_t num_q_tokens, int with_metadata, char* buf, size_t len);

const char* pka_status_string(pka_status s);
const char* pka_last_error(void);

/* Build identification, e.g. "pka 0.1 gfx950". */
const char* pka_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PKA_H */
