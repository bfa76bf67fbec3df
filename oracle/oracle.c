/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for paged KV
 * attention over one batch.  TEST INFRASTRUCTURE ONLY: it is called by the
 * tests, by the smoke check and by the benchmark's CPU-baseline leg, never by
 * the product path.  It shares no code, header or table with the HIP library.
 *
 * What it follows.  The pages define an attention backend as the class that
 * computes attention over the paged KV cache for one batch, building
 * per-batch metadata such as page tables and index buffers, and running
 * forward_extend (prefill) and forward_decode (decode) ("sglang-101 s4.2
 * --attention-backend", section "What an attention backend is").  The
 * backend's forward takes q, k, v and save_kv_cache=True, so new K/V are
 * written into the cache before attention ("[SGLang] Hybrid Attention",
 * section on forward delegation).  The pages never print the attention
 * formula; it is read as plain scaled-dot-product softmax attention,
 * out = softmax(scale * q K^T) V, with grouped query heads (head h reads KV
 * head h / (Hq/Hkv)) and bottom-right causal alignment for extend (query i
 * of a request with prefix p sees keys 0..p+i).
 *
 * Parity unpinned by the pages for two conventions: the head grouping
 * (contiguous groups) and the causal alignment (bottom-right) are readings,
 * not printed there.  The tests pin the oracle to them through torch's CPU
 * scaled-dot-product attention with explicit head repetition and an explicit
 * boolean mask, and through the grouping and causal-edit invariants; that
 * fixes the arithmetic, not the reading.
 *
 * Everything is fp64 with an explicit per-token page gather and a two-pass
 * softmax (max first, then exponentials); no blocking, no online softmax.
 *
 * dtype codes: 0 = fp32, 1 = bf16 (raw 16-bit patterns), 2 = fp8 e4m3fn
 * (OCP: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals,
 * S.1111.111 is NaN, no infinities, largest finite 448).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1
#define OR_FP8 2

/* ---------------------------------------------------------------- values */

double oracle_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Value of an e4m3fn code, read off the format definition. */
double oracle_fp8_value(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9); /* subnormal: m/8 * 2^(1-7) */
    else
        v = ldexp(8.0 + m, e - 7 - 3); /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/*
 * Round an fp32 value to e4m3fn: saturate magnitudes at 448, otherwise round
 * to the nearest representable value with ties to the even code.  The
 * representable values in the binade [2^E, 2^(E+1)) are multiples of
 * 2^(E-3); below 2^-6 they are multiples of 2^-9 (subnormals).
 */
uint8_t oracle_fp8_encode(float y) {
    if (isnan(y)) return 0x7F;
    int neg = signbit(y) ? 1 : 0;
    double a = fabs((double)y);
    uint8_t code;
    if (a >= 448.0) {
        code = 0x7E; /* 1.75 * 2^8 */
    } else if (a == 0.0) {
        code = 0;
    } else {
        int ex;
        frexp(a, &ex); /* a = f * 2^ex with f in [0.5, 1) */
        int E = ex - 1; /* a in [2^E, 2^(E+1)) */
        if (E < -6) E = -6;
        double quantum = ldexp(1.0, E - 3);
        double k = nearbyint(a / quantum); /* a/quantum is exact; RNE */
        double r = k * quantum;            /* at most 448 because a < 448 */
        if (r == 0.0) {
            code = 0;
        } else {
            int rx;
            frexp(r, &rx);
            int RE = rx - 1;
            if (RE < -6) {
                code = (uint8_t)(int)(r / ldexp(1.0, -9)); /* subnormal mantissa */
            } else {
                int mant = (int)(r / ldexp(1.0, RE - 3)) - 8;
                code = (uint8_t)(((RE + 7) << 3) | mant);
            }
        }
    }
    return (uint8_t)(code | (neg << 7));
}

/* fp8 cache write of one value: y = f32(x) * f32(1/scale), then encode. */
void oracle_fp8_quantize(int64_t n, const uint16_t* bf16_bits, float scale, uint8_t* out) {
    float inv = 1.0f / scale;
    for (int64_t i = 0; i < n; ++i) {
        float x = (float)oracle_bf16_value(bf16_bits[i]);
        float y = x * inv;
        out[i] = oracle_fp8_encode(y);
    }
}

static double load_value(int dtype, const void* base, int64_t idx, double fp8_scale) {
    switch (dtype) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_BF16: return oracle_bf16_value(((const uint16_t*)base)[idx]);
    default: return oracle_fp8_value(((const uint8_t*)base)[idx]) * fp8_scale;
    }
}

/* ------------------------------------------------------------- metadata */

/*
 * Per-batch index buffers over pages ("What an attention backend is": page
 * tables and index buffers).  Decode when extend_lens == NULL (one new token
 * per request).  Arithmetic in int64, range-checked into int32.
 *   kv_indptr[b+1]      = kv_indptr[b] + ceil(L_b / P)
 *   kv_indices          = first ceil(L_b / P) page ids of each page-table row
 *   kv_last_page_len[b] = L_b - (ceil(L_b / P) - 1) * P
 *   qo_indptr[b+1]      = qo_indptr[b] + n_b
 *   out_cache_loc[j]    = slot of the j-th new token: page * P + offset
 * Returns 0, or -1 for inconsistent input.
 */
int oracle_metadata(int32_t B, const int32_t* seq_lens, const int32_t* extend_lens,
                    const int32_t* page_table, int64_t stride, int32_t cols, int32_t P,
                    int32_t num_pages, int32_t* kv_indptr, int32_t* kv_indices,
                    int64_t kv_indices_cap, int32_t* kv_last_page_len, int32_t* qo_indptr,
                    int32_t* out_cache_loc, int64_t out_cap) {
    int64_t pages_acc = 0, q_acc = 0;
    kv_indptr[0] = 0;
    qo_indptr[0] = 0;
    for (int32_t b = 0; b < B; ++b) {
        int64_t L = seq_lens[b];
        int64_t n = extend_lens ? extend_lens[b] : 1;
        if (L < 1 || n < 0 || n > L) return -1;
        int64_t pages = (L + P - 1) / P;
        if (pages > cols) return -1;
        for (int64_t k = 0; k < pages; ++k) {
            int32_t pg = page_table[b * stride + k];
            if (pg < 0 || pg >= num_pages) return -1;
            if (pages_acc + k >= kv_indices_cap) return -1;
            kv_indices[pages_acc + k] = pg;
        }
        for (int64_t i = 0; i < n; ++i) {
            int64_t pos = L - n + i;
            int64_t slot = (int64_t)page_table[b * stride + pos / P] * P + pos % P;
            if (q_acc + i >= out_cap || slot > INT32_MAX) return -1;
            out_cache_loc[q_acc + i] = (int32_t)slot;
        }
        pages_acc += pages;
        q_acc += n;
        if (pages_acc > INT32_MAX || q_acc > INT32_MAX) return -1;
        kv_indptr[b + 1] = (int32_t)pages_acc;
        qo_indptr[b + 1] = (int32_t)q_acc;
        kv_last_page_len[b] = (int32_t)(L - (pages - 1) * P);
    }
    return 0;
}

/* --------------------------------------------------------------- save_kv */

/*
 * Write new K rows [N, Hkv, Dk] and V rows [N, Hkv, Dv] (source dtype fp32 or
 * bf16) into the pools [slots, Hkv, Dk] and [slots, Hkv, Dv] at the given
 * slots (K and V may have different head widths).  Same dtype: the bits are
 * copied.  bf16 -> fp8: oracle_fp8_quantize with the per-tensor scale.
 */
int oracle_save_kv(int64_t N, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t src_dtype,
                   int32_t kv_dtype, const int32_t* slots, const void* k_new, const void* v_new,
                   float k_scale, float v_scale, void* k_pool, void* v_pool) {
    int64_t krow = (int64_t)Hkv * Dk, vrow = (int64_t)Hkv * Dv;
    for (int64_t j = 0; j < N; ++j) {
        int64_t slot = slots[j];
        if (kv_dtype == src_dtype) {
            size_t eb = kv_dtype == OR_F32 ? 4 : 2;
            memcpy((char*)k_pool + slot * krow * eb, (const char*)k_new + j * krow * eb, krow * eb);
            memcpy((char*)v_pool + slot * vrow * eb, (const char*)v_new + j * vrow * eb, vrow * eb);
        } else if (src_dtype == OR_BF16 && kv_dtype == OR_FP8) {
            oracle_fp8_quantize(krow, (const uint16_t*)k_new + j * krow, k_scale,
                                (uint8_t*)k_pool + slot * krow);
            oracle_fp8_quantize(vrow, (const uint16_t*)v_new + j * vrow, v_scale,
                                (uint8_t*)v_pool + slot * vrow);
        } else {
            return -1;
        }
    }
    return 0;
}

/* ------------------------------------------------------------- attention */

/*
 * Attention for selected (query token, head) pairs.  sel[i] = token * Hq + h;
 * sel == NULL means every pair in order.  Queries and keys have head width
 * Dk, values and outputs Dv (a model may give K and V different widths).
 * out: [n_sel, Dv], lse: [n_sel] (natural log of the softmax denominator
 * including the max).  extend_lens == NULL means decode (one query per
 * request, at position L-1).
 */
int oracle_attention(int32_t B, int32_t Hq, int32_t Hkv, int32_t Dk, int32_t Dv, int32_t P,
                     const int32_t* seq_lens, const int32_t* extend_lens,
                     const int32_t* page_table, int64_t stride, int32_t num_pages,
                     int32_t q_dtype, const void* q, int32_t kv_dtype, const void* k_pool,
                     const void* v_pool, double scale, double k_scale, double v_scale,
                     int64_t n_sel, const int64_t* sel, double* out, double* lse,
                     int32_t num_threads) {
    if (Hkv <= 0 || Hq % Hkv != 0) return -1;
    int32_t G = Hq / Hkv;
    int64_t N = 0;
    int64_t max_len = 1;
    for (int32_t b = 0; b < B; ++b) {
        int64_t n = extend_lens ? extend_lens[b] : 1;
        if (seq_lens[b] < 1 || n < 0 || n > seq_lens[b]) return -1;
        N += n;
        if (seq_lens[b] > max_len) max_len = seq_lens[b];
    }
    /* token -> (request, index among its new tokens) */
    int32_t* tok_req = (int32_t*)malloc(sizeof(int32_t) * (N > 0 ? N : 1));
    int64_t* tok_idx = (int64_t*)malloc(sizeof(int64_t) * (N > 0 ? N : 1));
    if (!tok_req || !tok_idx) return -2;
    {
        int64_t j = 0;
        for (int32_t b = 0; b < B; ++b) {
            int64_t n = extend_lens ? extend_lens[b] : 1;
            for (int64_t i = 0; i < n; ++i, ++j) {
                tok_req[j] = b;
                tok_idx[j] = i;
            }
        }
    }
    int64_t total = sel ? n_sel : N * Hq;
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel reduction(| : bad)
#endif
    {
        double* s = (double*)malloc(sizeof(double) * max_len);
        double* acc = (double*)malloc(sizeof(double) * Dv);
        double* qv = (double*)malloc(sizeof(double) * Dk);
        if (!s || !acc || !qv) bad = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t it = 0; it < total; ++it) {
            if (!s || !acc || !qv) continue;
            int64_t pair = sel ? sel[it] : it;
            int64_t j = pair / Hq;
            int32_t h = (int32_t)(pair % Hq);
            if (j < 0 || j >= N) { bad = 1; continue; }
            int32_t b = tok_req[j];
            int64_t L = seq_lens[b];
            int64_t n = extend_lens ? extend_lens[b] : 1;
            int64_t pos = L - n + tok_idx[j]; /* bottom-right causal alignment */
            int32_t g = h / G;                /* grouped query heads */
            for (int32_t d = 0; d < Dk; ++d)
                qv[d] = load_value(q_dtype, q, (j * Hq + h) * (int64_t)Dk + d, 1.0);
            /* pass 1: scores s_t = scale * q . k_t over the explicit page gather */
            double m = -INFINITY;
            for (int64_t t = 0; t <= pos; ++t) {
                int32_t pg = page_table[b * stride + t / P];
                if (pg < 0 || pg >= num_pages) { bad = 1; break; }
                int64_t slot = (int64_t)pg * P + t % P;
                int64_t base = (slot * Hkv + g) * (int64_t)Dk;
                double dot = 0.0;
                for (int32_t d = 0; d < Dk; ++d)
                    dot += qv[d] * load_value(kv_dtype, k_pool, base + d, k_scale);
                s[t] = scale * dot;
                if (s[t] > m) m = s[t];
            }
            /* pass 2: weights, normaliser, weighted sum of V */
            double Z = 0.0;
            for (int32_t d = 0; d < Dv; ++d) acc[d] = 0.0;
            for (int64_t t = 0; t <= pos; ++t) {
                int32_t pg = page_table[b * stride + t / P];
                if (pg < 0 || pg >= num_pages) break;
                int64_t slot = (int64_t)pg * P + t % P;
                int64_t base = (slot * Hkv + g) * (int64_t)Dv;
                double w = exp(s[t] - m);
                Z += w;
                for (int32_t d = 0; d < Dv; ++d)
                    acc[d] += w * load_value(kv_dtype, v_pool, base + d, v_scale);
            }
            for (int32_t d = 0; d < Dv; ++d) out[it * Dv + d] = acc[d] / Z;
            if (lse) lse[it] = m + log(Z);
        }
        free(s);
        free(acc);
        free(qv);
    }
    free(tok_req);
    free(tok_idx);
    return bad ? -1 : 0;
}

/* Bytes of one token-major pool [tokens, heads, head_dim] with no padding. */
int64_t oracle_pool_bytes(int64_t tokens, int64_t heads, int64_t head_dim, int64_t elem_bytes) {
    return tokens * heads * head_dim * elem_bytes;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Vector form of oracle_fp8_encode, for exhaustive tests. */
void oracle_fp8_encode_array(int64_t n, const float* y, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_encode(y[i]);
}
