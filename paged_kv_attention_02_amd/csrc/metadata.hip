// Per-batch metadata: page-table rows -> CSR index buffers and the work plan.
//
// The pages define an attention backend as building per-batch metadata such
// as page tables and index buffers before running forward_extend or
// forward_decode ("sglang-101 s4.2 --attention-backend", section "What an
// attention backend is").  Two launches:
//   md_scan   one workgroup: clamps lengths, prefix sums (kv_indptr,
//             qo_indptr, flattened token prefix), kv_last_page_len, and the
//             decode / extend work partitions;
//   md_gather a grid over requests: kv_indices (page ids, clamped into the
//             pool) and out_cache_loc (slot of every new token).
#include <algorithm>

#include "pka_internal.h"

namespace pka {
namespace {

constexpr int SCAN_THREADS = 256;  // small workgroups: cheap barriers, more of them share the gather

// Inclusive block scan of NV int64 values per thread: a shuffle scan inside
// each wave, then the wave totals (two barriers in all).
template <int NV>
__device__ inline void block_scan(int64_t (&x)[NV], int64_t* sh) {
    constexpr int NW = SCAN_THREADS / 64;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    #pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int64_t y[NV];
        #pragma unroll
        for (int v = 0; v < NV; ++v) y[v] = __shfl_up(x[v], off);
        if (lane >= off) {
            #pragma unroll
            for (int v = 0; v < NV; ++v) x[v] += y[v];
        }
    }
    if (lane == 63) {
        #pragma unroll
        for (int v = 0; v < NV; ++v) sh[v * NW + wv] = x[v];
    }
    __syncthreads();
    #pragma unroll
    for (int v = 0; v < NV; ++v) {
        int64_t p = 0;
        for (int k = 0; k < wv; ++k) p += sh[v * NW + k];
        x[v] += p;
    }
    __syncthreads();
}

__global__ __launch_bounds__(SCAN_THREADS) void md_scan_kernel(MetaArgs a) {
    // scan scratch
    __shared__ int64_t sh[SCAN_THREADS];
    __shared__ int64_t carry[4];
    __shared__ int32_t s_status;
    // per-request prefixes kept in LDS when the gather is fused (B <= FUSE_MAX_B)
    __shared__ int32_t sP[FUSE_MAX_B + 1], sQ[FUSE_MAX_B + 1], sT[FUSE_MAX_B + 1],
        sLen[FUSE_MAX_B];
    const int t = threadIdx.x;
    const int blk = blockIdx.x;  // > 0 only when the gather is fused: slices of it
    const bool lead = blk == 0;  // the one workgroup that writes the CSR arrays and plan
    const int32_t P = 1 << a.page_shift;
    int32_t* F = a.plan + plan_seg_prefix(a.B);
    int32_t* T = a.plan + plan_tile_prefix(a.B);
    if (t == 0) {
        carry[0] = carry[1] = carry[2] = carry[3] = 0;
        s_status = 0;
        sP[0] = 0;
        sQ[0] = 0;
        sT[0] = 0;
        if (lead) {
            a.kv_indptr[0] = 0;
            a.qo_indptr[0] = 0;
            F[0] = 0;
            T[0] = 0;
        }
    }
    __syncthreads();
    int32_t flags = 0;
    for (int32_t base = 0; base < a.B; base += SCAN_THREADS) {
        const int32_t b = base + t;
        int64_t L = 0, n = 0, pages = 0;
        if (b < a.B) {
            L = a.seq_lens[b];
            n = a.is_decode ? 1 : a.extend_lens[b];
            flags |= md_clamp_request(L, n, pages, a.page_shift, a.pt_cols);
        }
        // pages, new tokens, tokens, decode tiles
        int64_t x[4] = {pages, n, L, (L + DEC_TILE - 1) / DEC_TILE};
        block_scan<4>(x, sh);
        if (b < a.B) {
            const int64_t cp = carry[0] + x[0], cq = carry[1] + x[1], cL = carry[2] + x[2],
                          cT = carry[3] + x[3];
            if (cp > a.max_kv_pages || cq > a.N || cL > INT32_MAX) flags |= PKA_DEV_CAPACITY;
            if (lead) {
                a.kv_indptr[b + 1] = (int32_t)min(cp, (int64_t)INT32_MAX);
                a.qo_indptr[b + 1] = (int32_t)min(cq, (int64_t)INT32_MAX);
                F[b + 1] = (int32_t)min(cL, (int64_t)INT32_MAX);
                T[b + 1] = (int32_t)min(cT, (int64_t)INT32_MAX);
                a.kv_last_page_len[b] = (int32_t)(L - ((pages - 1) << a.page_shift));
            }
            if (a.B <= FUSE_MAX_B) {
                sP[b + 1] = (int32_t)min(cp, (int64_t)INT32_MAX);
                sQ[b + 1] = (int32_t)min(cq, (int64_t)INT32_MAX);
                sT[b + 1] = (int32_t)min(cT, (int64_t)INT32_MAX);
                sLen[b] = (int32_t)L;
            }
        }
        __syncthreads();
        if (t == SCAN_THREADS - 1) {
            #pragma unroll
            for (int v = 0; v < 4; ++v) carry[v] += x[v];
        }
        __syncthreads();
    }
    __syncthreads();
    if (a.fuse_gather) {
        // kv_indices[i] and out_cache_loc[j].  Each thread takes U consecutive
        // items of its workgroup's slice per round: one binary search over the
        // LDS prefixes finds the request of the first (largest b with
        // prefix[b] <= i), the next items step forward from there.  Both
        // kinds of page-table reads go out before any store, so the two
        // gathers cost one round trip to memory.  With more than one
        // workgroup the lead one takes no slice (it builds the plan meanwhile).
        auto find = [&](const int32_t* pre, int32_t i) {
            int32_t lo = 0, hi = a.B - 1;
            while (lo < hi) {
                const int32_t mid = (lo + hi + 1) >> 1;
                if (pre[mid] <= i) lo = mid; else hi = mid - 1;
            }
            return lo;
        };
        constexpr int U = FUSE_PER_THREAD;
        const int32_t g0 = gridDim.x > 1 ? 1 : 0;
        const int32_t nblk = gridDim.x - g0, gblk = blk - g0;
        const int32_t npages = (int32_t)min((int64_t)sP[a.B], a.max_kv_pages);
        const int32_t pchunk = (npages + nblk - 1) / nblk;
        const int32_t p_lo = gblk * pchunk, p_hi = gblk < 0 ? p_lo : min(npages, p_lo + pchunk);
        const int32_t nnew = min(sQ[a.B], a.N);
        const int32_t qchunk = (nnew + nblk - 1) / nblk;
        const int32_t q_lo = gblk * qchunk, q_hi = gblk < 0 ? q_lo : min(nnew, q_lo + qchunk);
        auto clamp_page = [&](int32_t pg) {
            if (pg < 0 || pg >= a.num_pages) {
                flags |= PKA_DEV_BAD_PAGE;
                pg = min(max(pg, 0), a.num_pages - 1);
            }
            return pg;
        };
        for (int32_t k0 = U * t; k0 < max(p_hi - p_lo, q_hi - q_lo); k0 += U * SCAN_THREADS) {
            int32_t pg[U], qpg[U], pos[U];
            const int32_t i0 = p_lo + k0, j0 = q_lo + k0;
            int32_t bp = i0 < p_hi ? find(sP, i0) : 0;
            int32_t bq = j0 < q_hi ? find(sQ, j0) : 0;
            #pragma unroll
            for (int u = 0; u < U; ++u) {
                const int32_t i = i0 + u;
                if (i < p_hi) {
                    while (sP[bp + 1] <= i) ++bp;
                    pg[u] = a.page_table[(int64_t)bp * a.pt_stride + (i - sP[bp])];
                }
                const int32_t jq = j0 + u;
                if (jq < q_hi) {
                    while (sQ[bq + 1] <= jq) ++bq;
                    pos[u] = sLen[bq] - (sQ[bq + 1] - sQ[bq]) + (jq - sQ[bq]);
                    qpg[u] = a.page_table[(int64_t)bq * a.pt_stride + (pos[u] >> a.page_shift)];
                }
            }
            #pragma unroll
            for (int u = 0; u < U; ++u) {
                if (i0 + u < p_hi) a.kv_indices[i0 + u] = clamp_page(pg[u]);
                if (j0 + u < q_hi)
                    a.out_cache_loc[j0 + u] = (clamp_page(qpg[u]) << a.page_shift) | (pos[u] & (P - 1));
            }
        }
    }
    if (flags) atomicOr(&s_status, flags);
    __syncthreads();
    __threadfence_block();

    if (!lead) {  // a gather slice: report its flags in its own status slot
        if (flags) atomicOr(&s_status, flags);
        __syncthreads();
        if (t == 0) a.plan[PLAN_MDST + blk] = s_status;
        return;
    }
    const int64_t W = min(carry[3], (int64_t)INT32_MAX);
    {
        // Decode partition (built for every batch, so a verify batch can take
        // either path): every request is laid out as its ceil(L / DEC_TILE)
        // tiles, the requests end to end, and that tile range [0, W) is cut
        // into nwg shares of q or q + 1 tiles (at least DEC_MIN_SHARE);
        // share w starts in the request that holds its first tile.
        // Cutting at tile boundaries leaves no partial tile except a
        // request's last, so the shares differ by at most one tile of work.
        int64_t share, rem;
        decode_shares(W, a.nwg, share, rem);
        int32_t* wg_seg = a.plan + plan_wg_seg(a.B);
        int32_t* share_flags = a.plan + plan_share_flags(a.B);
        for (int32_t w = t; w < a.nwg; w += SCAN_THREADS) {
            share_flags[w] = 0;
            const int64_t pos = share_start(w, share, rem);
            int32_t seg = a.B;
            if (pos < W) {
                const int32_t* Ts = a.B <= FUSE_MAX_B ? sT : T;
                int32_t lo = 0, hi = a.B - 1;  // largest b with T[b] <= pos
                while (lo < hi) {
                    const int32_t mid = (lo + hi + 1) >> 1;
                    if (Ts[mid] <= pos) lo = mid; else hi = mid - 1;
                }
                seg = lo;
            }
            wg_seg[w] = seg;
        }
        if (t == 0) {
            a.plan[PLAN_SHARE] = (int32_t)share;
            a.plan[PLAN_SHARE_REM] = (int32_t)rem;
            a.plan[PLAN_TOTAL] = (int32_t)W;
            a.plan[PLAN_NWG] = a.nwg;
            a.plan[PLAN_EXT_COUNT] = 0;
            a.plan[PLAN_EXT_TQ] = a.ext_tq;
        }
    }
    if (!a.is_decode) {
        // Extend items (request, query tile of tq tokens), request by
        // request: the workgroups of one KV head run on one XCD in list order,
        // so the ones resident together work on one or two requests and
        // share their K/V pages in that XCD's L2 (a K/V head of a request is
        // at most a few MB; several requests at once overflow the L2).  A
        // tile's cost grows with the last key position it attends to, so
        // each request's tiles go last to first (heaviest first) and the
        // requests go longest first (ties: lower index first), which keeps
        // the heaviest items at the front of the list.  Batches beyond
        // FUSE_MAX_B requests keep request order.
        const int32_t tq = a.ext_tq;
        const int64_t cap = plan_ext_capacity(a.B, a.N, tq);
        int32_t* items = a.plan + plan_ext_items(a.B);
        __shared__ int32_t s_count;
        __shared__ int32_t sI[FUSE_MAX_B + 1];  // first item of each request (request order)
        __shared__ int32_t sR[FUSE_MAX_B];      // fused: rank of each request
        __shared__ int32_t sS[FUSE_MAX_B + 1];  // fused: first item of each rank
        if (t == 0) s_count = 0;
        __syncthreads();
        auto tiles_of = [&](int32_t b) {  // query tiles of request b (fused: from the LDS prefix)
            return (sQ[b + 1] - sQ[b] + tq - 1) / tq;
        };
        // exclusive prefix of v[0 .. n) into out[0 .. n], in chunks of the
        // workgroup (s_count carries the running total)
        auto prefix = [&](int32_t n, auto value, int32_t* out) {
            for (int32_t base = 0; base < n; base += SCAN_THREADS) {
                const int32_t j = base + t;
                int64_t x[1] = {j < n ? (int64_t)value(j) : 0};
                const int64_t own = x[0];
                block_scan<1>(x, sh);
                if (j < n) out[j] = s_count + (int32_t)(x[0] - own);
                __syncthreads();
                if (t == SCAN_THREADS - 1) s_count += (int32_t)x[0];
                __syncthreads();
            }
            if (t == 0) out[n] = s_count;
            __syncthreads();
        };
        int32_t count;
        if (a.B <= FUSE_MAX_B) {
            // rank of request b: requests that are longer, or as long and
            // earlier (the lengths are in LDS; every thread reads the same
            // entry at a time)
            for (int32_t b = t; b < a.B; b += SCAN_THREADS) {
                const int32_t L = sLen[b];
                int32_t r = 0;
                for (int32_t j = 0; j < a.B; ++j) {
                    const int32_t Lj = sLen[j];
                    r += (Lj > L) | ((Lj == L) & (j < b));
                }
                sR[b] = r;
                sS[r] = tiles_of(b);  // tile count by rank, scanned in place below
            }
            __syncthreads();
            prefix(a.B, [&](int32_t r) { return sS[r]; }, sS);
            if (t == 0) s_count = 0;
            __syncthreads();
            prefix(a.B, tiles_of, sI);
            count = sI[a.B];
            if (count > cap) { flags |= PKA_DEV_CAPACITY; count = (int32_t)cap; }
            // item i of the request-order list: request b (largest b with
            // sI[b] <= i), tile i - sI[b]; its place: the rank's first item
            // plus its distance from the request's last tile
            for (int32_t i = t; i < sI[a.B]; i += SCAN_THREADS) {
                int32_t lo = 0, hi = a.B - 1;
                while (lo < hi) {
                    const int32_t mid = (lo + hi + 1) >> 1;
                    if (sI[mid] <= i) lo = mid; else hi = mid - 1;
                }
                const int32_t b = lo, ti = i - sI[b];
                const int32_t pos = sS[sR[b]] + (sI[b + 1] - sI[b] - 1 - ti);
                if (pos < count) {
                    items[2 * pos] = b;
                    items[2 * pos + 1] = ti;
                }
            }
        } else {
            // large batches: request order, SCAN_THREADS requests at a time;
            // the chunk's items are written by all threads in parallel
            __shared__ int32_t cI[SCAN_THREADS + 1];
            for (int32_t base = 0; base < a.B; base += SCAN_THREADS) {
                const int32_t nb = min(SCAN_THREADS, a.B - base);
                prefix(nb, [&](int32_t j) {
                    const int32_t b = base + j;
                    return (a.qo_indptr[b + 1] - a.qo_indptr[b] + tq - 1) / tq;
                }, cI);
                for (int32_t i = cI[0] + t; i < cI[nb]; i += SCAN_THREADS) {
                    int32_t lo = 0, hi = nb - 1;
                    while (lo < hi) {
                        const int32_t mid = (lo + hi + 1) >> 1;
                        if (cI[mid] <= i) lo = mid; else hi = mid - 1;
                    }
                    const int32_t ti = i - cI[lo];
                    const int32_t pos = cI[lo] + (cI[lo + 1] - cI[lo] - 1 - ti);
                    if (pos < cap) {
                        items[2 * pos] = base + lo;
                        items[2 * pos + 1] = ti;
                    }
                }
                __syncthreads();  // cI is rewritten by the next chunk
            }
            count = s_count;
            if (count > cap) { flags |= PKA_DEV_CAPACITY; count = (int32_t)cap; }
        }
        if (t == 0) a.plan[PLAN_EXT_COUNT] = count;
    }
    if (flags) atomicOr(&s_status, flags);
    __syncthreads();
    if (t == 0) {
        a.plan[PLAN_MDST] = s_status;
        a.plan[PLAN_STATUS] = 0;  // later kernels OR their flags into it
    }
    for (int i = (int)gridDim.x + t; i < MD_SLOTS; i += SCAN_THREADS) a.plan[PLAN_MDST + i] = 0;
}

// kv_indices and out_cache_loc.  Grid (x, B); page ids outside the pool are
// clamped (and flagged) so that no later kernel reads outside the pools.
__global__ __launch_bounds__(256) void md_gather_kernel(MetaArgs a) {
    const int32_t b = blockIdx.y;
    const int32_t P = 1 << a.page_shift;
    const int32_t p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
    const int32_t L = (p1 - p0 - 1) * P + a.kv_last_page_len[b];
    const int32_t q0 = a.qo_indptr[b], q1 = a.qo_indptr[b + 1];
    const int32_t n = q1 - q0;
    const int32_t* row = a.page_table + (int64_t)b * a.pt_stride;
    int32_t flags = 0;
    const int32_t step = gridDim.x * blockDim.x;
    for (int32_t k = blockIdx.x * blockDim.x + threadIdx.x; k < p1 - p0; k += step) {
        int32_t pg = row[k];
        if (pg < 0 || pg >= a.num_pages) {
            flags |= PKA_DEV_BAD_PAGE;
            pg = min(max(pg, 0), a.num_pages - 1);
        }
        if (p0 + k < a.max_kv_pages) a.kv_indices[p0 + k] = pg;
    }
    for (int32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) {
        const int32_t pos = L - n + i;
        int32_t pg = row[pos >> a.page_shift];
        if (pg < 0 || pg >= a.num_pages) {
            flags |= PKA_DEV_BAD_PAGE;
            pg = min(max(pg, 0), a.num_pages - 1);
        }
        if (q0 + i < a.N) a.out_cache_loc[q0 + i] = (pg << a.page_shift) | (pos & (P - 1));
    }
    if (flags) atomicOr(a.plan + PLAN_STATUS, flags);
}

}  // namespace

hipError_t launch_metadata(const MetaArgs& a, hipStream_t s) {
    // fused: enough workgroups that each thread has at most FUSE_PER_THREAD
    // lookups of each kind
    int nblk = 1;
    if (a.fuse_gather) {
        // the lead workgroup, plus the gather slices
        const int64_t items = std::max<int64_t>(a.max_kv_pages, a.N);
        const int64_t per = (int64_t)SCAN_THREADS * FUSE_PER_THREAD;
        nblk = (int)std::min<int64_t>(MD_SLOTS, 1 + (items + per - 1) / per);
    }
    hipLaunchKernelGGL(md_scan_kernel, dim3(nblk), dim3(SCAN_THREADS), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.B == 0 || a.fuse_gather) return e;
    // enough blocks per request to cover its pages in one or two strides
    int64_t per_req = (a.max_kv_pages / a.B + 255) / 256;
    if (!a.is_decode) per_req = std::max<int64_t>(per_req, ((int64_t)a.N / a.B + 255) / 256);
    const int gx = (int)std::min<int64_t>(std::max<int64_t>(per_req, 1), 64);
    hipLaunchKernelGGL(md_gather_kernel, dim3(gx, a.B), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace pka
