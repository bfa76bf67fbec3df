// forward_decode: one query token per request against its paged cache.
//
// Decode reads one query against a long cache and is memory-bound
// ("sglang-101 s4.2 --attention-backend", section "Two backends in one
// server"; "[SGLang] Hybrid Attention", introduction).  The kernel is split-K
// flash decoding: the batch's 32-token tiles, laid end to end, are cut into
// shares equal to within a tile, one or more per workgroup; each wave serves
// one KV head (16 query heads of its group at most) over one share with an
// online softmax, and a share that covers only part of a request leaves a
// partial (its normalised output row in the output's type and an fp32
// log-sum-exp) that a merge kernel combines in fp32.
//
// gfx950 mapping of the MFMA variant (bf16 or fp8 e4m3fn cache):
//   S^T[token, head]  = K[token, :] . Q^T        v_mfma_f32_16x16x32_bf16
//   O^T[d, head]     += V^T[d, token] . P^T      v_mfma_f32_16x16x32_bf16
// K tiles reach a per-wave LDS tile by direct HBM -> LDS loads that read whole
// row pieces (the A operand's own layout would read 64-byte pieces, which
// HBM serves slower) and are read back as the A operand; the scores come out
// with one head per lane column, so the softmax row statistics stay in the
// lane and P^T feeds the second MFMA without a shuffle.  V rows are loaded
// into registers as whole 256-byte (bf16) rows per 16 lanes and transposed
// with v_perm_b32 (fp8: byte gather + v_cvt_scalef32_pk_bf16_fp8).  The token
// order inside a tile is a permutation chosen so every operand lines up.
// Each wave walks its share as one stream of tiles with one tile in flight.
#include "fp8.h"
#include "pka_internal.h"

namespace pka {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float LN2 = 0.69314718055994531f;

__device__ inline uint32_t bits(bf16x2_t v) { return __builtin_bit_cast(uint32_t, v); }

__device__ inline uint32_t pack_bf16(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
    return bits(v);
}

__device__ inline bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Uniform 32-bit load through the scalar data cache (read only).
__device__ inline int32_t load_uniform(const int32_t* p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)(uintptr_t)p)[i];
}

// Pool slot of token position `pos` of a request whose pages start at
// kv_indices[page_base]; indices and page ids are clamped into their buffers.
__device__ inline int32_t slot_of(const AttnArgs& a, int32_t page_base, int32_t pos) {
    int64_t idx = (int64_t)page_base + (pos >> a.page_shift);
    idx = idx < a.kv_cap ? idx : a.kv_cap - 1;
    int32_t pg = a.kv_indices[idx];
    pg = min(max(pg, 0), a.num_pages - 1);
    return (pg << a.page_shift) | (pos & ((1 << a.page_shift) - 1));
}

__device__ inline float wave_max_xor_16_32(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float wave_sum_xor_16_32(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// Write a finished (or partial) result of one wave: lane (n, j) owns head n
// and the D/4 consecutive dims starting at j * D/4, stored as O[c][r] with
// d = CPL * (4 j + r) + c.
template <int D, typename Emit>
__device__ inline void emit_rows(const f32x4_t (&O)[D / 16], float inv, int j, Emit emit) {
    constexpr int CPL = D / 16;
    float v[4 * CPL];
    #pragma unroll
    for (int r = 0; r < 4; ++r)
        #pragma unroll
        for (int c = 0; c < CPL; ++c) v[r * CPL + c] = O[c][r] * inv;
    emit(v, 4 * CPL * j);
}

// Cache write of one request's new token for KV head g, fused into decode,
// in two halves.  load_new_token reads this lane's part of the row (query row
// qr): K on lanes 0..31, V on lanes 32..63, 8 elements per lane; lanes past a
// row's width read nothing.
template <int DK, int DV>
__device__ inline u32x4_t load_new_token(const AttnArgs& a, int32_t qr, int g, int lane) {
    const bool is_v = lane >= 32;
    const int D = is_v ? DV : DK;
    const int e = (lane & 31) * 8;  // first element of this lane
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (e < D)
        w = *(const u32x4_t*)((const __bf16*)(is_v ? a.v_new : a.k_new) + ((int64_t)qr * a.Hkv + g) * D + e);
    return w;
}

// store_new_token writes it to pool slot `slot` (bf16 copy or bf16 -> fp8
// quantisation).  Nothing waits for the store: a wave's vector memory
// instructions reach memory in issue order, so the wave's own later load of
// that slot (the only one in the launch) returns the new row.
template <int DK, int DV, bool FP8>
__device__ inline void store_new_token(const AttnArgs& a, u32x4_t w, int32_t slot, int g, int lane) {
    if (slot < 0 || slot >= a.pool_slots) {
        if (lane == 0) atomicOr((int32_t*)a.plan + PLAN_STATUS, PKA_DEV_BAD_PAGE);
        return;
    }
    const bool is_v = lane >= 32;
    const int D = is_v ? DV : DK;
    const int e = (lane & 31) * 8;
    if (e < D) {
        const int64_t dst = ((int64_t)slot * a.Hkv + g) * D + e;
        if constexpr (FP8) {
            const float inv = is_v ? a.v_inv : a.k_inv;
            *(u32x2_t*)((uint8_t*)(is_v ? a.v_pool : a.k_pool) + dst) =
                u32x2_t{quant4(w.x, w.y, inv), quant4(w.z, w.w, inv)};
        } else {
            *(u32x4_t*)((__bf16*)(is_v ? a.v_pool : a.k_pool) + dst) = w;
        }
    }
}

// DK: key (and query) width; DV: value (and output) width.
template <int DK, int DV, bool FP8>
struct DecodeShape {
    static constexpr int ESZ = FP8 ? 1 : 2;    // cache bytes per element
    static constexpr int KE = 16 / ESZ;        // elements per 16-byte K load
    static constexpr int NKL = DK * ESZ / 64;  // 16-byte K loads per lane per 16 tokens
    static constexpr int KSTEPS = DK / 32;     // MFMA k-steps of q.k
    static constexpr int SPL = KE / 8;         // k-steps per K load
    static constexpr int CPL = DV / 16;        // V dims per lane per token = PV MFMAs
    static_assert(NKL * SPL == KSTEPS, "k-step bookkeeping");
    using vrow_t = typename std::conditional<
        CPL * ESZ == 16, u32x4_t,
        typename std::conditional<CPL * ESZ == 8, u32x2_t, uint32_t>::type>::type;
    // K goes through one LDS tile per wave (see load_k), V into registers.
    static constexpr int KROW = DK * ESZ;       // bytes of one token's K row (one head)
    static constexpr int KCPR = KROW / 16;      // 16-byte chunks per K row
    static constexpr int KDMA = KCPR / 2;       // direct-to-LDS loads per lane and tile
    static constexpr int KTILE = DEC_TILE * KROW;  // bytes of the LDS K tile
    static_assert(KCPR == 4 || KCPR == 8 || KCPR == 12 || KCPR == 16 || KCPR == 24, "K row width");
    // Chunk swizzle of the LDS K tile: the K operand reads 16 rows at one
    // logical chunk, and those 16 rows must hit 16 different 16-byte bank
    // groups (256 bytes per bank cycle).  An XOR inside the chunk's aligned
    // group keeps every chunk in its row.
    __device__ static constexpr int kswz(int row, int c) {
        return KCPR == 16 ? c ^ (row & 15)
             : (KCPR == 8 || KCPR == 24) ? c ^ ((row >> 1) & 7)
             : c ^ ((row >> 2) & 3);
    }
};

// LDS bytes of one decode wave: the K tile and the queries of cb column
// blocks (1 KB per k-step each).
template <int DK, int DV, bool FP8>
__host__ __device__ constexpr int decode_wave_lds(int cb) {
    return DecodeShape<DK, DV, FP8>::KTILE + cb * DecodeShape<DK, DV, FP8>::KSTEPS * 1024;
}

typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;

// Direct HBM -> LDS load of 16 bytes per lane: lane i's bytes land at
// lds_dst + 16 * i (lds_dst is wave-uniform; the compiler moves it to M0).
// The load counts in vmcnt like any other; the kernel still waits for it
// with an explicit vmcnt(0) before the data is read.  STREAM: the
// non-temporal policy, for cache rows that are read once per call.
template <bool STREAM = false>
__device__ inline void lds_dma16(const void* src, const uint8_t* lds_dst) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds_dst, 16, 0,
                                     STREAM ? 2 /* nt */ : 0);
}

// V of one 32-token tile in registers: k-slot q of lane group j holds tile
// token 16*(q/4) + 4*j + q%4, the order in which the scores come out of the
// first MFMA, so P^T needs no shuffle.
template <int DK, int DV, bool FP8>
struct VTile {
    typename DecodeShape<DK, DV, FP8>::vrow_t vr[8];
};

// The loads of one tile.  `slot` is the pool slot of tile token (lane & 31);
// lanes exchange slots with cross-lane moves.  The cache is read once per
// call, so the K direct loads and the V loads carry the non-temporal policy
// (the split partials, written between the reads, then stay cached).
//
// K goes to the wave's LDS tile `kst`: a wave instruction moves 1 KB of the
// tile, lane i the 16-byte chunk f = 64 q + i of the tile's rows laid end to
// end (row f / KCPR, physical chunk f % KCPR, fetched from the logical chunk
// the swizzle puts there), so every instruction reads whole 128- to
// 256-byte row pieces; the K operand's own layout (four lanes per token)
// would read 64-byte pieces, which HBM serves markedly slower.
template <int DK, int DV, bool FP8>
__device__ inline void load_k(uint8_t* kst, int32_t slot, const uint8_t* kbase, int64_t krow) {
    using S = DecodeShape<DK, DV, FP8>;
    const int lane = threadIdx.x & 63;
    // every row's slot first, so one wait covers the cross-lane moves
    int32_t ks[S::KDMA];
    #pragma unroll
    for (int q = 0; q < S::KDMA; ++q) ks[q] = __shfl(slot, (64 * q + lane) / S::KCPR);
    #pragma unroll
    for (int q = 0; q < S::KDMA; ++q) {
        const int f = 64 * q + lane;
        const int row = f / S::KCPR, pc = f % S::KCPR;
        lds_dma16<true>(kbase + ks[q] * krow + 16 * S::kswz(row, pc), kst + 1024 * q);
    }
}
template <int DK, int DV, bool FP8>
__device__ inline void load_v(VTile<DK, DV, FP8>& T, int32_t slot, const uint8_t* vbase, int64_t vrow,
                              int n, int j) {
    using S = DecodeShape<DK, DV, FP8>;
    #pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int32_t vs = __shfl(slot, 16 * (q >> 2) + 4 * j + (q & 3));
        T.vr[q] = __builtin_nontemporal_load(
            (const typename S::vrow_t*)(vbase + vs * vrow + n * (S::CPL * S::ESZ)));
    }
}

// S^T = K . Q^T for one tile, two 16-token row blocks, K from the wave's LDS
// tile: lane (n, j) of row block sb reads chunk 4 s + j of token 16 sb + n.
// qop(k, ks): the Q^T operand of k-step ks for column block k (CB blocks of
// 16 columns share every K operand read).
template <int DK, int DV, bool FP8, int CB, typename QOp>
__device__ inline void tile_scores(const uint8_t* kst, QOp qop, f32x4_t (&st)[CB][2], int j) {
    using S = DecodeShape<DK, DV, FP8>;
    const int n = threadIdx.x & 15;
    auto kraw = [&](int sb, int s) -> u32x4_t {
        const int row = 16 * sb + n;
        return *(lds_u32x4_t*)(kst + row * S::KROW + 16 * S::kswz(row, 4 * s + j));
    };
    // k-step outer: one Q^T operand per k-step serves both row blocks (each
    // block's accumulation still runs over the k-steps in order)
    #pragma unroll
    for (int k = 0; k < CB; ++k) st[k][0] = st[k][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) {
        bf16x8_t q[CB];
        #pragma unroll
        for (int k = 0; k < CB; ++k) q[k] = qop(k, ks);
        #pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            u32x4_t kw;
            if constexpr (FP8) {
                const u32x4_t raw = kraw(sb, ks / S::SPL);
                const uint32_t w0 = (ks % S::SPL) ? raw.z : raw.x;
                const uint32_t w1 = (ks % S::SPL) ? raw.w : raw.y;
                kw = u32x4_t{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                             fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1)};
            } else {
                kw = kraw(sb, ks);
            }
            #pragma unroll
            for (int k = 0; k < CB; ++k)
                st[k][sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kw), q[k], st[k][sb], 0, 0, 0);
        }
    }
}

// Online-softmax update and P.V for one tile whose first `valid` tokens are
// real for this lane's column (the rest are masked out).  With MQ a column
// may have no real token yet (its causal limit lies beyond the tile): its
// maximum stays -inf and it accumulates nothing.
template <int DK, int DV, bool FP8, bool MQ>
__device__ inline void tile_update(const VTile<DK, DV, FP8>& T, const f32x4_t (&st)[2], f32x4_t* O,
                                   float& m2, float& lsum, int valid, float scale_log2, int j) {
    using S = DecodeShape<DK, DV, FP8>;
    // online softmax (log2 domain); lane (n, j) holds head n, tile tokens
    // 16*sb + 4*j + r
    float p[8];
    float mx = -INFINITY;
    #pragma unroll
    for (int sb = 0; sb < 2; ++sb)
        #pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = 16 * sb + 4 * j + r < valid ? st[sb][r] * scale_log2 : -INFINITY;
            p[sb * 4 + r] = v;
            mx = fmaxf(mx, v);
        }
    mx = wave_max_xor_16_32(mx);
    const float mnew = fmaxf(m2, mx);
    // an empty column (mnew = -inf) subtracts 0: alpha and p become 0
    const float msub = (MQ && mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m2 - msub);
    m2 = mnew;
    float psum = 0.f;
    #pragma unroll
    for (int i = 0; i < 8; ++i) {
        p[i] = __builtin_amdgcn_exp2f(p[i] - msub);
        psum += p[i];
    }
    lsum = lsum * alpha + psum;
    #pragma unroll
    for (int c = 0; c < S::CPL; ++c) O[c] *= alpha;
    const u32x4_t pw = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                        pack_bf16(p[6], p[7])};
    const bf16x8_t pop = as_bf16x8(pw);

    // O^T += V^T . P^T, one MFMA per d-row block c (d = CPL*m + c)
    if constexpr (!FP8) {
        #pragma unroll
        for (int c = 0; c < S::CPL; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t av;
            #pragma unroll
            for (int u = 0; u < 4; ++u)
                av[u] = __builtin_amdgcn_perm(T.vr[2 * u + 1][c >> 1], T.vr[2 * u][c >> 1], sel);
            O[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), pop, O[c], 0, 0, 0);
        }
    } else {
        #pragma unroll
        for (int c = 0; c < S::CPL; c += 2) {
            const uint32_t sel = ((c & 3) == 0) ? 0x05010400u : 0x07030602u;
            u32x4_t a0, a1;
            #pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t lo_w, hi_w;
                if constexpr (S::CPL == 8) {
                    lo_w = T.vr[2 * u][c >> 2];
                    hi_w = T.vr[2 * u + 1][c >> 2];
                } else {
                    lo_w = T.vr[2 * u];
                    hi_w = T.vr[2 * u + 1];
                }
                const uint32_t x = __builtin_amdgcn_perm(hi_w, lo_w, sel);
                a0[u] = fp8x2_to_bf16x2<false>(x);
                a1[u] = fp8x2_to_bf16x2<true>(x);
            }
            O[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), pop, O[c], 0, 0, 0);
            O[c + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), pop, O[c + 1], 0, 0, 0);
        }
    }
}

// LDS of a decode kernel that builds its own metadata, after the waves'
// regions: the page, token and tile prefixes of the batch ([B + 1] int32
// each), the scan's wave totals and one flag word.
__host__ __device__ inline size_t md_prefix_bytes(int32_t B) { return ((3 * ((size_t)B + 1) * 4 + 7) / 8) * 8; }
__host__ __device__ inline size_t md_lds_bytes(int32_t B) { return md_prefix_bytes(B) + 3 * 8 * 8 + 8; }

// Per-request prefixes of a decode batch, built by the whole workgroup into
// LDS from the clamped lengths (the same clamping and sums as the metadata
// kernel, so the partition and every page id agree with it): sP = pages
// (kv_indptr), sF = tokens, sT = decode tiles, each [B + 1] from 0.  Returns
// the tile total and the OR of the clamping flags in every thread.
__device__ inline void md_prefixes(const MetaArgs& m, uint8_t* base, int64_t& W, int32_t& flags_out) {
    int32_t* const sP = (int32_t*)base;
    int32_t* const sF = sP + (m.B + 1);
    int32_t* const sT = sF + (m.B + 1);
    int64_t* const wsum = (int64_t*)(base + md_prefix_bytes(m.B));  // [3][8]
    int32_t* const sflag = (int32_t*)(wsum + 24);
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, nw = blockDim.x >> 6;
    if (t == 0) {
        sP[0] = sF[0] = sT[0] = 0;
        *sflag = 0;
    }
    int64_t carry[3] = {0, 0, 0};
    int32_t flags = 0;
    for (int32_t b0 = 0; b0 < m.B; b0 += blockDim.x) {
        const int32_t b = b0 + t;
        int64_t x[3] = {0, 0, 0};  // pages, tokens, tiles
        if (b < m.B) {
            int64_t L = m.seq_lens[b], n = 1, pages = 0;
            flags |= md_clamp_request(L, n, pages, m.page_shift, m.pt_cols);
            x[0] = pages;
            x[1] = L;
            x[2] = (L + DEC_TILE - 1) / DEC_TILE;
        }
        #pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            int64_t y[3];
            #pragma unroll
            for (int v = 0; v < 3; ++v) y[v] = __shfl_up(x[v], off);
            if (lane >= off) {
                #pragma unroll
                for (int v = 0; v < 3; ++v) x[v] += y[v];
            }
        }
        if (lane == 63) {
            #pragma unroll
            for (int v = 0; v < 3; ++v) wsum[8 * v + wv] = x[v];
        }
        __syncthreads();
        int64_t before[3] = {carry[0], carry[1], carry[2]};
        for (int k = 0; k < nw; ++k) {
            #pragma unroll
            for (int v = 0; v < 3; ++v) {
                const int64_t s = wsum[8 * v + k];
                if (k < wv) before[v] += s;
                carry[v] += s;
            }
        }
        if (b < m.B) {
            const int64_t cp = before[0] + x[0], cL = before[1] + x[1], cT = before[2] + x[2];
            if (cp > m.max_kv_pages || cL > INT32_MAX) flags |= PKA_DEV_CAPACITY;
            sP[b + 1] = (int32_t)min(cp, (int64_t)INT32_MAX);
            sF[b + 1] = (int32_t)min(cL, (int64_t)INT32_MAX);
            sT[b + 1] = (int32_t)min(cT, (int64_t)INT32_MAX);
        }
        __syncthreads();  // the wave totals are rewritten next round
    }
    if (flags) atomicOr(sflag, flags);
    __syncthreads();
    flags_out = *sflag;
    W = min(carry[2], (int64_t)INT32_MAX);
}

// Batches of at most 64 requests: every wave builds the prefixes itself in
// registers, lane b holding the sums through request b (inclusive), so
// neither LDS nor a barrier is needed.  `flags` is the OR of the clamping
// flags over the batch.
struct MdWave {
    int32_t P, F, T;  // pages, tokens, tiles through request `lane`
};
__device__ inline MdWave md_prefixes_wave(const MetaArgs& m, int32_t& flags_out) {
    const int lane = threadIdx.x & 63;
    int64_t L = 0, n = 1, pages = 0;
    int32_t flags = 0;
    if (lane < m.B) {
        L = m.seq_lens[lane];
        flags = md_clamp_request(L, n, pages, m.page_shift, m.pt_cols);
    }
    int64_t x[3] = {pages, L, (L + DEC_TILE - 1) / DEC_TILE};
    #pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int64_t y[3];
        #pragma unroll
        for (int v = 0; v < 3; ++v) y[v] = __shfl_up(x[v], off);
        if (lane >= off) {
            #pragma unroll
            for (int v = 0; v < 3; ++v) x[v] += y[v];
        }
    }
    if (lane < m.B && (x[0] > m.max_kv_pages || x[1] > INT32_MAX)) flags |= PKA_DEV_CAPACITY;
    int32_t all = 0;
    #pragma unroll
    for (int bit = 1; bit <= PKA_DEV_CAPACITY; bit <<= 1)
        if (__ballot((flags & bit) != 0)) all |= bit;
    flags_out = __builtin_amdgcn_readfirstlane(all);
    MdWave r;
    r.P = (int32_t)min(x[0], (int64_t)INT32_MAX);
    r.F = (int32_t)min(x[1], (int64_t)INT32_MAX);
    r.T = (int32_t)min(x[2], (int64_t)INT32_MAX);
    return r;
}

// The plan's partition and status words of a batch built in-kernel.
__device__ inline void md_write_plan_words(const MetaArgs& m, int64_t W, int32_t flags) {
    const int lane = threadIdx.x & 63;
    for (int i = lane; i < MD_SLOTS; i += 64) m.plan[PLAN_MDST + i] = i == 0 ? flags : 0;
    if (lane == 0) {
        int64_t q, r;
        decode_shares(W, m.nwg, q, r);
        m.plan[PLAN_STATUS] = 0;
        m.plan[PLAN_SHARE] = (int32_t)q;
        m.plan[PLAN_SHARE_REM] = (int32_t)r;
        m.plan[PLAN_TOTAL] = (int32_t)W;
        m.plan[PLAN_NWG] = m.nwg;
        m.plan[PLAN_EXT_COUNT] = 0;
        m.plan[PLAN_EXT_TQ] = m.ext_tq;
    }
}

// The batch-wide metadata outputs, written by one wave: kv_indptr, qo_indptr
// (request b's query row is b), kv_last_page_len, the plan's prefixes, and
// the partition and status words (clamping flags; the per-share page flags
// are written by the shares).  From the workgroup's LDS prefixes ...
__device__ inline void md_write_batch(const MetaArgs& m, const uint8_t* base, int64_t W, int32_t flags) {
    const int32_t* const sP = (const int32_t*)base;
    const int32_t* const sF = sP + (m.B + 1);
    const int32_t* const sT = sF + (m.B + 1);
    int32_t* const F = m.plan + plan_seg_prefix(m.B);
    int32_t* const T = m.plan + plan_tile_prefix(m.B);
    const int lane = threadIdx.x & 63;
    for (int32_t b = lane; b <= m.B; b += 64) {
        m.kv_indptr[b] = sP[b];
        m.qo_indptr[b] = b;
        F[b] = sF[b];
        T[b] = sT[b];
        if (b < m.B) {
            const int32_t L = sF[b + 1] - sF[b], pages = sP[b + 1] - sP[b];
            m.kv_last_page_len[b] = L - ((pages - 1) << m.page_shift);
        }
    }
    md_write_plan_words(m, W, flags);
}
// ... or from the wave's register prefixes (at most 64 requests)
__device__ inline void md_write_batch(const MetaArgs& m, const MdWave& r, int64_t W, int32_t flags) {
    int32_t* const F = m.plan + plan_seg_prefix(m.B);
    int32_t* const T = m.plan + plan_tile_prefix(m.B);
    const int lane = threadIdx.x & 63;
    // every lane takes part in the shuffles (a lane reading an inactive one gets nothing)
    const int32_t Fu = __shfl_up(r.F, 1), Pu = __shfl_up(r.P, 1);
    const int32_t F0 = lane ? Fu : 0, P0 = lane ? Pu : 0;
    if (lane == 0) {
        m.kv_indptr[0] = m.qo_indptr[0] = 0;
        F[0] = T[0] = 0;
    }
    if (lane < m.B) {
        m.kv_indptr[lane + 1] = r.P;
        m.qo_indptr[lane + 1] = lane + 1;
        F[lane + 1] = r.F;
        T[lane + 1] = r.T;
        m.kv_last_page_len[lane] = (r.F - F0) - ((r.P - P0 - 1) << m.page_shift);
    }
    md_write_plan_words(m, W, flags);
}

typedef __attribute__((address_space(3))) const int32_t lds_i32_t;

// MQ: several query tokens per request (speculative verify on the decode
// path).  Columns are then (query token i, head h) pairs of the request, in
// blocks of 16; a pass of the wave over its share takes CB adjacent blocks
// (CB = 2: one K operand read and one set of V registers serve both, their
// queries read from LDS at every tile); token i of a request with n query
// tokens sits at position L - n + i and sees keys 0 .. L - n + i.  Partials
// of token i go to slot (b + w) * qslots + i.
//
// MD: the kernel builds the batch's metadata itself (decode batches of at
// most DEC_MD_MAX_B requests, m set).  Every wave scans the lengths itself in
// registers (up to 64 requests), or every workgroup into LDS (more), and the
// waves read page ids straight from the page table.  As the waves exit, wave
// 0 of workgroup 0 writes the batch-wide arrays and the wave of each share
// that serves unit 0 the share's first request and its page flags;
// kv_indices and the new tokens' slots are left to the merge, so no store
// waits in the tile stream (stores count in vmcnt like loads).  The
// partition and the page ids are those the metadata kernel would produce,
// so the outputs are bit-identical to running it first.
template <int DK, int DV, bool FP8, bool MQ, bool MD, int CB = 1>
__global__ __launch_bounds__(512) void decode_mfma_kernel(AttnArgs a, MetaArgs m) {
    static_assert(!(MQ && MD), "metadata is built in-kernel for one query per request only");
    static_assert(CB == 1 || MQ, "several column blocks per wave only for several query rows");
    using S = DecodeShape<DK, DV, FP8>;
    constexpr int WLDS = decode_wave_lds<DK, DV, FP8>(CB);  // this wave's LDS bytes
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, j = lane >> 4;
    // a workgroup holds a.spw shares of wpb waves (one KV-head unit each)
    const int waves = blockDim.x >> 6;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = waves / a.spw;
    const int unit = blockIdx.y * wpb + wv % wpb;
    // unit = (KV head g, group of up to 16 of its query heads, column split
    // ps): with MQ the csplit waves of one head group take its passes of
    // 16 * CB columns in turn (pass k goes to wave k % csplit), side by side
    // in one workgroup, so they read the same tiles at the same time
    const int ps = unit % a.csplit, uh = unit / a.csplit;
    const int g = uh / a.qgroups;
    const int h0 = g * a.G + (uh % a.qgroups) * 16;
    const int nh = min(16, a.G - (uh % a.qgroups) * 16);

    // this wave's LDS: the K tile, then the queries of the next unit; after
    // the waves' regions, one progress word per wave
    extern __shared__ __attribute__((aligned(1024))) uint8_t dec_lds[];
    uint8_t* const kst = dec_lds + wv * WLDS;
    uint8_t* const qbuf = kst + S::KTILE;  // column block k's queries at qbuf + k * KSTEPS KB
    int32_t* const prog = (int32_t*)(dec_lds + waves * WLDS);
    // Waves wv and wv ^ 4 of an 8-wave workgroup share a SIMD, and the one
    // with the higher priority gets the larger part of the memory pipeline
    // (equal priorities favour the older wave, ~8% on the Llama-shaped
    // batch).  Partners serve about the same number of tiles (the same share,
    // or shares one tile apart), so each step the wave that is behind its
    // partner, or level with it and younger, takes the higher priority; the
    // pair then ends together.  The words are read without synchronisation:
    // a stale value only shifts a priority.
    const bool pair = waves == 8;
    int32_t nst = 0;  // tiles computed so far
    if (pair) __hip_atomic_store(prog + wv, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // MD: the metadata area, 8-byte aligned after the progress words
    uint8_t* const md_lds = dec_lds + ((waves * (WLDS + 4) + 7) & ~7);
    // MD: prefixes in registers (at most 64 requests) or in LDS
    const bool md_reg = MD && a.B <= 64;
    int64_t W_md = 0;
    int32_t len_flags = 0;
    MdWave mw{};
    if constexpr (MD) {
        if (md_reg) {
            mw = md_prefixes_wave(m, len_flags);
            W_md = __builtin_amdgcn_readlane(mw.T, a.B - 1);
        } else {
            md_prefixes(m, md_lds, W_md, len_flags);
        }
    }
    lds_i32_t* const sF = (lds_i32_t*)md_lds + (a.B + 1);  // MD, LDS path: token and tile prefixes
    lds_i32_t* const sT = sF + (a.B + 1);
    if (g >= a.Hkv) return;

    const int32_t* plan = a.plan;
    const int32_t w = blockIdx.x * a.spw + wv / wpb;
    const int32_t nwg = MD ? a.nwg : plan[PLAN_NWG];
    if (w >= nwg) return;
    // this wave's share: tiles [start, end) of the requests' tiles laid end
    // to end
    int64_t shq, shr, W;
    if constexpr (MD) {
        W = W_md;
        decode_shares(W, nwg, shq, shr);
    } else {
        shq = plan[PLAN_SHARE];
        shr = plan[PLAN_SHARE_REM];
        W = plan[PLAN_TOTAL];
    }
    const int64_t start = share_start(w, shq, shr);
    // MD: the wave of unit 0 records its share (first request, page flags)
    // and wave 0 of workgroup 0 the batch-wide arrays, as each wave leaves:
    // nothing in this launch reads them, and a store issued earlier would
    // hold up the next vmcnt wait for a tile
    const bool md_rec = MD && unit == 0;
    int32_t pflags = 0;  // MD: a page id outside the pool was clamped
    int32_t seg;
    auto md_close = [&]() {
        if (md_rec) {
            const bool bad = __ballot(pflags != 0) != 0;
            if (lane == 0) {
                m.plan[plan_share_flags(a.B) + w] = bad ? PKA_DEV_BAD_PAGE : 0;
                m.plan[plan_wg_seg(a.B) + w] = start < W ? seg : a.B;
            }
        }
        if (MD && blockIdx.x == 0 && blockIdx.y == 0 && wv == 0) {
            if (md_reg) md_write_batch(m, mw, W, len_flags);
            else md_write_batch(m, md_lds, W, len_flags);
        }
    };
    if constexpr (MD) {
        seg = a.B;
        if (start < W && md_reg) {
            // largest b with T[b] <= start: T[0] = 0, T[b] = lane b - 1's sum
            seg = __builtin_popcountll(__ballot(lane < a.B - 1 && mw.T <= start));
        } else if (start < W) {
            int32_t lo = 0, hi = a.B - 1;  // largest b with T[b] <= start
            while (lo < hi) {
                const int32_t mid = (lo + hi + 1) >> 1;
                if (__builtin_amdgcn_readfirstlane(sT[mid]) <= start) lo = mid; else hi = mid - 1;
            }
            seg = lo;
        }
    }
    if (start >= W) {
        md_close();
        return;
    }
    const int64_t end = min(share_start(w + 1, shq, shr), W);
    const int32_t* F = plan + plan_seg_prefix(a.B);
    const int32_t* T = plan + plan_tile_prefix(a.B);
    if constexpr (!MD) seg = plan[plan_wg_seg(a.B) + w];
    // request prefixes: tokens F, tiles T
    auto Fat = [&](int32_t i) -> int32_t {
        if constexpr (MD) return md_reg ? (i ? __builtin_amdgcn_readlane(mw.F, i - 1) : 0)
                                        : __builtin_amdgcn_readfirstlane(sF[i]);
        else return load_uniform(F, i);
    };
    auto Tat = [&](int32_t i) -> int32_t {
        if constexpr (MD) return md_reg ? (i ? __builtin_amdgcn_readlane(mw.T, i - 1) : 0)
                                        : __builtin_amdgcn_readfirstlane(sT[i]);
        else return load_uniform(T, i);
    };
    const int32_t P = 1 << a.page_shift;

    // one pool slot, all KV heads
    const int64_t krow = (int64_t)a.Hkv * DK * S::ESZ, vrow = (int64_t)a.Hkv * DV * S::ESZ;
    const uint8_t* kbase = (const uint8_t*)a.k_pool + (int64_t)g * DK * S::ESZ;
    const uint8_t* vbase = (const uint8_t*)a.v_pool + (int64_t)g * DV * S::ESZ;
    const int tok = lane & 31;  // tile token whose slot this lane looks up

    // The wave's work is one stream of 32-position tiles.  A unit is one
    // pass of 16 * CB columns over one piece (the part of a request inside this
    // wave's tile share); units follow each other in request order, and
    // the loads of a unit's first tile and its queries go out while the
    // previous unit's last tile is computed, so a request boundary costs no
    // extra round trip to memory.
    // Iterator state is kept small (wave-uniform scalars): the piece's
    // request, token range, pass and page offset, and the tile start; the
    // request's query rows are read again where they are needed.
    struct It {
        int32_t seg;  // request; a.B: past the end of the share
        int32_t lo, hi, c0, pb, t0;
    };
    // query rows of request sg: one (its last row) without MQ
    struct Rows {
        int32_t L, q0, nq, pfx;
    };
    auto rows_of = [&](int32_t sg) {
        Rows r;
        r.L = Fat(sg + 1) - Fat(sg);
        if constexpr (MD) {
            r.q0 = sg;
            r.nq = 1;
            r.pfx = r.L - 1;
        } else if constexpr (MQ) {
            r.q0 = load_uniform(a.qo_indptr, sg);
            const int32_t nb = load_uniform(a.qo_indptr, sg + 1) - r.q0;
            r.nq = min(nb, a.qslots);
            r.pfx = r.L - nb;
        } else {
            r.q0 = min(max(load_uniform(a.qo_indptr, sg + 1) - 1, 0), a.N - 1);
            r.nq = 1;
            r.pfx = r.L - 1;
        }
        return r;
    };
    // first non-empty piece from request sg on (seg = a.B: the share is done)
    auto open_piece = [&](int32_t sg, It& it) {
        for (; sg < a.B; ++sg) {
            const int32_t t0 = Tat(sg), t1 = Tat(sg + 1);
            if (t0 >= end) break;
            // token range of the piece: whole tiles, up to the request's end
            const int32_t L = Fat(sg + 1) - Fat(sg);
            const int32_t lo = (int32_t)(max(start, (int64_t)t0) - t0) * DEC_TILE;
            const int32_t hi = end >= t1 ? L : (int32_t)(end - t0) * DEC_TILE;
            if (hi <= lo) continue;
            if constexpr (MQ) {
                const int32_t nb = load_uniform(a.qo_indptr, sg + 1) - load_uniform(a.qo_indptr, sg);
                // (every lane: a lane condition inside this loop would make
                // the compiler keep the whole iterator in vector registers)
                if (nb > a.qslots && lo == 0 && unit == 0)
                    atomicOr((int32_t*)a.plan + PLAN_STATUS, PKA_DEV_BAD_LENGTH);
                // no query rows, or none in this wave's passes
                if (16 * CB * ps >= min(nb, a.qslots) * nh) continue;
            }
            it.seg = sg;
            it.lo = lo;
            it.hi = hi;
            it.c0 = 16 * CB * ps;
            it.pb = MD ? 0 : load_uniform(a.kv_indptr, sg);  // MD reads the page table instead
            it.t0 = lo;
            return;
        }
        it.seg = a.B;
    };
    // the tile after `cur`: the next 32 positions, else the next pass, else
    // the next piece
    auto advance = [&](const It& cur, It& nx) {
        nx = cur;
        if (cur.seg >= a.B) return;
        nx.t0 = cur.t0 + DEC_TILE;
        if (nx.t0 < cur.hi) return;
        if (MQ && cur.c0 + 16 * CB * a.csplit < rows_of(cur.seg).nq * nh) {
            nx.c0 = cur.c0 + 16 * CB * a.csplit;
            nx.t0 = cur.lo;
        } else {
            open_piece(cur.seg + 1, nx);
        }
    };
    // Pool slot of tile token `tok`; positions past the piece repeat its last
    // token (loaded, never counted).  In two halves: page_id loads the page
    // id (MD: from the page table; else from kv_indices, the index clamped
    // into it), and slot_from clamps it into the pool (MD: flagging an id
    // outside it) and adds the offset in the page.  The id of the tile after
    // next is loaded a step ahead and used only after the next step's wait:
    // loads complete in order, so a use right after the load would wait for
    // the tile loads issued before it as well.
    auto page_id = [&](const It& it) -> int32_t {
        const int32_t pos = it.t0 + tok;
        const int32_t pc = pos < it.hi ? pos : it.hi - 1;
        if constexpr (MD) {
            return m.page_table[(int64_t)it.seg * m.pt_stride + (pc >> a.page_shift)];
        } else {
            int64_t idx = (int64_t)it.pb + (pc >> a.page_shift);
            idx = idx < a.kv_cap ? idx : a.kv_cap - 1;
            return a.kv_indices[idx];
        }
    };
    auto slot_from = [&](const It& it, int32_t pg) {
        const int32_t pos = it.t0 + tok;
        const int32_t pc = pos < it.hi ? pos : it.hi - 1;
        if (pg < 0 || pg >= a.num_pages) {
            if constexpr (MD) pflags = 1;
            pg = min(max(pg, 0), a.num_pages - 1);
        }
        return (pg << a.page_shift) | (pc & (P - 1));
    };
    // this lane's column of a unit: query token qi, head h
    struct Col {
        bool ok;
        int32_t qi, h, qr, kend;  // keys of the column within the piece: positions < kend
    };
    auto column = [&](const It& u, const Rows& r, int k) {
        Col c;
        const int32_t cc = u.c0 + 16 * k + n;
        c.ok = MQ ? cc < r.nq * nh : n < nh;
        c.qi = MQ ? (c.ok ? cc / nh : 0) : 0;
        c.h = h0 + (MQ ? cc % nh : n);
        c.qr = r.q0 + c.qi;
        c.kend = MQ ? min(u.hi, r.pfx + c.qi + 1) : u.hi;
        return c;
    };
    // Q^T operand: lane (n, j) holds its column at the dims its K lanes load.
    // A unit's queries go to the wave's LDS buffer by direct loads (lane l's
    // 16 bytes of k-step ks at 1024 ks + 16 l) when its first tile is issued,
    // and into registers once that tile has landed; lanes without a column
    // load nothing and take zeros.
    auto fetch_q = [&](const It& u) {
        const Rows r = rows_of(u.seg);
        #pragma unroll
        for (int k = 0; k < CB; ++k) {
            const Col c = column(u, r, k);
            if (c.ok) {
                const __bf16* qrow = (const __bf16*)a.q + ((int64_t)c.qr * a.Hq + c.h) * DK;
                #pragma unroll
                for (int ks = 0; ks < S::KSTEPS; ++ks) {
                    const int d0 = (ks / S::SPL) * 4 * S::KE + j * S::KE + (ks % S::SPL) * 8;
                    lds_dma16(qrow + d0, qbuf + 1024 * (k * S::KSTEPS + ks));
                }
            }
        }
    };
    // The wave whose tile holds a request's last position writes the new
    // token just before that tile's loads go out.  For 128-wide heads the row
    // and the slot are read with the loads of the tile before (prep_new_token,
    // waited for with them), so the store waits for nothing unless the tile
    // is the wave's first; for the other widths they are read when the store
    // is due, as holding them across a step would cost occupancy or spill
    // registers.
    constexpr bool EARLY = DK == 128;
    struct NewTok {
        u32x4_t w;
        int32_t slot;
        bool on;
    };
    auto prep_new_token = [&](const It& u, NewTok& t) {
        t.on = false;
        if constexpr (MD || !MQ) {
            if (!a.k_new || u.seg >= a.B || u.t0 + DEC_TILE < u.hi) return;
            const Rows r = rows_of(u.seg);
            if (u.hi != r.L) return;
            t.on = true;
            t.w = load_new_token<DK, DV>(a, r.q0, g, lane);
            if constexpr (MD) {
                const int32_t pos = r.L - 1;
                int32_t pg = load_uniform(m.page_table, (int64_t)u.seg * m.pt_stride + (pos >> a.page_shift));
                pg = min(max(pg, 0), a.num_pages - 1);  // flagged where the tile reads it
                t.slot = (pg << a.page_shift) | (pos & (P - 1));
            } else {
                t.slot = a.out_cache_loc[r.q0];
            }
        }
    };

    It cur, nx, nn;
    open_piece(seg, cur);
    if (cur.seg >= a.B) {
        md_close();
        return;
    }
    NewTok nt;
    prep_new_token(cur, nt);
    if (nt.on) store_new_token<DK, DV, FP8>(a, nt.w, nt.slot, g, lane);
    VTile<DK, DV, FP8> A, Bt;
    {
        const int32_t s0 = slot_from(cur, page_id(cur));
        load_k<DK, DV, FP8>(kst, s0, kbase, krow);
        load_v(A, s0, vbase, vrow, n, j);
    }
    fetch_q(cur);
    advance(cur, nx);
    int32_t id_nx = nx.seg < a.B ? page_id(nx) : 0;  // tile nx's page id, turned into its slot in the step
    if constexpr (EARLY) prep_new_token(nx, nt);
    Rows crow = rows_of(cur.seg);  // query rows of cur's request
    Col col[CB];
    #pragma unroll
    for (int k = 0; k < CB; ++k) col[k] = column(cur, crow, k);
    // The Q^T operand of the unit: held in registers from its first tile on
    // (128-wide keys and less), or read from the LDS buffer at every tile
    // (192-wide keys: six k-steps would take 24 more registers and push the
    // kernel into spills).  Either way the reads of the buffer are done
    // before the next unit's queries are loaded into it, which happens after
    // the scores of the unit's last tile.  Two column blocks per wave read
    // both from LDS (two register sets would spill).
    constexpr bool QLDS = DK > 128 || CB > 1;
    bf16x8_t qreg[QLDS ? 1 : S::KSTEPS];
    auto q_lds = [&](int k, int ks) {
        const u32x4_t v = *(lds_u32x4_t*)(qbuf + 1024 * (k * S::KSTEPS + ks) + 16 * lane);
        return as_bf16x8(col[k].ok ? v : u32x4_t{0u, 0u, 0u, 0u});
    };
    auto qop = [&](int k, int ks) {
        if constexpr (QLDS) return q_lds(k, ks);
        else return qreg[ks];
    };
    auto take_q = [&]() {
        if constexpr (!QLDS) {
            #pragma unroll
            for (int ks = 0; ks < S::KSTEPS; ++ks) qreg[ks] = q_lds(0, ks);
            // the reads are done before a later direct load refills the buffer
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
            asm volatile("" ::: "memory");
        }
    };
    f32x4_t O[CB][S::CPL];
    float m2[CB], lsum[CB];
    auto reset = [&]() {
        #pragma unroll
        for (int k = 0; k < CB; ++k) {
            #pragma unroll
            for (int cc = 0; cc < S::CPL; ++cc) O[k][cc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            m2[k] = -INFINITY;
            lsum[k] = 0.f;
        }
    };
    reset();

    // finish a unit's column block k: denominator over the four lane groups
    // of each column; a column with no key in this piece leaves weight 0
    // (lse -inf, o 0)
    auto finish_block = [&](const It& u, int k) {
        const Col& c = col[k];
        const float ltot = wave_sum_xor_16_32(lsum[k]);
        const float inv = MQ && !(ltot > 0.f) ? 0.f : 1.0f / ltot;
        const float lse_nat = MQ && !(ltot > 0.f) ? -INFINITY : (m2[k] + __builtin_amdgcn_logf(ltot)) * LN2;
        if (!c.ok) return;
        // the output row when the piece is the whole request, else the
        // partial row of (request, workgroup, query token); both bf16 (the
        // merge weighs the partials in fp32), the lse in fp32
        const bool whole = u.lo == 0 && u.hi == crow.L;
        const int64_t ps = ((int64_t)u.seg + w) * a.qslots + c.qi;
        __bf16* const orow = whole ? (__bf16*)a.out + ((int64_t)c.qr * a.Hq + c.h) * DV
                                   : (__bf16*)a.ws_o + (ps * a.Hq + c.h) * DV;
        emit_rows<DV>(O[k], inv * a.v_scale, j, [&](const float* v, int d0) {
            #pragma unroll
            for (int i = 0; i < 4 * S::CPL; i += 8) {
                const u32x4_t pk = {pack_bf16(v[i], v[i + 1]), pack_bf16(v[i + 2], v[i + 3]),
                                    pack_bf16(v[i + 4], v[i + 5]), pack_bf16(v[i + 6], v[i + 7])};
                *(u32x4_t*)(orow + d0 + i) = pk;
            }
        });
        if (j == 0) {
            if (!whole) a.ws_lse[ps * a.Hq + c.h] = lse_nat;
            else if (a.lse) a.lse[(int64_t)c.qr * a.Hq + c.h] = lse_nat;
        }
    };
    auto finish = [&](const It& u) {
        #pragma unroll
        for (int k = 0; k < CB; ++k) finish_block(u, k);
    };

    // One step: wait for tile `cur` (K in LDS, V in X); its scores; then,
    // once the scores' LDS reads are done, the loads of tile `nx` (K into
    // the same LDS tile, V into Y) and the slot lookups of the tile after
    // it; then cur's softmax and P.V.  Every tile's loads are waited for
    // before the next tile's go out, so one tile is in flight while
    // another is computed.
    auto step = [&](VTile<DK, DV, FP8>& X, VTile<DK, DV, FP8>& Y) -> bool {
        // vmcnt(0): tile cur, its queries and nx's new token landed.  With
        // lgkmcnt(0) as well (nothing of the scalar or LDS kind is pending
        // here), the compiler also knows the direct loads' LDS writes are
        // done; without it, it would make every LDS wait of the step a full
        // lgkmcnt(0).
        __builtin_amdgcn_s_waitcnt(0x0070);
        asm volatile("" ::: "memory");       // LDS reads stay after the wait
        if (cur.t0 == cur.lo) take_q();      // cur opens its unit
        int32_t other = 0;
        if (pair) {
            ++nst;
            __hip_atomic_store(prog + wv, nst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            other = __hip_atomic_load(prog + (wv ^ 4), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        f32x4_t st[CB][2];
        tile_scores<DK, DV, FP8, CB>(kst, qop, st, j);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the K reads are done ...
        asm volatile("" ::: "memory");       // ... before the direct loads refill the tile
        if (pair) {
            const int32_t o = __builtin_amdgcn_readfirstlane(other);
            if (o > nst || (o == nst && wv >= 4)) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }
        if (nx.seg < a.B) {
            const int32_t s_nx = slot_from(nx, id_nx);  // its id landed before this step's wait
            const bool opens = nx.t0 == nx.lo;  // nx is the first tile of its unit
            if constexpr (EARLY) {
                if (nt.on) store_new_token<DK, DV, FP8>(a, nt.w, nt.slot, g, lane);
            } else {
                NewTok t;
                prep_new_token(nx, t);
                if (t.on) store_new_token<DK, DV, FP8>(a, t.w, t.slot, g, lane);
            }
            load_k<DK, DV, FP8>(kst, s_nx, kbase, krow);
            load_v(Y, s_nx, vbase, vrow, n, j);
            if (opens) fetch_q(nx);
        }
        advance(nx, nn);
        const int32_t id_nn = nn.seg < a.B ? page_id(nn) : 0;
        if constexpr (EARLY) prep_new_token(nn, nt);
        #pragma unroll
        for (int k = 0; k < CB; ++k)
            tile_update<DK, DV, FP8, MQ>(X, st[k], O[k], m2[k], lsum[k], col[k].kend - cur.t0, a.scale_log2, j);
        if (cur.t0 + DEC_TILE >= cur.hi) {  // last tile of its unit
            finish(cur);
            if (nx.seg >= a.B) return false;
            if (nx.seg != cur.seg) crow = rows_of(nx.seg);
            #pragma unroll
            for (int k = 0; k < CB; ++k) col[k] = column(nx, crow, k);
            reset();
        }
        cur = nx;
        nx = nn;
        id_nx = id_nn;
        return true;
    };
    for (;;) {
        if (!step(A, Bt)) break;
        if (!step(Bt, A)) break;
    }
    md_close();
}

// fp32 cache: a plain VALU variant with the same work partition (lanes over
// head_dim, one token at a time, 16 columns per pass as in the MFMA variant;
// its launches have csplit 1).  Used for fp32 workloads.
template <int DK, int DV, bool MQ>
__global__ __launch_bounds__(256) void decode_f32_kernel(AttnArgs a) {
    constexpr int EPK = DK / 64, EPV = DV / 64;  // key and value dims per lane
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int wpb = (blockDim.x >> 6) / a.spw;
    const int unit = blockIdx.y * wpb + wv % wpb;
    const int g = unit / a.qgroups;
    const int h0 = g * a.G + (unit % a.qgroups) * 16;
    const int nh = min(16, a.G - (unit % a.qgroups) * 16);
    if (g >= a.Hkv) return;
    const int32_t* plan = a.plan;
    const int32_t w = blockIdx.x * a.spw + wv / wpb;
    if (w >= plan[PLAN_NWG]) return;
    const int64_t shq = plan[PLAN_SHARE], shr = plan[PLAN_SHARE_REM], W = plan[PLAN_TOTAL];  // in tiles
    const int64_t start = share_start(w, shq, shr);
    if (start >= W) return;
    const int64_t end = min(share_start(w + 1, shq, shr), W);
    const int32_t* F = plan + plan_seg_prefix(a.B);
    const int32_t* T = plan + plan_tile_prefix(a.B);
    const float scale2 = a.scale_log2;
    for (int32_t seg = plan[plan_wg_seg(a.B) + w]; seg < a.B; ++seg) {
        const int32_t t0 = T[seg], t1 = T[seg + 1];
        if (t0 >= end) break;
        const int32_t L = F[seg + 1] - F[seg];
        const int32_t lo = (int32_t)(max(start, (int64_t)t0) - t0) * DEC_TILE;
        const int32_t hi = end >= t1 ? L : (int32_t)(end - t0) * DEC_TILE;
        const int32_t b = seg, page_base = a.kv_indptr[b];
        int32_t q0, nq, pfx;
        if constexpr (MQ) {
            q0 = a.qo_indptr[b];
            const int32_t nb = a.qo_indptr[b + 1] - q0;
            nq = min(nb, a.qslots);
            if (nb > a.qslots && lo == 0 && lane == 0 && unit == 0)
                atomicOr((int32_t*)a.plan + PLAN_STATUS, PKA_DEV_BAD_LENGTH);
            pfx = L - nb;
        } else {
            q0 = min(max(a.qo_indptr[b + 1] - 1, 0), a.N - 1);
            nq = 1;
            pfx = L - 1;
        }
        const int32_t cols = nq * nh;
        for (int32_t c0 = 0; c0 < cols; c0 += 16) {
            const int ncol = min(16, cols - c0);
            float q[16][EPK], o[16][EPV], m[16], l[16];
            int32_t kend[16];
            #pragma unroll
            for (int cc = 0; cc < 16; ++cc) {
                m[cc] = -INFINITY;
                l[cc] = 0.f;
                const int32_t c = c0 + cc;
                const int32_t qi = cc < ncol ? c / nh : 0;
                kend[cc] = min(hi, pfx + qi + 1);
                #pragma unroll
                for (int e = 0; e < EPK; ++e)
                    q[cc][e] = cc < ncol ? ((const float*)a.q)[((int64_t)(q0 + qi) * a.Hq + h0 + c % nh) * DK + e * 64 + lane] : 0.f;
                #pragma unroll
                for (int e = 0; e < EPV; ++e) o[cc][e] = 0.f;
            }
            for (int32_t t = lo; t < hi; ++t) {
                const int64_t sg = (int64_t)slot_of(a, page_base, t) * a.Hkv + g;
                float k[EPK], v[EPV];
                #pragma unroll
                for (int e = 0; e < EPK; ++e) k[e] = ((const float*)a.k_pool)[sg * DK + e * 64 + lane];
                #pragma unroll
                for (int e = 0; e < EPV; ++e) v[e] = ((const float*)a.v_pool)[sg * DV + e * 64 + lane];
                #pragma unroll
                for (int cc = 0; cc < 16; ++cc) {
                    if (cc >= ncol || t >= kend[cc]) continue;
                    float dot = 0.f;
                    #pragma unroll
                    for (int e = 0; e < EPK; ++e) dot += q[cc][e] * k[e];
                    #pragma unroll
                    for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
                    const float sc = dot * scale2;
                    const float mn = fmaxf(m[cc], sc);
                    const float al = __builtin_amdgcn_exp2f(m[cc] - mn);
                    const float p = __builtin_amdgcn_exp2f(sc - mn);
                    m[cc] = mn;
                    l[cc] = l[cc] * al + p;
                    #pragma unroll
                    for (int e = 0; e < EPV; ++e) o[cc][e] = o[cc][e] * al + p * v[e];
                }
            }
            const bool full = lo == 0 && hi == L;
            #pragma unroll
            for (int cc = 0; cc < 16; ++cc) {
                if (cc >= ncol) continue;
                const int32_t c = c0 + cc, qi = c / nh, h = h0 + c % nh, qr = q0 + qi;
                // a column with no key in this piece leaves weight 0 (lse -inf, o 0)
                const bool empty = !(l[cc] > 0.f);
                const float inv = empty ? 0.f : 1.0f / l[cc];
                const float lse_nat = empty ? -INFINITY : (m[cc] + __builtin_amdgcn_logf(l[cc])) * LN2;
                if (full) {
                    #pragma unroll
                    for (int e = 0; e < EPV; ++e)
                        ((float*)a.out)[((int64_t)qr * a.Hq + h) * DV + e * 64 + lane] = o[cc][e] * inv;
                    if (a.lse && lane == 0) a.lse[(int64_t)qr * a.Hq + h] = lse_nat;
                } else {
                    const int64_t ps = ((int64_t)b + w) * a.qslots + qi;
                    #pragma unroll
                    for (int e = 0; e < EPV; ++e)
                        ((float*)a.ws_o)[(ps * a.Hq + h) * DV + e * 64 + lane] = o[cc][e] * inv;
                    if (lane == 0) a.ws_lse[ps * a.Hq + h] = lse_nat;
                }
            }
        }
    }
}

// Log-sum-exp merge of the partials of requests that were split across
// workgroups: out = sum_c e^(lse_c - M) o_c / sum_c e^(lse_c - M) and
// lse = M + ln(sum_c e^(lse_c - M)).  One wave per (request, head, query
// row; grid z = query rows): lanes first take one partial each (max and
// normaliser by wave reductions), then lanes take head dims and sweep the
// partials with several loads in flight.  D: the value (output) width.
// Dims of a row that lane `lane` reads and writes in the merge: EPL
// consecutive ones (lane * EPL + e) for bf16 rows, so a lane moves them in
// one access; e * 64 + lane for fp32 rows.
template <int EPL, bool BF>
__device__ inline int merge_dim(int lane, int e) { return BF ? lane * EPL + e : e * 64 + lane; }
// This lane's EPL values of one partial row, as fp32.
template <int EPL, bool BF>
__device__ inline void load_partial(const void* row, int lane, float (&v)[EPL]) {
    if constexpr (BF && EPL == 2) {
        const uint32_t w = ((const uint32_t*)row)[lane];
        v[0] = __uint_as_float(w << 16);
        v[1] = __uint_as_float(w & 0xffff0000u);
    } else if constexpr (BF) {
        static_assert(EPL == 1, "bf16 rows of 64 or 128 values");
        v[0] = __uint_as_float((uint32_t)((const uint16_t*)row)[lane] << 16);
    } else {
        #pragma unroll
        for (int e = 0; e < EPL; ++e) v[e] = ((const float*)row)[merge_dim<EPL, false>(lane, e)];
    }
}

template <int D, bool OUT_BF16>
__device__ inline void merge_column(const AttnArgs& a, int32_t b) {
    static_assert(D == 64 || D == 128, "value width");
    constexpr int EPL = D / 64;
    constexpr int UNROLL = 8;
    // partial rows in the output's type
    using PT = typename std::conditional<OUT_BF16, __bf16, float>::type;
    const int lane = threadIdx.x & 63;
    const int32_t h = blockIdx.y * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (h >= a.Hq) return;
    // The partition, the request's tile range and its query rows, read
    // together (one round trip; the wait below keeps the compiler from
    // issuing them one branch at a time).
    const int32_t* plan = a.plan;
    const int32_t* T = plan + plan_tile_prefix(a.B);
    const uint32_t shq = (uint32_t)load_uniform(plan, PLAN_SHARE);
    const uint32_t shr = (uint32_t)load_uniform(plan, PLAN_SHARE_REM);
    const int32_t t0 = load_uniform(T, b), t1 = load_uniform(T, b + 1);
    const int32_t qa = load_uniform(a.qo_indptr, b), qb = load_uniform(a.qo_indptr, b + 1);
    asm volatile("" ::"s"(shq), "s"(shr), "s"(t0), "s"(t1), "s"(qa), "s"(qb));
    if (t1 <= t0) return;
    // share_of in 32 bits: tile indices and both partition words fit, and
    // shr * (shq + 1) <= total tiles (shq >= DEC_MIN_SHARE)
    auto share32 = [&](uint32_t t) -> int32_t {
        const uint32_t big = shr * (shq + 1);
        return (int32_t)(t < big ? t / (shq + 1) : shr + (t - big) / shq);
    };
    const int32_t w0 = share32((uint32_t)t0), w1 = share32((uint32_t)(t1 - 1));
    if (w0 == w1) return;  // written directly by its only workgroup
    const int32_t np = w1 - w0 + 1;
    // query rows of the request (one without multi-query partials)
    int32_t q0, nq;
    if (a.qslots > 1) {
        q0 = qa;
        nq = min(qb - qa, a.qslots);
    } else {
        q0 = min(max(qb - 1, 0), a.N - 1);
        nq = 1;
    }
    const int64_t lstride = (int64_t)a.qslots * a.Hq;  // per partial
    const int64_t ostride = lstride * D;
    const int32_t qi = blockIdx.z;
    if (qi >= nq) return;
    {
        const float* lse_col = a.ws_lse + ((int64_t)(b + w0) * a.qslots + qi) * a.Hq + h;
        const PT* o_col = (const PT*)a.ws_o + (((int64_t)(b + w0) * a.qslots + qi) * a.Hq + h) * D;

        float M = -INFINITY;
        float den = 0.f, acc[EPL];
        #pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
        if (np <= UNROLL) {
            // few partials: their outputs are loaded together with the
            // log-sum-exps (one round trip), then weighted
            const float lv = lane < np ? lse_col[(int64_t)lane * lstride] : -INFINITY;
            float v[UNROLL][EPL];
            #pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                load_partial<EPL, OUT_BF16>(o_col + (int64_t)min(u, np - 1) * ostride, lane, v[u]);
            M = lv;
            #pragma unroll
            for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
            const float wk = lane < np ? expf(lv - M) : 0.f;
            den = wk;
            #pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const float wt = u < np ? __shfl(wk, u) : 0.f;
                #pragma unroll
                for (int e = 0; e < EPL; ++e) acc[e] += wt * v[u][e];
            }
        } else {
            for (int32_t k = lane; k < np; k += 64) M = fmaxf(M, lse_col[(int64_t)k * lstride]);
            #pragma unroll
            for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
            for (int32_t k0 = 0; k0 < np; k0 += 64) {
                const int32_t k = k0 + lane;
                const float wk = k < np ? expf(lse_col[(int64_t)k * lstride] - M) : 0.f;
                den += wk;
                const int32_t cnt = min(64, np - k0);
                for (int32_t i = 0; i < cnt; i += UNROLL) {
                    float v[UNROLL][EPL], wt[UNROLL];
                    #pragma unroll
                    for (int u = 0; u < UNROLL; ++u) {
                        const int32_t kk = min(i + u, cnt - 1);
                        wt[u] = i + u < cnt ? __shfl(wk, kk) : 0.f;
                        load_partial<EPL, OUT_BF16>(o_col + (int64_t)(k0 + kk) * ostride, lane, v[u]);
                    }
                    #pragma unroll
                    for (int u = 0; u < UNROLL; ++u)
                        #pragma unroll
                        for (int e = 0; e < EPL; ++e) acc[e] += wt[u] * v[u][e];
                }
            }
        }
        #pragma unroll
        for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
        const float inv = 1.0f / den;
        const int32_t qr = q0 + qi;
        const int64_t orow = ((int64_t)qr * a.Hq + h) * D;
        if constexpr (OUT_BF16 && EPL == 2) {
            ((uint32_t*)((__bf16*)a.out + orow))[lane] = pack_bf16(acc[0] * inv, acc[1] * inv);
        } else {
            #pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int64_t o = orow + merge_dim<EPL, OUT_BF16>(lane, e);
                if constexpr (OUT_BF16)
                    ((__bf16*)a.out)[o] = (__bf16)(acc[e] * inv);
                else
                    ((float*)a.out)[o] = acc[e] * inv;
            }
        }
        if (a.lse && lane == 0) a.lse[(int64_t)qr * a.Hq + h] = M + logf(den);
    }
}

// MD: the decode kernel built the metadata in-kernel; the merge writes what
// it left out: kv_indices and the request's new-token slot in out_cache_loc.
// The grid has MERGE_GATHER_WGS more workgroups per request (grid y beyond
// the merging ones) that only copy equal slices of the request's page ids
// from the page table, clamped into the pool as the decode kernel read them,
// so the copy runs beside the merge instead of inside its workgroups.
constexpr int MERGE_GATHER_WGS = 16;
template <int D, bool OUT_BF16, bool MD>
__global__ __launch_bounds__(256) void decode_merge_kernel(AttnArgs a, MetaArgs m) {
    const int32_t b = blockIdx.x;
    const int32_t ym = (a.Hq + 3) / 4;  // merging workgroups per request
    if (!MD || (int32_t)blockIdx.y < ym) {
        if (blockIdx.z < a.qslots) merge_column<D, OUT_BF16>(a, b);
        if constexpr (MD) {
            if (blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) {
                const int32_t p0 = a.kv_indptr[b], pl = a.kv_indptr[b + 1] - p0 - 1;  // page of position L - 1
                const int32_t last = a.kv_last_page_len[b];
                const int32_t pg = min(max(m.page_table[(int64_t)b * m.pt_stride + pl], 0), a.num_pages - 1);
                m.out_cache_loc[b] = (pg << a.page_shift) | (last - 1);
            }
        }
        return;
    }
    if constexpr (MD) {
        if (blockIdx.z != 0) return;
        const int32_t p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
        const int32_t* row = m.page_table + (int64_t)b * m.pt_stride;
        const int32_t chunk = (p1 - p0 + MERGE_GATHER_WGS - 1) / MERGE_GATHER_WGS;
        const int32_t i0 = p0 + (blockIdx.y - ym) * chunk, i1 = min(p1, i0 + chunk);
        // four ids per thread and round, all loaded before any is stored (a
        // store may alias the next load); every load is issued, indices past
        // the slice reading the request's last id, which is not stored
        constexpr int PER = 4;
        for (int32_t i = i0 + threadIdx.x; i < i1; i += PER * blockDim.x) {
            int32_t v[PER];
            #pragma unroll
            for (int k = 0; k < PER; ++k) v[k] = row[min(i + k * (int32_t)blockDim.x, p1 - 1) - p0];
            #pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int32_t j = i + k * blockDim.x;
                if (j < i1 && j < m.max_kv_pages) m.kv_indices[j] = min(max(v[k], 0), a.num_pages - 1);
            }
        }
    }
}

// Dynamic LDS of a decode workgroup of `waves` waves: their regions and one
// progress word each; with in-kernel metadata, the 8-byte aligned metadata
// area of a batch of B requests after them.
template <int DK, int DV, bool FP8>
size_t decode_lds_bytes(int waves, int cb = 1) {
    return (size_t)waves * (decode_wave_lds<DK, DV, FP8>(cb) + 4);
}
template <int DK, int DV, bool FP8>
size_t decode_md_lds_bytes(int waves, int32_t B) {
    if (B <= 64) return decode_lds_bytes<DK, DV, FP8>(waves);  // prefixes in registers
    return ((decode_lds_bytes<DK, DV, FP8>(waves) + 7) & ~(size_t)7) + md_lds_bytes(B);
}

// The merge after a decode launch (md: after the decode kernel that built
// the metadata; the merge then writes kv_indices and out_cache_loc).
template <int DV>
hipError_t launch_merge(pka_dtype q, const AttnArgs& a, const MetaArgs* md, hipStream_t s) {
    const dim3 mgrid(a.B, (a.Hq + 3) / 4 + (md ? MERGE_GATHER_WGS : 0), a.qslots);
    const MetaArgs none{};
    if (md && q == PKA_BF16)
        hipLaunchKernelGGL((decode_merge_kernel<DV, true, true>), mgrid, dim3(256), 0, s, a, *md);
    else if (md)
        hipLaunchKernelGGL((decode_merge_kernel<DV, false, true>), mgrid, dim3(256), 0, s, a, *md);
    else if (q == PKA_BF16)
        hipLaunchKernelGGL((decode_merge_kernel<DV, true, false>), mgrid, dim3(256), 0, s, a, none);
    else
        hipLaunchKernelGGL((decode_merge_kernel<DV, false, false>), mgrid, dim3(256), 0, s, a, none);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_decode_d(pka_dtype q, pka_dtype kv, const AttnArgs& a, int wpb, hipStream_t s) {
    const int units = a.Hkv * a.qgroups * a.csplit;
    const int waves = wpb * a.spw;
    const dim3 grid((a.nwg + a.spw - 1) / a.spw, units / wpb);
    const dim3 block(64 * waves);
    const bool mq = a.qslots > 1;
    // two column blocks per wave: several query rows, keys of at most 128
    constexpr bool CB2 = DK <= 128;
    const bool cb2 = CB2 && mq && a.cb == 2;
    const MetaArgs none{};
    if (kv == PKA_BF16) {
        const size_t lds = decode_lds_bytes<DK, DV, false>(waves, cb2 ? 2 : 1);
        if (cb2) hipLaunchKernelGGL((decode_mfma_kernel<DK, DV, false, true, false, CB2 ? 2 : 1>), grid, block, lds, s, a, none);
        else if (mq) hipLaunchKernelGGL((decode_mfma_kernel<DK, DV, false, true, false>), grid, block, lds, s, a, none);
        else hipLaunchKernelGGL((decode_mfma_kernel<DK, DV, false, false, false>), grid, block, lds, s, a, none);
    } else if (kv == PKA_FP8_E4M3FN) {
        const size_t lds = decode_lds_bytes<DK, DV, true>(waves, cb2 ? 2 : 1);
        if (cb2) hipLaunchKernelGGL((decode_mfma_kernel<DK, DV, true, true, false, CB2 ? 2 : 1>), grid, block, lds, s, a, none);
        else if (mq) hipLaunchKernelGGL((decode_mfma_kernel<DK, DV, true, true, false>), grid, block, lds, s, a, none);
        else hipLaunchKernelGGL((decode_mfma_kernel<DK, DV, true, false, false>), grid, block, lds, s, a, none);
    } else {
        if (mq) hipLaunchKernelGGL((decode_f32_kernel<DK, DV, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((decode_f32_kernel<DK, DV, false>), grid, block, 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge<DV>(q, a, nullptr, s);
}

template <int DK, int DV>
hipError_t launch_decode_md_d(pka_dtype q, pka_dtype kv, const AttnArgs& a, const MetaArgs& m, int wpb,
                              hipStream_t s) {
    const int units = a.Hkv * a.qgroups * a.csplit;
    const int waves = wpb * a.spw;
    const dim3 grid((a.nwg + a.spw - 1) / a.spw, units / wpb);
    const dim3 block(64 * waves);
    if (kv == PKA_BF16) {
        const size_t lds = decode_md_lds_bytes<DK, DV, false>(waves, a.B);
        hipLaunchKernelGGL((decode_mfma_kernel<DK, DV, false, false, true>), grid, block, lds, s, a, m);
    } else if (kv == PKA_FP8_E4M3FN) {
        const size_t lds = decode_md_lds_bytes<DK, DV, true>(waves, a.B);
        hipLaunchKernelGGL((decode_mfma_kernel<DK, DV, true, false, true>), grid, block, lds, s, a, m);
    } else {
        return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge<DV>(q, a, &m, s);
}

template <typename K>
int occupancy(K kernel, int waves, size_t lds) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 64 * waves, lds);
    return e == hipSuccess ? n : 0;
}

template <int DK, int DV>
int blocks_per_cu_d(pka_dtype kv, int waves) {
    if (kv == PKA_BF16)
        return occupancy(decode_mfma_kernel<DK, DV, false, false, false>, waves, decode_lds_bytes<DK, DV, false>(waves));
    if (kv == PKA_FP8_E4M3FN)
        return occupancy(decode_mfma_kernel<DK, DV, true, false, false>, waves, decode_lds_bytes<DK, DV, true>(waves));
    return occupancy(decode_f32_kernel<DK, DV, false>, waves, 0);
}

// the in-kernel metadata variant at the largest batch it takes
template <int DK, int DV>
int blocks_per_cu_md_d(pka_dtype kv, int waves) {
    if (kv == PKA_BF16)
        return occupancy(decode_mfma_kernel<DK, DV, false, false, true>, waves,
                         decode_md_lds_bytes<DK, DV, false>(waves, DEC_MD_MAX_B));
    if (kv == PKA_FP8_E4M3FN)
        return occupancy(decode_mfma_kernel<DK, DV, true, false, true>, waves,
                         decode_md_lds_bytes<DK, DV, true>(waves, DEC_MD_MAX_B));
    return 0;
}

}  // namespace

int decode_blocks_per_cu(pka_dtype kv, int DK, int DV, int waves) {
    if (DK == 128 && DV == 128) return blocks_per_cu_d<128, 128>(kv, waves);
    if (DK == 64 && DV == 64) return blocks_per_cu_d<64, 64>(kv, waves);
    if (DK == 192 && DV == 128) return blocks_per_cu_d<192, 128>(kv, waves);
    return 0;
}

bool decode_md_fits(pka_dtype kv, int DK, int DV, int waves) {
    int md = 0;
    if (DK == 128 && DV == 128) md = blocks_per_cu_md_d<128, 128>(kv, waves);
    else if (DK == 64 && DV == 64) md = blocks_per_cu_md_d<64, 64>(kv, waves);
    else if (DK == 192 && DV == 128) md = blocks_per_cu_md_d<192, 128>(kv, waves);
    return md > 0 && md == decode_blocks_per_cu(kv, DK, DV, waves);
}

hipError_t launch_decode(pka_dtype q, pka_dtype kv, int DK, int DV, const AttnArgs& a, int wpb,
                         hipStream_t s) {
    if (DK == 128 && DV == 128) return launch_decode_d<128, 128>(q, kv, a, wpb, s);
    if (DK == 64 && DV == 64) return launch_decode_d<64, 64>(q, kv, a, wpb, s);
    if (DK == 192 && DV == 128) return launch_decode_d<192, 128>(q, kv, a, wpb, s);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_md(pka_dtype q, pka_dtype kv, int DK, int DV, const AttnArgs& a,
                            const MetaArgs& m, int wpb, hipStream_t s) {
    if (DK == 128 && DV == 128) return launch_decode_md_d<128, 128>(q, kv, a, m, wpb, s);
    if (DK == 64 && DV == 64) return launch_decode_md_d<64, 64>(q, kv, a, m, wpb, s);
    if (DK == 192 && DV == 128) return launch_decode_md_d<192, 128>(q, kv, a, m, wpb, s);
    return hipErrorInvalidValue;
}

}  // namespace pka
