// forward_extend: a causal block of new tokens against the cached prefix plus
// themselves.
//
// Prefill reads long query blocks and is compute-bound ("sglang-101 s4.2
// --attention-backend", section "Two backends in one server"; "[SGLang]
// Hybrid Attention", introduction).  New token i of request b sits at
// position p_b + i and attends to positions 0 .. p_b + i (bottom-right
// causal alignment across the prefix/new boundary); its K/V were written by
// save_kv before this call.
//
// gfx950 mapping of the bf16 variant.  A workgroup (4 waves) owns one
// (request, query tile, KV head) item; its 128 query columns are the tile's
// tokens times the G query heads sharing the KV head (GQA packing), so every
// K/V tile staged in LDS feeds 128 columns.  Per 64-key tile and wave:
//   S^T[key, col] = K . Q^T      16 x v_mfma_f32_32x32x16_bf16 (D = 128)
//   O^T[d, col]  += V^T . P^T    16 x v_mfma_f32_32x32x16_bf16
// Column statistics of the online softmax live in the lane (two lanes per
// column), P^T is used in place as the B operand, and V^T comes from LDS
// through transposing reads.  K/V tiles are double-buffered in LDS and
// filled by direct HBM -> LDS loads one tile ahead; within a wave the scores
// of tile t+1 are computed while the probabilities of tile t are formed, so
// the matrix cores have independent work during the softmax.  Workgroups of
// one KV head are kept on one XCD, whose L2 then serves the K/V pages that
// all query tiles of a request read.
#include <type_traits>

#include "fp8.h"
#include "pka_internal.h"

namespace pka {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float LN2 = 0.69314718055994531f;
constexpr int EXT_WAVES = 4;   // waves per workgroup
constexpr int EXT_COLS = 32 * EXT_WAVES;  // query columns per workgroup (32 per wave)
constexpr int BN = 64;         // keys per tile (two 32-key MFMA blocks)
constexpr int EXT_XCDS = 8;    // accelerator dies (each with its own L2)

__device__ inline uint32_t pack_bf16(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ inline bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ inline int32_t slot_of(const AttnArgs& a, int32_t page_base, int32_t pos) {
    int64_t idx = (int64_t)page_base + (pos >> a.page_shift);
    idx = idx < a.kv_cap ? idx : a.kv_cap - 1;
    int32_t pg = a.kv_indices[idx];
    pg = min(max(pg, 0), a.num_pages - 1);
    return (pg << a.page_shift) | (pos & ((1 << a.page_shift) - 1));
}

// row of the 32x32 MFMA accumulator held by register r of lane half hh
__device__ constexpr int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// Online-softmax state of one query column (two lanes per column).  The
// running max is raised lazily: only when a tile's max exceeds it by more
// than LAZY (log2 units) are O and the normaliser rescaled, so most tiles
// skip the rescale and the cross-lane exchange; p = 2^(s*c - m) then stays
// below 2^LAZY.
constexpr float LAZY = 8.0f;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Max of x over the two lane halves (lanes l and l^32).
__device__ inline float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct HBM -> LDS loads of 16 bytes per lane: lane i's bytes land at
// lds_dst + 16 * i (lds_dst is wave-uniform; the compiler moves it to M0).
// The caller orders them with an explicit vmcnt(0) wait and a barrier before
// any wave reads the destination.  The buffer form addresses a wave-uniform
// base (a raw buffer resource) plus a 32-bit per-lane offset; the compiler
// counts it in vmcnt alone, so the LDS operand reads issued after it keep
// their partial lgkmcnt waits (the global form also counts as an LDS access
// and turns those into full waits).  The global form takes any 64-bit
// address and serves pools beyond 4 GiB on pages of under 64 tokens.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ inline void lds_dma16(const void* src, const uint8_t* lds_dst) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (lds_void_t*)lds_dst, 16, 0, 0);
}
// raw buffer of `bytes` bytes from `base`: offsets at or beyond it read zero
__device__ inline __amdgpu_buffer_rsrc_t raw_buffer(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                             0x00020000 /* 32-bit data format */);
}
__device__ inline void lds_dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, const uint8_t* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_dst, 16, voff, 0, 0, 0);
}

// LDS tiles: BN keys x D dims of K or of V, rows of 16-byte chunks with no
// padding, filled by direct HBM -> LDS loads (each lane's 16 bytes land at
// base + 16 * lane).  Chunks are XOR-swizzled per row so the reads are
// bank-conflict free: K is read 16 rows x one chunk at a time, so the 16
// rows must land on 16 different 16-byte bank groups (256 bytes per bank
// cycle): 256-byte rows use chunk ^ row; 128-byte rows (two per cycle) and
// 384-byte rows (starting alternately at bank 0 and half-way round) use
// chunk ^ (row / 2 % 8), which keeps every chunk inside its aligned group of
// 8.  V is read by the transposing loads, 4 rows x 4 chunks at a time
// (chunk ^ 4 * (row % 4)).
template <int D> struct ExtTile {
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row (bf16)
    static constexpr int ROWB = D * 2;
    static constexpr int TILEB = BN * ROWB;            // bytes of one tile
    static constexpr int LOADS = TILEB / (64 * EXT_WAVES * 16);  // DMA instructions per thread per tile
    static constexpr bool POW2 = (CPR & (CPR - 1)) == 0;
    static_assert(CPR == 8 || CPR == 16 || CPR == 24, "row widths: 64, 128 or 192 dims");
    __device__ static constexpr int kchunk(int row, int c) {
        return CPR == 16 ? c ^ (row & 15) : c ^ ((row >> 1) & 7);
    }
    __device__ static constexpr int vchunk(int row, int c) { return c ^ ((4 * (row & 3)) & (CPR - 1)); }
};

// Which part of a tile thread `tid` of a workgroup moves (move j of NR).
// bf16: wave instruction j of wave w fills bytes 1024 (LOADS w + j) .. of
// the tile, lane i the 16-byte chunk 64 (LOADS w + j) + i, i.e. row
// chunk / CPR at physical position chunk % CPR.  fp8: 16-byte pieces
// tid + 256 j of the tile's rows (D / 16 per row) pass through registers.
template <int D, bool FP8> struct Mover {
    using T = ExtTile<D>;
    static constexpr int PPR = D / 16;                 // fp8 16-byte pieces per row
    static constexpr int NR = FP8 ? D / 64 : T::LOADS;  // moves per thread and tile
    static_assert(FP8 ? 256 * NR == BN * PPR : 64 * EXT_WAVES * NR == BN * T::CPR, "tile coverage");
    __device__ static int flat(int tid, int j) { return (T::LOADS * (tid >> 6) + j) * 64 + (tid & 63); }
    __device__ static int row(int tid, int j) { return FP8 ? (tid + 256 * j) / PPR : flat(tid, j) / T::CPR; }
    // bf16: physical chunk within the row; fp8: piece within the row
    __device__ static int pos(int tid, int j) { return FP8 ? (tid + 256 * j) % PPR : flat(tid, j) % T::CPR; }
};

// Uniform 32-bit load through the scalar data cache (read only).
__device__ inline int32_t load_uniform(const int32_t* p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)(uintptr_t)p)[i];
}

// Software pipeline over 64-key tiles t (per wave):
//   top of iteration t: K(t+1) and V(t) are in LDS, the raw scores S(t) are
//   in registers; the direct loads of K(t+2) and V(t+1) start into the
//   buffers that iteration t-1 finished with;
//   softmax statistics of S(t), then one interleaved block in which the
//   exponentials of S(t), the P.V MFMAs of tile t and the K.Q^T MFMAs of
//   tile t+1 (independent of the softmax) are issued together, so the matrix
//   cores run while the vector ALUs compute probabilities.
// BIGPAGE (page size >= 64): a tile lies in one page, so its pool address is
// a scalar and each lane only adds a fixed row offset.  Smaller pages gather
// rows by slot: SLOT64 when a pool spans more than 4 GiB (64-bit addresses),
// else 32-bit offsets from the pool's base.
// DK: key (and query) width; DV: value (and output) width.
template <int DK, int DV, bool POS, bool BIGPAGE, bool FP8, bool SLOT64>
__global__ __launch_bounds__(64 * EXT_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2))) void extend_mfma_kernel(AttnArgs a) {
    using TK = ExtTile<DK>;
    using TV = ExtTile<DV>;
    using MK = Mover<DK, FP8>;
    using MV = Mover<DV, FP8>;
    static_assert(TV::POW2, "value rows are read by the transposing loads");
    constexpr bool SAME = DK == DV;             // K and V tiles moved by the same rows
    constexpr int KSTEPS = DK / 16;             // k-steps of q.k (32x32x16)
    constexpr int VC = DV / 32;                 // 32-dim blocks of O^T (d = 32 c + row)
    constexpr int SB = BN / 32;                 // 32-key score blocks per tile
    constexpr int PK = BN / 16;                 // P.V k-steps per tile
    constexpr int QPK = KSTEPS * SB / PK;       // next-tile K.Q^T MFMAs per P.V k-step
    static_assert(QPK * PK == KSTEPS * SB, "K.Q^T MFMAs spread over the P.V k-steps");
    __shared__ __attribute__((aligned(1024))) uint8_t sK0[TK::TILEB], sK1[TK::TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t sV0[TV::TILEB], sV1[TV::TILEB];

    // Workgroups are dealt to the 8 XCDs round-robin (linear id mod 8).  The
    // (KV head, item) list is cut into 8 contiguous chunks, one per XCD, so
    // the items of one KV head (same K/V pages) share one XCD's L2.
    const int32_t* plan = a.plan;
    // XCD x receives grid/8 workgroups, plus one when x < grid % 8.
    // With a key-range split (a.ext_split = C > 1) each item has C
    // consecutive workgroups, one per chunk of its key tiles.
    const int32_t C = a.ext_split;
    const int32_t cap = gridDim.x / (a.Hkv * C);  // item slots per KV head
    const int32_t xcd = blockIdx.x % EXT_XCDS;
    const int32_t base = gridDim.x / EXT_XCDS, extra = gridDim.x % EXT_XCDS;
    const int32_t w = xcd * base + min(xcd, extra) + blockIdx.x / EXT_XCDS;
    const int32_t g = w / (cap * C), item = (w % (cap * C)) / C, chunk = w % C;
    if (item >= plan[PLAN_EXT_COUNT]) return;
    const int32_t TQ = plan[PLAN_EXT_TQ];
    const int32_t* items = plan + plan_ext_items(a.B);
    const int32_t b = items[2 * item], ti = items[2 * item + 1];
    const int32_t* F = plan + plan_seg_prefix(a.B);
    const int32_t q0 = a.qo_indptr[b];
    const int32_t nb = a.qo_indptr[b + 1] - q0;
    const int32_t L = F[b + 1] - F[b];
    const int32_t pb = L - nb;
    const int32_t tok_lo = ti * TQ;
    const int32_t tok_hi = min(tok_lo + TQ, nb);
    const int32_t page_base = a.kv_indptr[b];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hh = lane >> 5;
    const int col = wave * 32 + n;
    const int ctok = tok_lo + col / a.G;
    const bool col_ok = col < TQ * a.G && ctok < tok_hi && q0 + ctok < a.N;
    const int32_t qtok = col_ok ? ctok : tok_lo;  // invalid columns mirror a valid one
    const int32_t head = g * a.G + col % a.G;
    const int32_t qpos = pb + qtok;
    const int32_t qpos_min = pb + tok_lo;  // tiles wholly at or below it need no mask

    // Q^T operand: k-step s covers dims 16 s + 8 hh .. + 8
    bf16x8_t qop[KSTEPS];
    {
        const int32_t qr = min(q0 + qtok, a.N - 1);  // rows past N only under a flagged batch
        const __bf16* qrow = (const __bf16*)a.q + ((int64_t)qr * a.Hq + head) * DK;
        #pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qop[s] = as_bf16x8(*(const u32x4_t*)(qrow + 16 * s + 8 * hh));
    }

    const int32_t kend = pb + tok_hi;  // keys 0 .. kend-1
    // This workgroup's key tiles: all of the item's, or with a split, chunk
    // `chunk` of them.  A chunk may start only at a tile whose first key is
    // at or below the item's first query position, so every column has a
    // visible key in every chunk; the last non-empty chunk runs to the end.
    int32_t t_lo = 0, ntiles = (kend + BN - 1) / BN;
    if (C > 1) {
        const int32_t nstart = min(ntiles, qpos_min / BN + 1);  // tiles a chunk may start at
        const int32_t per = (nstart + C - 1) / C;
        t_lo = chunk * per;
        if (t_lo >= nstart) {
            // empty chunk: a zero-weight partial (lse -inf, o 0)
            if (col_ok) {
                const int64_t pi = ((int64_t)(q0 + ctok) * a.Hq + head) * C + chunk;
                #pragma unroll
                for (int c = 0; c < VC; ++c)
                    #pragma unroll
                    for (int r = 0; r < 16; r += 4)
                        *(u32x2_t*)((__bf16*)a.ws_o + pi * DV + 32 * c + acc_row(r, hh)) = u32x2_t{0u, 0u};
                if (hh == 0) a.ws_lse[pi] = -INFINITY;
            }
            return;
        }
        ntiles = ((chunk + 1) * per < nstart ? (chunk + 1) * per : ntiles) - t_lo;
    }
    const int32_t kb0 = t_lo * BN;  // key position of this workgroup's first tile
    constexpr int ESZ = FP8 ? 1 : 2;  // cache bytes per element
    const int32_t krow = a.Hkv * DK * ESZ, vrow = a.Hkv * DV * ESZ;  // bytes of one pool slot
    const uint8_t* kbase = (const uint8_t*)a.k_pool + (int64_t)g * DK * ESZ;
    const uint8_t* vbase = (const uint8_t*)a.v_pool + (int64_t)g * DV * ESZ;
    const int32_t P = 1 << a.page_shift;

    // Moving a tile into LDS (per tensor, as Mover lays out).  bf16: direct
    // loads; the lane fetches the logical chunk that the swizzle puts at its
    // physical position.  fp8: 16-byte pieces are loaded into registers and,
    // once the current tile is done, written converted to bf16 into the
    // same swizzled layout.  Rows past the last key repeat it.
    // Tensor tags: K_ / V_ select the tile type, pool and registers.
    using K_ = std::integral_constant<bool, false>;
    using V_ = std::integral_constant<bool, true>;
    // per-thread byte offsets of move j: the fetched chunk within a row (small
    // pages), plus the row within the tile (BIGPAGE)
    uint32_t koff[MK::NR], voff[MV::NR];
    #pragma unroll
    for (int j = 0; j < MK::NR; ++j) {
        const int r = MK::row(tid, j);
        koff[j] = 16 * (FP8 ? MK::pos(tid, j) : TK::kchunk(r, MK::pos(tid, j))) + (BIGPAGE ? r * krow : 0);
    }
    #pragma unroll
    for (int j = 0; j < MV::NR; ++j) {
        const int r = MV::row(tid, j);
        voff[j] = 16 * (FP8 ? MV::pos(tid, j) : TV::vchunk(r, MV::pos(tid, j))) + (BIGPAGE ? r * vrow : 0);
    }
    u32x4_t rk[MK::NR], rv[MV::NR];  // fp8: tiles on their way to LDS
    // per-tensor views (the unused branch of each is discarded at compile time)
    auto offs = [&](auto vt) -> auto& { if constexpr (decltype(vt)::value) return voff; else return koff; };
    auto regs = [&](auto vt) -> auto& { if constexpr (decltype(vt)::value) return rv; else return rk; };
    // logical chunk c of row r: its physical position
    auto phys = [](auto vt, int r, int c) {
        if constexpr (decltype(vt)::value) return TV::vchunk(r, c);
        else return TK::kchunk(r, c);
    };

    // pool byte offset of a tile's first row (BIGPAGE; wave-uniform)
    auto tile_base = [&](int32_t pg, int32_t kt0, int32_t row_bytes) -> int64_t {
        pg = min(max(pg, 0), a.num_pages - 1);
        return (((int64_t)pg << a.page_shift) | (kt0 & (P - 1))) * (int64_t)row_bytes;
    };
    auto page_of_tile = [&](int32_t kt0) -> int32_t {
        int64_t idx = (int64_t)page_base + (kt0 >> a.page_shift);
        idx = idx < a.kv_cap ? idx : a.kv_cap - 1;
        return load_uniform(a.kv_indices, idx);
    };
    // BIGPAGE: one tensor's tile from page pg
    auto dma_big = [&](auto vt, int32_t pg, int32_t kt0, uint8_t* dst) {
        constexpr bool V = decltype(vt)::value;
        using M = typename std::conditional<V, MV, MK>::type;
        using TT = typename std::conditional<V, TV, TK>::type;
        const int32_t rb = V ? vrow : krow;
        const uint8_t* tb = (V ? vbase : kbase) + tile_base(pg, kt0, rb);
        const auto& off = offs(vt);
        const int32_t lim = kend - 1 - kt0;  // last row of the tile holding a key
        if constexpr (FP8) {
            auto& rg = regs(vt);
            #pragma unroll
            for (int j = 0; j < M::NR; ++j) {
                const uint32_t o = lim >= BN - 1 ? off[j] : (uint32_t)(min(M::row(tid, j), lim) * rb + 16 * M::pos(tid, j));
                rg[j] = __builtin_nontemporal_load((const u32x4_t*)(tb + o));
            }
        } else if (lim >= BN - 1) {
            const auto rs = raw_buffer(tb, BN * rb);
            #pragma unroll
            for (int j = 0; j < M::NR; ++j) lds_dma16_buf(rs, off[j], dst + (TT::LOADS * wave + j) * 1024);
        } else {
            const auto rs = raw_buffer(tb, BN * rb);
            #pragma unroll
            for (int j = 0; j < M::NR; ++j) {
                const int r = M::row(tid, j);
                const int ch = phys(vt, r, M::pos(tid, j));
                lds_dma16_buf(rs, (uint32_t)(min(r, lim) * rb + 16 * ch), dst + (TT::LOADS * wave + j) * 1024);
            }
        }
    };
    // small pages: per-row slots; raw page ids are looked up an iteration
    // before the slots are formed
    auto lookup = [&](auto vt, int32_t kt0, auto& pg, auto& kp) {
        using M = typename std::conditional<decltype(vt)::value, MV, MK>::type;
        #pragma unroll
        for (int j = 0; j < M::NR; ++j) {
            kp[j] = min(kt0 + M::row(tid, j), kend - 1);
            int64_t idx = (int64_t)page_base + (kp[j] >> a.page_shift);
            idx = idx < a.kv_cap ? idx : a.kv_cap - 1;
            pg[j] = a.kv_indices[idx];
        }
    };
    auto form_slots = [&](auto vt, const auto& pg, const auto& kp, auto& slot) {
        using M = typename std::conditional<decltype(vt)::value, MV, MK>::type;
        #pragma unroll
        for (int j = 0; j < M::NR; ++j)
            slot[j] = (min(max(pg[j], 0), a.num_pages - 1) << a.page_shift) | (kp[j] & (P - 1));
    };
    auto dma_small = [&](auto vt, const auto& slot, uint8_t* dst) {
        constexpr bool V = decltype(vt)::value;
        using M = typename std::conditional<V, MV, MK>::type;
        using TT = typename std::conditional<V, TV, TK>::type;
        const int32_t rb = V ? vrow : krow;
        const uint8_t* src = V ? vbase : kbase;
        const auto& off = offs(vt);
        if constexpr (FP8) {
            auto& rg = regs(vt);
            #pragma unroll
            for (int j = 0; j < M::NR; ++j)
                rg[j] = __builtin_nontemporal_load((const u32x4_t*)(src + (int64_t)slot[j] * rb + off[j]));
        } else if constexpr (SLOT64) {
            #pragma unroll
            for (int j = 0; j < M::NR; ++j)
                lds_dma16(src + (int64_t)slot[j] * rb + off[j], dst + (TT::LOADS * wave + j) * 1024);
        } else {
            // the pool from this head on fits in 32-bit offsets (checked at launch)
            const int64_t pool_bytes = a.pool_slots * (int64_t)rb;
            const auto rs = raw_buffer(src, pool_bytes < (int64_t)UINT32_MAX ? (uint32_t)pool_bytes : UINT32_MAX);
            #pragma unroll
            for (int j = 0; j < M::NR; ++j)
                lds_dma16_buf(rs, (uint32_t)slot[j] * (uint32_t)rb + off[j], dst + (TT::LOADS * wave + j) * 1024);
        }
    };
    // fp8: write one tensor's tile (registers) into LDS as bf16; each 16-byte
    // piece becomes logical chunks 2 p and 2 p + 1 of its row (exact)
    auto f8_finish = [&](auto vt, uint8_t* dst) {
        using M = typename std::conditional<decltype(vt)::value, MV, MK>::type;
        using TT = typename std::conditional<decltype(vt)::value, TV, TK>::type;
        const auto& rg = regs(vt);
        #pragma unroll
        for (int j = 0; j < M::NR; ++j) {
            const int r = M::row(tid, j), p2 = 2 * M::pos(tid, j);
            const u32x4_t w = rg[j];
            const u32x4_t c0 = {fp8x2_to_bf16x2<false>(w.x), fp8x2_to_bf16x2<true>(w.x),
                                fp8x2_to_bf16x2<false>(w.y), fp8x2_to_bf16x2<true>(w.y)};
            const u32x4_t c1 = {fp8x2_to_bf16x2<false>(w.z), fp8x2_to_bf16x2<true>(w.z),
                                fp8x2_to_bf16x2<false>(w.w), fp8x2_to_bf16x2<true>(w.w)};
            *(u32x4_t*)(dst + r * TT::ROWB + 16 * phys(vt, r, p2)) = c0;
            *(u32x4_t*)(dst + r * TT::ROWB + 16 * phys(vt, r, p2 + 1)) = c1;
        }
    };

    // V^T operand: lane group G = lane/16 reads keys 4 (G/2) + s16/4 (+ 16 ks
    // + 8 r) at dims 16 (G%2) + 4 (s16%4) (+ 32 c) with the transposing load.
    const int G16 = lane >> 4, s16 = lane & 15;
    const int v_row = 4 * (G16 >> 1) + (s16 >> 2);
    const int v_byte = 32 * (G16 & 1) + 8 * (s16 & 3);  // byte within the 64-byte group of block c

    f32x16_t O[VC];
    #pragma unroll
    for (int c = 0; c < VC; ++c)
        #pragma unroll
        for (int r = 0; r < 16; ++r) O[c][r] = 0.f;
    float m2 = -INFINITY, lsum = 0.f;
    const float c2 = a.scale_log2;
    const uint32_t ones = 0x3f803f80u;  // two bf16 1.0

    // K.Q^T MFMA q (of KSTEPS * SB) of a tile: k-step q / SB, key block q % SB
    auto qk_mfma = [&](const uint8_t* ks_, int q, f32x16_t* S) {
        const int s = q / SB, u = q % SB;
        const int row = 32 * u + n;
        const u32x4_t kw = *(const u32x4_t*)(ks_ + row * TK::ROWB + 16 * TK::kchunk(row, 2 * s + hh));
        // the first k-step starts from an inline zero accumulator
        S[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw), qop[s], s == 0 ? f32x16_t{} : S[u],
                                                       0, 0, 0);
    };

    // Where the next tile's scores are computed.  Equal widths: inside the
    // P.V block, interleaved with the exponentials (two score sets that swap
    // roles from one iteration to the next).  Wider keys (192/128): after
    // the block, into the registers this tile's scores held; the score
    // phase is then long enough on its own (24 MFMAs) and one score set
    // fewer leaves registers to the block.
    constexpr bool SPLITQK = DK > DV;
    f32x16_t SA[SB], SBn[SPLITQK ? 1 : SB];
    auto second = [&]() -> f32x16_t (&)[SB] {
        if constexpr (SPLITQK) return SA;
        else return SBn;
    };
    f32x16_t (&SB2)[SB] = second();

    // prologue: K(0), V(0), K(1) resident, S(0) computed
    // BIGPAGE: page ids by tile parity.  At the top of iteration t, pgp[t & 1]
    // holds the page of tile t+2 (its K goes out now) and pgp[~t & 1] that of
    // tile t+1 (its V goes out now); that slot then takes tile t+3's id, which
    // is first used an iteration later, so the lookup is never waited for
    // where it is issued.
    int32_t pgp[2] = {0, 0};
    // small pages.  Equal widths: V(t+1) reuses the slots K(t+1) was loaded
    // with.  Otherwise V's rows have lookups of their own, also an iteration
    // ahead (rawV holds the page ids of V(t+1) at the top of iteration t).
    int32_t rawK[MK::NR], kpK[MK::NR], slotK[MK::NR];
    int32_t rawV[MV::NR], kpV[MV::NR], slotV[MV::NR];
    if constexpr (BIGPAGE) {
        const int32_t p0 = page_of_tile(kb0);
        dma_big(K_{}, p0, kb0, sK0);
        dma_big(V_{}, p0, kb0, sV0);
        if constexpr (FP8) {
            f8_finish(K_{}, sK0);
            f8_finish(V_{}, sV0);
        }
        if (ntiles > 1) {
            const int32_t p1 = page_of_tile(kb0 + BN);
            dma_big(K_{}, p1, kb0 + BN, sK1);
            if constexpr (FP8) f8_finish(K_{}, sK1);
            pgp[1] = p1;
        }
        if (ntiles > 2) pgp[0] = page_of_tile(kb0 + 2 * BN);
    } else if constexpr (SAME) {
        lookup(K_{}, kb0, rawK, kpK);
        form_slots(K_{}, rawK, kpK, slotK);
        dma_small(K_{}, slotK, sK0);
        dma_small(V_{}, slotK, sV0);
        if constexpr (FP8) {
            f8_finish(K_{}, sK0);
            f8_finish(V_{}, sV0);
        }
        lookup(K_{}, kb0 + BN, rawK, kpK);
        form_slots(K_{}, rawK, kpK, slotV);
        if (ntiles > 1) {
            dma_small(K_{}, slotV, sK1);
            if constexpr (FP8) f8_finish(K_{}, sK1);
        }
        lookup(K_{}, kb0 + 2 * BN, rawK, kpK);
    } else {
        lookup(K_{}, kb0, rawK, kpK);
        form_slots(K_{}, rawK, kpK, slotK);
        dma_small(K_{}, slotK, sK0);
        lookup(V_{}, kb0, rawV, kpV);
        form_slots(V_{}, rawV, kpV, slotV);
        dma_small(V_{}, slotV, sV0);
        if constexpr (FP8) {
            f8_finish(K_{}, sK0);
            f8_finish(V_{}, sV0);
        }
        if (ntiles > 1) {
            lookup(K_{}, kb0 + BN, rawK, kpK);
            form_slots(K_{}, rawK, kpK, slotK);
            dma_small(K_{}, slotK, sK1);
            if constexpr (FP8) f8_finish(K_{}, sK1);
        }
        lookup(V_{}, kb0 + BN, rawV, kpV);
        lookup(K_{}, kb0 + 2 * BN, rawK, kpK);
    }
    if constexpr (!FP8) __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the direct loads landed
    __syncthreads();
    #pragma unroll
    for (int q = 0; q < KSTEPS * SB; ++q) qk_mfma(sK0, q, SA);

    auto iteration = [&](auto odd_c, auto next_c, int32_t t, f32x16_t (&S)[SB], f32x16_t (&Sn)[SB]) {
        constexpr bool ODD = decltype(odd_c)::value;
        constexpr bool NEXT = decltype(next_c)::value;  // t + 1 < ntiles
        const uint8_t* vcur = ODD ? sV1 : sV0;  // V(t)
        const uint8_t* knext = ODD ? sK0 : sK1; // K(t+1)
        uint8_t* kdst = ODD ? sK1 : sK0;        // K(t+2)
        uint8_t* vdst = ODD ? sV0 : sV1;        // V(t+1)
        const int32_t kt0 = kb0 + t * BN;

        // bf16: K(t+1), V(t) and the lookups have landed (fp8 tiles were
        // written to LDS at the end of the previous iteration)
        if constexpr (!FP8) __builtin_amdgcn_s_waitcnt(0x0f70);
        __syncthreads();  // ... for every wave; iteration t-1 is done
        if constexpr (BIGPAGE) {
            constexpr int PI = ODD ? 1 : 0;  // t & 1
            if (t + 2 < ntiles) dma_big(K_{}, pgp[PI], kt0 + 2 * BN, kdst);
            if (NEXT) dma_big(V_{}, pgp[1 - PI], kt0 + BN, vdst);
            if (t + 3 < ntiles) pgp[1 - PI] = page_of_tile(kt0 + 3 * BN);
        } else if constexpr (SAME) {
            if (NEXT) dma_small(V_{}, slotV, vdst);
            if (t + 2 < ntiles) {
                form_slots(K_{}, rawK, kpK, slotK);
                dma_small(K_{}, slotK, kdst);
                #pragma unroll
                for (int j = 0; j < MK::NR; ++j) slotV[j] = slotK[j];
                lookup(K_{}, kt0 + 3 * BN, rawK, kpK);
            }
        } else {
            if (NEXT) {
                form_slots(V_{}, rawV, kpV, slotV);
                dma_small(V_{}, slotV, vdst);
                lookup(V_{}, kt0 + 2 * BN, rawV, kpV);
            }
            if (t + 2 < ntiles) {
                form_slots(K_{}, rawK, kpK, slotK);
                dma_small(K_{}, slotK, kdst);
                lookup(K_{}, kt0 + 3 * BN, rawK, kpK);
            }
        }

        // causal mask only where the tile crosses the diagonal of some column
        if (kt0 + BN - 1 > qpos_min) {
            #pragma unroll
            for (int u = 0; u < SB; ++u)
                #pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kt0 + 32 * u + acc_row(r, hh) > qpos) S[u][r] = -INFINITY;
        }
        if constexpr (!POS) {
            #pragma unroll
            for (int u = 0; u < SB; ++u)
                #pragma unroll
                for (int r = 0; r < 16; ++r) S[u][r] = S[u][r] == -INFINITY ? -INFINITY : S[u][r] * c2;
        }
        float mx = -INFINITY;
        #pragma unroll
        for (int u = 0; u < SB; ++u)
            #pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[u][r]);
        const float mc = POS ? mx * c2 : mx;  // this half's candidate max, log2 units
        if (__any(mc > m2 + LAZY)) {
            const float mnew = fmaxf(m2, max_halves(mc));
            const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
            m2 = mnew;
            lsum *= alpha;
            #pragma unroll
            for (int c = 0; c < VC; ++c) O[c] *= alpha;
        }

        // The compiler's interleaving strategies for MFMA-heavy regions
        // order this block's MFMAs, operand reads and vector work: strategy
        // 0 over a bf16 cache and 3 over an fp8 cache (whose tile
        // conversions share the iteration) each gain 2-3% at equal widths,
        // and 3 gains 1-3% at 192/128 over a bf16 cache (A/B in one process;
        // 0 cost 3% over fp8 and 2-5% at 192/128).  Over a bf16 cache the
        // wave also raises its issue priority for the block, so that of the
        // two waves sharing a SIMD the one feeding the matrix core issues
        // first while the other runs its softmax prologue (+1-2%; over fp8,
        // whose conversions follow the block, no gain).
        if constexpr (!FP8) __builtin_amdgcn_s_setprio(1);
        if constexpr (!SPLITQK) __builtin_amdgcn_iglp_opt(FP8 ? 3 : 0);
        else if constexpr (!FP8) __builtin_amdgcn_iglp_opt(3);
        // interleaved block: probabilities of S(t) (bf16; the normaliser sums
        // the same rounded values), O^T += V^T . P^T over tile t, and the
        // scores of tile t+1.  A column has a valid key in every tile up to
        // its own position and tiles start at key 0, so m2 is finite here.
        #pragma unroll
        for (int pk = 0; pk < PK; ++pk) {
            const int u = pk >> 1, r0 = 8 * (pk & 1);
            uint32_t pw[4];
            #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s0 = S[u][r0 + 2 * i], s1 = S[u][r0 + 2 * i + 1];
                const float e0 = POS ? __builtin_fmaf(s0, c2, -m2) : s0 - m2;
                const float e1 = POS ? __builtin_fmaf(s1, c2, -m2) : s1 - m2;
                pw[i] = pack_bf16(__builtin_amdgcn_exp2f(e0), __builtin_amdgcn_exp2f(e1));
                lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[i]),
                                                        __builtin_bit_cast(bf16x2_t, ones), lsum, false);
            }
            if constexpr (NEXT && !SPLITQK) {
                #pragma unroll
                for (int qq = 0; qq < QPK; ++qq) qk_mfma(knext, pk * QPK + qq, Sn);
            }
            const bf16x8_t pop = as_bf16x8(u32x4_t{pw[0], pw[1], pw[2], pw[3]});
            #pragma unroll
            for (int c = 0; c < VC; ++c) {
                u32x2_t half[2];
                #pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int row = 16 * pk + 8 * r + v_row;
                    const int lc = 4 * c + (v_byte >> 4);
                    const uint8_t* p = vcur + row * TV::ROWB + 16 * TV::vchunk(row, lc) + (v_byte & 15);
                    half[r] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
                }
                const u32x4_t av = {half[0][0], half[0][1], half[1][0], half[1][1]};
                O[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), pop, O[c], 0, 0, 0);
            }
        }
        if constexpr (NEXT && SPLITQK) {
            #pragma unroll
            for (int q = 0; q < KSTEPS * SB; ++q) qk_mfma(knext, q, Sn);
        }
        if constexpr (!FP8) __builtin_amdgcn_s_setprio(0);
        // fp8: the next tiles go into the stages this iteration did not read;
        // the next iteration's barrier publishes them
        if constexpr (FP8) {
            if (t + 2 < ntiles) f8_finish(K_{}, kdst);
            if (NEXT) f8_finish(V_{}, vdst);
        }
    };

    using F_ = std::integral_constant<bool, false>;
    using T_ = std::integral_constant<bool, true>;
    int32_t t = 0;
    for (; t + 2 < ntiles; t += 2) {
        iteration(F_{}, T_{}, t, SA, SB2);
        iteration(T_{}, T_{}, t + 1, SB2, SA);
    }
    if (t + 1 < ntiles) {
        iteration(F_{}, T_{}, t, SA, SB2);
        iteration(T_{}, F_{}, t + 1, SB2, SA);
    } else {
        iteration(F_{}, F_{}, t, SA, SB2);
    }

    // finish: the two lanes of a column hold halves of the sums
    const float ltot = sum_halves(lsum);
    if (!col_ok) return;
    const float inv = a.v_scale / ltot;  // v_scale: fp8 V dequantisation (1 otherwise)
    if (C > 1) {
        // a chunk's partial: normalised output row (bf16; the merge weighs
        // the chunks in fp32) and natural-log lse, slot (row, head, chunk)
        const int64_t pi = ((int64_t)(q0 + ctok) * a.Hq + head) * C + chunk;
        __bf16* const prow = (__bf16*)a.ws_o + pi * DV;
        #pragma unroll
        for (int c = 0; c < VC; ++c)
            #pragma unroll
            for (int r = 0; r < 16; r += 4)
                *(u32x2_t*)(prow + 32 * c + acc_row(r, hh)) =
                    u32x2_t{pack_bf16(O[c][r] * inv, O[c][r + 1] * inv), pack_bf16(O[c][r + 2] * inv, O[c][r + 3] * inv)};
        if (hh == 0) a.ws_lse[pi] = (m2 + __builtin_amdgcn_logf(ltot)) * LN2;
        return;
    }
    __bf16* orow = (__bf16*)a.out + ((int64_t)(q0 + ctok) * a.Hq + head) * DV;
    #pragma unroll
    for (int c = 0; c < VC; ++c)
        #pragma unroll
        for (int r = 0; r < 16; r += 4) {
            // rows acc_row(r..r+3, hh) are consecutive dims 32 c + acc_row(r, hh) ...
            const u32x2_t pk = {pack_bf16(O[c][r] * inv, O[c][r + 1] * inv),
                                pack_bf16(O[c][r + 2] * inv, O[c][r + 3] * inv)};
            *(u32x2_t*)(orow + 32 * c + acc_row(r, hh)) = pk;
        }
    if (a.lse && hh == 0)
        a.lse[(int64_t)(q0 + ctok) * a.Hq + head] = (m2 + __builtin_amdgcn_logf(ltot)) * LN2;
}

// fp32 variant: one wave per (new token, query head), lanes over head_dim.
template <int DK, int DV>
__global__ __launch_bounds__(256) void extend_f32_kernel(AttnArgs a) {
    constexpr int EPK = DK / 64, EPV = DV / 64;  // key and value dims per lane
    const int lane = threadIdx.x & 63;
    const int32_t item = blockIdx.x;
    if (item >= a.plan[PLAN_EXT_COUNT]) return;
    const int32_t TQ = a.plan[PLAN_EXT_TQ];
    const int32_t* items = a.plan + plan_ext_items(a.B);
    const int32_t b = items[2 * item], ti = items[2 * item + 1];
    const int32_t h = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (h >= a.Hq) return;
    const int32_t g = h / a.G;
    const int32_t* F = a.plan + plan_seg_prefix(a.B);
    const int32_t q0 = a.qo_indptr[b], nb = a.qo_indptr[b + 1] - q0;
    const int32_t L = F[b + 1] - F[b], pb = L - nb;
    const int32_t page_base = a.kv_indptr[b];
    for (int32_t i = ti * TQ; i < min(ti * TQ + TQ, nb); ++i) {
        if (q0 + i >= a.N) break;
        float q[EPK], o[EPV];
        #pragma unroll
        for (int e = 0; e < EPK; ++e) q[e] = ((const float*)a.q)[((int64_t)(q0 + i) * a.Hq + h) * DK + e * 64 + lane];
        #pragma unroll
        for (int e = 0; e < EPV; ++e) o[e] = 0.f;
        float m = -INFINITY, l = 0.f;
        for (int32_t t = 0; t <= pb + i; ++t) {
            const int64_t sg = (int64_t)slot_of(a, page_base, t) * a.Hkv + g;
            float dot = 0.f;
            #pragma unroll
            for (int e = 0; e < EPK; ++e) dot += q[e] * ((const float*)a.k_pool)[sg * DK + e * 64 + lane];
            #pragma unroll
            for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
            const float s = dot * a.scale_log2;
            const float mn = fmaxf(m, s);
            const float al = __builtin_amdgcn_exp2f(m - mn);
            const float p = __builtin_amdgcn_exp2f(s - mn);
            m = mn;
            l = l * al + p;
            #pragma unroll
            for (int e = 0; e < EPV; ++e)
                o[e] = o[e] * al + p * ((const float*)a.v_pool)[sg * DV + e * 64 + lane];
        }
        #pragma unroll
        for (int e = 0; e < EPV; ++e)
            ((float*)a.out)[((int64_t)(q0 + i) * a.Hq + h) * DV + e * 64 + lane] = o[e] / l;
        if (a.lse && lane == 0)
            a.lse[(int64_t)(q0 + i) * a.Hq + h] = (m + __builtin_amdgcn_logf(l)) * LN2;
    }
}

}  // namespace

#ifndef PKA_EXTEND_DK192_TU
int extend_tq(pka_dtype q, pka_dtype /*kv*/, int G, int /*page_size*/) {
    if (q == PKA_F32) return 16;
    return G >= EXT_COLS ? 1 : EXT_COLS / G;
}

int extend_max_group(pka_dtype q, int /*page_size*/) {
    if (q == PKA_F32) return 1 << 30;
    return EXT_COLS;
}
#endif

namespace {
// Merge of a key-range split: each (query row, head) of the batch has C
// partials (normalised bf16 output row, natural-log lse; a chunk with no key
// leaves lse -inf and a zero row); out = sum_c e^(lse_c - M) o_c / sum_c
// e^(lse_c - M), lse = M + ln(sum_c e^(lse_c - M)), in fp32.  One wave per
// (row, head); lane l holds the EPL consecutive value dims from EPL * l (one
// access per row); chunk 0 always holds keys, so M is finite.
template <int DV>
__global__ __launch_bounds__(256) void extend_split_merge_kernel(AttnArgs a) {
    constexpr int EPL = DV / 64;
    static_assert(EPL == 1 || EPL == 2, "value rows of 64 or 128 dims");
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int32_t rows = min(a.qo_indptr[a.B], a.N);  // the batch's query rows
    if (pair >= (int64_t)rows * a.Hq) return;
    const int32_t C = a.ext_split;
    const float lv = lane < C ? a.ws_lse[pair * C + lane] : -INFINITY;
    float v[EXT_MAX_SPLIT][EPL];
    #pragma unroll
    for (int c = 0; c < EXT_MAX_SPLIT; ++c) {
        const __bf16* prow = (const __bf16*)a.ws_o + (pair * C + min(c, C - 1)) * DV;
        if constexpr (EPL == 2) {
            const uint32_t w = ((const uint32_t*)prow)[lane];
            v[c][0] = __uint_as_float(w << 16);
            v[c][1] = __uint_as_float(w & 0xffff0000u);
        } else {
            v[c][0] = __uint_as_float((uint32_t)((const uint16_t*)prow)[lane] << 16);
        }
    }
    float M = lv;
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float wk = lane < C ? expf(lv - M) : 0.f;
    float den = wk, acc[EPL];
    #pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    #pragma unroll
    for (int c = 0; c < EXT_MAX_SPLIT; ++c) {
        const float wt = __shfl(wk, c);
        #pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += wt * v[c][e];
    }
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
    const float inv = 1.0f / den;
    if constexpr (EPL == 2)
        ((uint32_t*)((__bf16*)a.out + pair * DV))[lane] = pack_bf16(acc[0] * inv, acc[1] * inv);
    else
        ((__bf16*)a.out)[pair * DV + lane] = (__bf16)(acc[0] * inv);
    if (a.lse && lane == 0) a.lse[pair] = M + logf(den);
}

// One launch of the MFMA kernel for a (widths, scale sign, page path, cache
// dtype) combination; the fp8 path moves tiles through registers and has no
// 64-bit gather variant.
template <int DK, int DV, bool POS, bool F8>
void launch_ext_p(const AttnArgs& a, bool big, bool wide, dim3 grid, hipStream_t s) {
    const dim3 block(64 * EXT_WAVES);
    if (big)
        hipLaunchKernelGGL((extend_mfma_kernel<DK, DV, POS, true, F8, false>), grid, block, 0, s, a);
    else if (F8 || !wide)
        hipLaunchKernelGGL((extend_mfma_kernel<DK, DV, POS, false, F8, false>), grid, block, 0, s, a);
    else if constexpr (!F8)
        hipLaunchKernelGGL((extend_mfma_kernel<DK, DV, POS, false, false, true>), grid, block, 0, s, a);
}
template <int DK, int DV>
void launch_ext_d(const AttnArgs& a, bool pos, bool big, bool wide, bool f8, dim3 grid, hipStream_t s) {
    if (f8) {
        if (pos) launch_ext_p<DK, DV, true, true>(a, big, wide, grid, s);
        else launch_ext_p<DK, DV, false, true>(a, big, wide, grid, s);
    } else {
        if (pos) launch_ext_p<DK, DV, true, false>(a, big, wide, grid, s);
        else launch_ext_p<DK, DV, false, false>(a, big, wide, grid, s);
    }
}
}  // namespace

// The MFMA kernels for 192-wide keys and 128-wide values over a bf16 cache
// are instantiated in a translation unit of their own (extend_dk192.hip,
// which includes this file), so that the build can compile them with the
// compiler's max-ILP scheduling strategy: +1-5% at page size 128 and 13-15%
// at page size 16, where the kernel is short of registers, while the same
// strategy costs the fp8 variants 1-4% (so those stay here).
void launch_extend_dk192(const AttnArgs& a, bool pos, bool big, bool wide, dim3 grid, hipStream_t s);
#ifdef PKA_EXTEND_DK192_TU
void launch_extend_dk192(const AttnArgs& a, bool pos, bool big, bool wide, dim3 grid, hipStream_t s) {
    if (pos) launch_ext_p<192, 128, true, false>(a, big, wide, grid, s);
    else launch_ext_p<192, 128, false, false>(a, big, wide, grid, s);
}
#else
hipError_t launch_extend(pka_dtype q, pka_dtype kv, int DK, int DV, const AttnArgs& a, hipStream_t s) {
    const int P = 1 << a.page_shift;
    const int tq = extend_tq(q, kv, a.G, P);
    const int64_t items = plan_ext_capacity(a.B, a.N, tq);
    if (items == 0) return hipSuccess;
    if (q == PKA_F32) {
        const dim3 grid((unsigned)items, (a.Hq + 3) / 4);
        if (DK == 128 && DV == 128) hipLaunchKernelGGL((extend_f32_kernel<128, 128>), grid, dim3(256), 0, s, a);
        else if (DK == 64 && DV == 64) hipLaunchKernelGGL((extend_f32_kernel<64, 64>), grid, dim3(256), 0, s, a);
        else if (DK == 192 && DV == 128) hipLaunchKernelGGL((extend_f32_kernel<192, 128>), grid, dim3(256), 0, s, a);
        else return hipErrorInvalidValue;
        return hipGetLastError();
    }
    const int C = a.ext_split;
    if (C < 1 || C > EXT_MAX_SPLIT) return hipErrorInvalidValue;
    if (items * a.Hkv * C * 64 * EXT_WAVES > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(items * a.Hkv * C));
    const bool pos = a.scale_log2 > 0.f;
    const bool big = P >= BN;
    // pages under 64 tokens gather rows by slot: 32-bit offsets while every
    // pool byte is within 4 GiB of the pool's base
    const int64_t row_bytes = (int64_t)a.Hkv * (DK > DV ? DK : DV) * (kv == PKA_FP8_E4M3FN ? 1 : 2);
    const bool wide = !big && a.pool_slots * row_bytes > (int64_t)UINT32_MAX;
    const bool f8 = kv == PKA_FP8_E4M3FN;
    if (DK == 128 && DV == 128) launch_ext_d<128, 128>(a, pos, big, wide, f8, grid, s);
    else if (DK == 64 && DV == 64) launch_ext_d<64, 64>(a, pos, big, wide, f8, grid, s);
    else if (DK == 192 && DV == 128 && f8) {
        if (pos) launch_ext_p<192, 128, true, true>(a, big, wide, grid, s);
        else launch_ext_p<192, 128, false, true>(a, big, wide, grid, s);
    } else if (DK == 192 && DV == 128) {
        launch_extend_dk192(a, pos, big, wide, grid, s);
    }
    else return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || C == 1) return e;
    const int64_t pairs = (int64_t)a.N * a.Hq;  // waves: one per (query row, head)
    const dim3 mgrid((unsigned)((pairs + 3) / 4));
    if (DV == 128) hipLaunchKernelGGL((extend_split_merge_kernel<128>), mgrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((extend_split_merge_kernel<64>), mgrid, dim3(256), 0, s, a);
    return hipGetLastError();
}
#endif

}  // namespace pka
