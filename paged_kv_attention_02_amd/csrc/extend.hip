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
// K/V tile staged in LDS feeds 128 columns.  Per 32-key tile and wave:
//   S^T[key, col] = K . Q^T      8 x v_mfma_f32_32x32x16_bf16 (D = 128)
//   O^T[d, col]  += V^T . P^T    8 x v_mfma_f32_32x32x16_bf16
// Column statistics of the online softmax live in the lane (two lanes per
// column), P^T is used in place as the B operand, and V^T is built from
// 8-byte LDS row reads with v_perm_b32.  K/V tiles are double-buffered in LDS
// (next tile's global loads are in flight during the current tile's MFMAs).
#include <type_traits>

#include "pka_internal.h"

namespace pka {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float LN2 = 0.69314718055994531f;
constexpr int EXT_COLS = 128;  // query columns per workgroup (4 waves x 32)
constexpr int BN = 64;         // keys per tile (two 32-key MFMA blocks)

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

// Direct HBM -> LDS load of 16 bytes per lane: lane i's bytes land at
// lds_dst + 16 * i (lds_dst is wave-uniform).  Issued as a plain instruction
// the compiler does not track: the caller orders it with an explicit
// vmcnt(0) wait and a barrier before any wave reads the destination.
__device__ inline void lds_dma16(const void* src, const uint8_t* lds_dst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
    // one wait state between the M0 write and the LDS-DMA instruction reading it
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "m0");
}

// LDS tiles: BN keys x D dims of K and of V, rows of 16-byte chunks with no
// padding, filled by direct HBM -> LDS loads (each lane's 16 bytes land at
// base + 16 * lane).  Chunks are XOR-swizzled per row so the reads are
// bank-conflict free: K is read 16 rows x one chunk at a time (chunk ^ row),
// V by the transposing loads, 4 rows x 4 chunks at a time
// (chunk ^ 4 * (row % 4)).
template <int D> struct ExtTile {
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row (bf16)
    static constexpr int ROWB = D * 2;
    static constexpr int TILEB = BN * ROWB;            // bytes of one K or V tile
    static constexpr int LOADS = TILEB / (256 * 16);   // DMA instructions per thread per tile
    __device__ static constexpr int kchunk(int row, int c) { return c ^ (row & (CPR - 1)); }
    __device__ static constexpr int vchunk(int row, int c) { return c ^ ((4 * (row & 3)) & (CPR - 1)); }
};

template <int D, bool POS>
__global__ __launch_bounds__(256) void extend_mfma_kernel(AttnArgs a) {
    using T = ExtTile<D>;
    constexpr int KSTEPS = D / 16;           // k-steps of q.k (32x32x16)
    constexpr int VC = D / 32;               // 32-dim blocks of O^T (d = 32 c + row)
    constexpr int SB = BN / 32;              // 32-key score blocks per tile
    constexpr int ROWS_PER_LOAD = 64 / T::CPR;  // rows one wave instruction fills
    // one LDS object per stage and tensor, so the compiler can tell a tile
    // being read from the next tile's direct loads
    __shared__ __attribute__((aligned(1024))) uint8_t sK0[T::TILEB], sK1[T::TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t sV0[T::TILEB], sV1[T::TILEB];

    const int32_t* plan = a.plan;
    const int32_t item = blockIdx.x;
    if (item >= plan[PLAN_EXT_COUNT]) return;
    const int32_t TQ = plan[PLAN_EXT_TQ];
    const int32_t* items = plan + plan_ext_items(a.B);
    const int32_t b = items[2 * item], ti = items[2 * item + 1];
    const int32_t g = blockIdx.y;
    const int32_t* F = plan + plan_seg_prefix(a.B);
    const int32_t q0 = a.qo_indptr[b];
    const int32_t nb = a.qo_indptr[b + 1] - q0;
    const int32_t L = F[b + 1] - F[b];
    const int32_t pb = L - nb;
    const int32_t tok_lo = ti * TQ;
    const int32_t tok_hi = min(tok_lo + TQ, nb);
    const int32_t page_base = a.kv_indptr[b];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
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
        const __bf16* qrow = (const __bf16*)a.q + ((int64_t)qr * a.Hq + head) * D;
        #pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qop[s] = as_bf16x8(*(const u32x4_t*)(qrow + 16 * s + 8 * hh));
    }

    const int32_t kend = pb + tok_hi;  // keys 0 .. kend-1
    const int32_t ntiles = (kend + BN - 1) / BN;
    const int64_t row_bytes = (int64_t)a.Hkv * T::ROWB;
    const uint8_t* kbase = (const uint8_t*)a.k_pool + (int64_t)g * T::ROWB;
    const uint8_t* vbase = (const uint8_t*)a.v_pool + (int64_t)g * T::ROWB;
    const int32_t P = 1 << a.page_shift;

    // Direct loads of one tile.  Wave instruction j of wave w fills rows
    // ROWS_PER_LOAD * (LOADS * w + j) .. ; lane i writes physical chunk
    // i % CPR of its row, so it fetches the logical chunk that the swizzle
    // places there.  Rows past the last key repeat it.  The pool slots of a
    // tile's rows are looked up one tile ahead (slots_for), so the loads
    // issue without waiting.
    // raw page ids of the tile's rows (clamped and combined at use, a tile
    // later, so nothing waits for these loads now)
    auto slots_for = [&](int32_t kt0, int32_t (&pg)[T::LOADS], int32_t (&kp)[T::LOADS]) {
        #pragma unroll
        for (int j = 0; j < T::LOADS; ++j) {
            const int row = ROWS_PER_LOAD * (T::LOADS * wave + j) + lane / T::CPR;
            kp[j] = min(kt0 + row, kend - 1);
            int64_t idx = (int64_t)page_base + (kp[j] >> a.page_shift);
            idx = idx < a.kv_cap ? idx : a.kv_cap - 1;
            pg[j] = a.kv_indices[idx];
        }
    };
    auto load_tile = [&](const int32_t (&pg)[T::LOADS], const int32_t (&kp)[T::LOADS], uint8_t* dk,
                         uint8_t* dv) {
        #pragma unroll
        for (int j = 0; j < T::LOADS; ++j) {
            const int row = ROWS_PER_LOAD * (T::LOADS * wave + j) + lane / T::CPR;
            const int pc = lane % T::CPR;
            const int32_t page = min(max(pg[j], 0), a.num_pages - 1);
            const int64_t slot = ((int64_t)page << a.page_shift) | (kp[j] & (P - 1));
            const int64_t off = slot * row_bytes;
            const int ldsb = (T::LOADS * wave + j) * 1024;
            lds_dma16(kbase + off + 16 * T::kchunk(row, pc), dk + ldsb);
            lds_dma16(vbase + off + 16 * T::vchunk(row, pc), dv + ldsb);
        }
    };
    // V^T operand: lane group G = lane/16 reads keys 4 (G/2) + s16/4 (+ 16 ks
    // + 8 r) at dims 16 (G%2) + 4 (s16%4) (+ 32 c) with the transposing load.
    const int G16 = lane >> 4, s16 = lane & 15;
    const int v_row = 4 * (G16 >> 1) + (s16 >> 2);
    const int v_byte = 32 * (G16 & 1) + 8 * (s16 & 3);  // byte within the 64-byte group of block c
    // K operand: lane (n, hh) reads row 32 u + n, logical chunk 2 s + hh

    f32x16_t O[VC];
    #pragma unroll
    for (int c = 0; c < VC; ++c)
        #pragma unroll
        for (int r = 0; r < 16; ++r) O[c][r] = 0.f;
    float m2 = -INFINITY, lsum = 0.f;
    const float c2 = a.scale_log2;
    const uint32_t ones = 0x3f803f80u;  // two bf16 1.0

    // One tile: wait for its loads, start the next tile's loads into the
    // other stage, then scores -> probabilities -> O += P.V.
    int32_t pgs[T::LOADS], kps[T::LOADS];
    auto tile = [&](int32_t t, const uint8_t* ks_, const uint8_t* vs_, uint8_t* kn, uint8_t* vn) {
        const int32_t kt0 = t * BN;
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this tile's loads (and the slots) have landed
        __syncthreads();                       // ... for every wave; the other stage is free
        if (t + 1 < ntiles) {
            load_tile(pgs, kps, kn, vn);
            slots_for(kt0 + 2 * BN, pgs, kps);
        }

        // S^T = K . Q^T, SB independent 32-key blocks
        f32x16_t S[SB];
        #pragma unroll
        for (int u = 0; u < SB; ++u)
            #pragma unroll
            for (int r = 0; r < 16; ++r) S[u][r] = 0.f;
        #pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
            #pragma unroll
            for (int u = 0; u < SB; ++u) {
                const int row = 32 * u + n;
                const u32x4_t kw = *(const u32x4_t*)(ks_ + row * T::ROWB + 16 * T::kchunk(row, 2 * s + hh));
                S[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw), qop[s], S[u], 0, 0, 0);
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

        // probabilities in bf16 (the normaliser sums the same rounded values),
        // then O^T += V^T . P^T in k-steps of 16 keys.  A column has a valid
        // key in every tile up to its own position, and tiles start at key 0,
        // so m2 is finite from the first tile on.
        #pragma unroll
        for (int u = 0; u < SB; ++u) {
            uint32_t pw[8];
            #pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float e0 = POS ? __builtin_fmaf(S[u][2 * i], c2, -m2) : S[u][2 * i] - m2;
                const float e1 = POS ? __builtin_fmaf(S[u][2 * i + 1], c2, -m2) : S[u][2 * i + 1] - m2;
                pw[i] = pack_bf16(__builtin_amdgcn_exp2f(e0), __builtin_amdgcn_exp2f(e1));
                lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[i]),
                                                        __builtin_bit_cast(bf16x2_t, ones), lsum, false);
            }
            #pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int ks = 2 * u + k2;
                const bf16x8_t pop = as_bf16x8(u32x4_t{pw[4 * k2], pw[4 * k2 + 1], pw[4 * k2 + 2], pw[4 * k2 + 3]});
                #pragma unroll
                for (int c = 0; c < VC; ++c) {
                    u32x2_t half[2];
                    #pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const int row = 16 * ks + 8 * r + v_row;
                        const int lc = 4 * c + (v_byte >> 4);
                        const uint8_t* p = vs_ + row * T::ROWB + 16 * T::vchunk(row, lc) + (v_byte & 15);
                        half[r] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
                    }
                    const u32x4_t av = {half[0][0], half[0][1], half[1][0], half[1][1]};
                    O[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), pop, O[c], 0, 0, 0);
                }
            }
        }
        };

    slots_for(0, pgs, kps);
    load_tile(pgs, kps, sK0, sV0);
    slots_for(BN, pgs, kps);
    for (int32_t t = 0; t < ntiles; t += 2) {
        tile(t, sK0, sV0, sK1, sV1);
        if (t + 1 >= ntiles) break;
        tile(t + 1, sK1, sV1, sK0, sV0);
    }

    // finish: the two lanes of a column hold halves of the sums
    const float ltot = sum_halves(lsum);
    if (!col_ok) return;
    const float inv = 1.0f / ltot;
    __bf16* orow = (__bf16*)a.out + ((int64_t)(q0 + ctok) * a.Hq + head) * D;
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
template <int D>
__global__ __launch_bounds__(256) void extend_f32_kernel(AttnArgs a) {
    constexpr int EPL = D / 64;
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
        float q[EPL], o[EPL];
        #pragma unroll
        for (int e = 0; e < EPL; ++e) {
            q[e] = ((const float*)a.q)[((int64_t)(q0 + i) * a.Hq + h) * D + e * 64 + lane];
            o[e] = 0.f;
        }
        float m = -INFINITY, l = 0.f;
        for (int32_t t = 0; t <= pb + i; ++t) {
            const int64_t base = ((int64_t)slot_of(a, page_base, t) * a.Hkv + g) * D;
            float dot = 0.f;
            #pragma unroll
            for (int e = 0; e < EPL; ++e) dot += q[e] * ((const float*)a.k_pool)[base + e * 64 + lane];
            #pragma unroll
            for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
            const float s = dot * a.scale_log2;
            const float mn = fmaxf(m, s);
            const float al = __builtin_amdgcn_exp2f(m - mn);
            const float p = __builtin_amdgcn_exp2f(s - mn);
            m = mn;
            l = l * al + p;
            #pragma unroll
            for (int e = 0; e < EPL; ++e)
                o[e] = o[e] * al + p * ((const float*)a.v_pool)[base + e * 64 + lane];
        }
        #pragma unroll
        for (int e = 0; e < EPL; ++e)
            ((float*)a.out)[((int64_t)(q0 + i) * a.Hq + h) * D + e * 64 + lane] = o[e] / l;
        if (a.lse && lane == 0)
            a.lse[(int64_t)(q0 + i) * a.Hq + h] = (m + __builtin_amdgcn_logf(l)) * LN2;
    }
}

}  // namespace

int extend_tq(pka_dtype q, pka_dtype /*kv*/, int /*D*/, int G) {
    if (q == PKA_F32) return 16;
    return G >= EXT_COLS ? 1 : EXT_COLS / G;
}

hipError_t launch_extend(pka_dtype q, pka_dtype kv, int D, const AttnArgs& a, hipStream_t s) {
    const int tq = extend_tq(q, kv, D, a.G);
    const int64_t items = plan_ext_capacity(a.B, a.N, tq);
    if (items == 0) return hipSuccess;
    if (q == PKA_F32) {
        const dim3 grid((unsigned)items, (a.Hq + 3) / 4);
        if (D == 128) hipLaunchKernelGGL((extend_f32_kernel<128>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((extend_f32_kernel<64>), grid, dim3(256), 0, s, a);
    } else {
        const dim3 grid((unsigned)items, a.Hkv);
        const bool pos = a.scale_log2 > 0.f;
        if (D == 128) {
            if (pos) hipLaunchKernelGGL((extend_mfma_kernel<128, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((extend_mfma_kernel<128, false>), grid, dim3(256), 0, s, a);
        } else {
            if (pos) hipLaunchKernelGGL((extend_mfma_kernel<64, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((extend_mfma_kernel<64, false>), grid, dim3(256), 0, s, a);
        }
    }
    return hipGetLastError();
}

}  // namespace pka
