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
constexpr int KT = 32;         // keys per tile (one 32-key MFMA block; keeps two waves per SIMD)

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
// skip the rescale; p = 2^(s*c - m) then stays below 2^LAZY.
constexpr float LAZY = 8.0f;

template <int D, bool POS>
__global__ __launch_bounds__(256) void extend_mfma_kernel(AttnArgs a) {
    constexpr int ROWB = D * 2;              // bytes of one K/V row of one head
    constexpr int STRIDE = ROWB + 16;        // LDS row stride (padding against bank conflicts)
    constexpr int CH = ROWB / 16;            // 16-byte chunks per row
    constexpr int RPP = 256 / CH;            // rows per cooperative pass
    constexpr int PASSES = KT / RPP;         // passes per tile and tensor
    constexpr int KSTEPS = D / 16;           // k-steps of q.k (32x32x16)
    constexpr int VC = D / 32;               // d-row blocks of O^T (d = VC*m + c)
    constexpr int SUB = KT / 32;             // 32-key sub-tiles per tile
    __shared__ __attribute__((aligned(16))) uint8_t sK[2][KT * STRIDE];
    __shared__ __attribute__((aligned(16))) uint8_t sV[2][KT * STRIDE];

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
    const int32_t ntiles = (kend + KT - 1) / KT;
    const int64_t row_bytes = (int64_t)a.Hkv * ROWB;
    const uint8_t* kbase = (const uint8_t*)a.k_pool + (int64_t)g * ROWB;
    const uint8_t* vbase = (const uint8_t*)a.v_pool + (int64_t)g * ROWB;
    const int lrow = tid / CH, lch = tid % CH;

    u32x4_t kreg[PASSES], vreg[PASSES];
    auto load_tile = [&](int32_t kt0) {
        #pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            int32_t kp = kt0 + p * RPP + lrow;
            kp = kp < kend ? kp : kend - 1;
            const int64_t off = (int64_t)slot_of(a, page_base, kp) * row_bytes + lch * 16;
            kreg[p] = *(const u32x4_t*)(kbase + off);
            vreg[p] = *(const u32x4_t*)(vbase + off);
        }
    };
    auto store_tile = [&](int buf) {
        #pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int r = p * RPP + lrow;
            *(u32x4_t*)(&sK[buf][r * STRIDE + lch * 16]) = kreg[p];
            *(u32x4_t*)(&sV[buf][r * STRIDE + lch * 16]) = vreg[p];
        }
    };

    f32x16_t O[VC];
    #pragma unroll
    for (int c = 0; c < VC; ++c)
        #pragma unroll
        for (int r = 0; r < 16; ++r) O[c][r] = 0.f;
    float m2 = -INFINITY, lsum = 0.f;
    // POS: scores are scaled by c > 0 inside one FMA, so the max is taken on
    // raw scores; otherwise the scaled scores are formed first.
    const float c2 = a.scale_log2;

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int32_t t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int32_t kt0 = t * KT;
        if (t + 1 < ntiles) load_tile(kt0 + KT);

        // S^T = K . Q^T for each 32-key sub-tile
        f32x16_t S[SUB];
        #pragma unroll
        for (int u = 0; u < SUB; ++u) {
            #pragma unroll
            for (int r = 0; r < 16; ++r) S[u][r] = 0.f;
            const uint8_t* krow = &sK[buf][(32 * u + n) * STRIDE + 16 * hh];
            #pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const u32x4_t kw = *(const u32x4_t*)(krow + 32 * s);
                S[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kw), qop[s], S[u], 0, 0, 0);
            }
        }

        // causal mask only where the tile crosses the diagonal of some column
        if (kt0 + KT - 1 > qpos_min) {
            #pragma unroll
            for (int u = 0; u < SUB; ++u)
                #pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kt0 + 32 * u + acc_row(r, hh) > qpos) S[u][r] = -INFINITY;
        }
        if constexpr (!POS) {
            #pragma unroll
            for (int u = 0; u < SUB; ++u)
                #pragma unroll
                for (int r = 0; r < 16; ++r) S[u][r] = S[u][r] == -INFINITY ? -INFINITY : S[u][r] * c2;
        }
        float mx = -INFINITY;
        #pragma unroll
        for (int u = 0; u < SUB; ++u)
            #pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[u][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mc = POS ? mx * c2 : mx;  // candidate max, log2 units
        if (__any(mc > m2 + LAZY)) {
            const float mnew = fmaxf(m2, mc);
            const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
            m2 = mnew;
            lsum *= alpha;
            #pragma unroll
            for (int c = 0; c < VC; ++c) O[c] *= alpha;
        }
        // a column has a valid key in every tile up to its own position, and
        // tiles start at key 0, so m2 is finite from the first tile on
        #pragma unroll
        for (int u = 0; u < SUB; ++u)
            #pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = POS ? __builtin_fmaf(S[u][r], c2, -m2) : S[u][r] - m2;
                S[u][r] = __builtin_amdgcn_exp2f(e);
                lsum += S[u][r];
            }

        // O^T += V^T . P^T in k-steps of 16 keys
        #pragma unroll
        for (int ks = 0; ks < 2 * SUB; ++ks) {
            const f32x16_t& P = S[ks >> 1];
            const int r0 = 8 * (ks & 1);
            const u32x4_t pw = {pack_bf16(P[r0 + 0], P[r0 + 1]), pack_bf16(P[r0 + 2], P[r0 + 3]),
                                pack_bf16(P[r0 + 4], P[r0 + 5]), pack_bf16(P[r0 + 6], P[r0 + 7])};
            const bf16x8_t pop = as_bf16x8(pw);
            // key of B-operand slot e (lane half hh): 16 ks + 8 (e/4) + 4 hh + e%4
            typedef typename std::conditional<VC == 4, u32x2_t, uint32_t>::type vrow_t;
            vrow_t R[8];
            #pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = 16 * ks + 8 * (e >> 2) + 4 * hh + (e & 3);
                R[e] = *(const vrow_t*)(&sV[buf][key * STRIDE + n * (VC * 2)]);
            }
            #pragma unroll
            for (int c = 0; c < VC; ++c) {
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                u32x4_t av;
                #pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t lo_w, hi_w;
                    if constexpr (VC == 4) {
                        lo_w = R[2 * w][c >> 1];
                        hi_w = R[2 * w + 1][c >> 1];
                    } else {
                        lo_w = R[2 * w];
                        hi_w = R[2 * w + 1];
                    }
                    av[w] = __builtin_amdgcn_perm(hi_w, lo_w, sel);
                }
                O[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), pop, O[c], 0, 0, 0);
            }
        }

        if (t + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    }

    // finish: two lanes per column hold halves of the keys' sums
    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (!col_ok) return;
    const float inv = 1.0f / ltot;
    __bf16* orow = (__bf16*)a.out + ((int64_t)(q0 + ctok) * a.Hq + head) * D;
    #pragma unroll
    for (int r = 0; r < 16; r += 4) {
        // rows acc_row(r..r+3, hh) are consecutive: dims VC*m .. VC*(m+4)-1
        const int m0 = acc_row(r, hh);
        float v[4 * VC];
        #pragma unroll
        for (int i = 0; i < 4; ++i)
            #pragma unroll
            for (int c = 0; c < VC; ++c) v[i * VC + c] = O[c][r + i] * inv;
        #pragma unroll
        for (int i = 0; i < 4 * VC; i += 8) {
            const u32x4_t pk = {pack_bf16(v[i], v[i + 1]), pack_bf16(v[i + 2], v[i + 3]),
                                pack_bf16(v[i + 4], v[i + 5]), pack_bf16(v[i + 6], v[i + 7])};
            *(u32x4_t*)(orow + VC * m0 + i) = pk;
        }
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
