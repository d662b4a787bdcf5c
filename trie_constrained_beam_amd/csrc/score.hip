// gfx950 kernels of single-pass scoring of every valid SID.
//
// SPRINT summary (method and inference paragraphs): one forward pass gives, per user,
// an L x V table of per-position token distributions and a user vector; each valid SID
// of the catalog's prefix trie is scored by the sum of its tokens' log-probabilities
// plus a SID-level similarity (a table lookup plus one matrix product), the best K are
// kept, and the softmax runs over the valid SIDs only:
//   score(u, s) = sum_d T_u[d][c_d(s)] + w <v_u, e_s>,   lse(u) = log sum_s exp score(u, s)
//
// Three kernels:
//   k_score_table   each user's table, normalised per position when it holds raw logits,
//                   rewritten user-minor: [group][depth][code][user in group]
//   k_score_scan    one persistent 512-thread workgroup per CU and group of users (32 at
//                   L <= 4). The group's tables sit in LDS; each wave streams blocks of
//                   256 SIDs as 16 tiles of 16 (a tile is a group): token sums from LDS (a
//                   16-byte read gives 4 users), similarities from v_mfma_f32_16x16x32_bf16
//                   (16 users x 16 SIDs x 32 embedding elements per step, two user halves),
//                   SID codes and embeddings read once with nontemporal loads. It writes
//                   the best score of every group and of every block per user, and
//                   per-workgroup (max, sum of exp) partials of the log-normaliser.
//   k_score_select  one workgroup per user. Ranking is (score desc, SID asc) and groups
//                   and blocks are runs of consecutive SIDs, so the best K SIDs lie in the
//                   best K groups (ranked by their best score, then by position), and those
//                   in the best K blocks: if K groups ranked above a SID's group, each
//                   would hold a SID ranked above it. The kernel takes the exact top K of
//                   the blocks, then of the groups inside them, rescores the SIDs of the
//                   chosen groups with the very same arithmetic as the scan (same operands,
//                   same MFMA, same order of additions), takes their exact top K and sorts
//                   it. Every top-K is a radix selection on order-preserving keys with ties
//                   taken in ascending position, so the result is deterministic.
#include "score_internal.h"

namespace tcb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ uint32_t f2ord(float f) {   // order-preserving, -0 == +0
    const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord2f(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF,
                                                                 0xF, false));
}
// maximum over a row of 16 lanes, left in every lane of the row
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));     // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_f<0x4E>(v));     // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f<0x141>(v));    // row_half_mirror
    v = fmaxf(v, dpp_f<0x140>(v));    // row_mirror
    return v;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// (m, s) represents sum exp(x - m) = s over a set of scores; merging two sets is
// symmetric in its operands, so butterfly partners end with identical values.
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    if (M == kNegInf) {
        m = M;
        s = 0.0f;
        return;
    }
    s = s * exp2_fast(kLog2e * (m - M)) + s2 * exp2_fast(kLog2e * (m2 - M));
    m = M;
}

template <bool WIDE>
__device__ __forceinline__ uint64_t load_codes(const void *codes, int64_t leaf) {
    if constexpr (WIDE)
        return __builtin_nontemporal_load(static_cast<const uint64_t *>(codes) + leaf);
    else
        return __builtin_nontemporal_load(static_cast<const uint32_t *>(codes) + leaf);
}

// MFMA operands of the similarity tile (v_mfma_f32_16x16x32_bf16). Lane (j = lane & 15,
// g = lane >> 4) supplies, for k-step ks, 8 bf16 of row j: elements g D/4 + 8 ks ... + 7 of
// the vector, so a lane reads D/2 contiguous bytes over the k-steps. The user vectors
// (A, rows = users) and the SID embeddings (B, columns = SIDs) list the elements in the
// same order, and a dot product does not depend on that order.
template <int KS>
__device__ __forceinline__ void load_rows(const uint16_t *base, int64_t row, bool valid, int g,
                                          u32x4 (&v)[KS], bool stream) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(base + (size_t)row * (KS * 32) + g * (KS * 8));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (!valid)
            v[ks] = u32x4{0u, 0u, 0u, 0u};
        else if (stream)
            v[ks] = __builtin_nontemporal_load(p + ks);
        else
            v[ks] = p[ks];
    }
}

// D[user 4 g + e][SID j] in register e of lane (j, g)
template <int KS>
__device__ __forceinline__ f32x4 sim_tile(const u32x4 (&av)[KS], const u32x4 (&bv)[KS]) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[ks]),
                                                      __builtin_bit_cast(bf16x8, bv[ks]), acc, 0, 0, 0);
    return acc;
}

// Token sums of one SID for the lane's users: register 4 hh + e holds user row
// 16 hh + 4 g + e (the MFMA output layout, one 16-user half per hh), added level by
// level from 0.
template <int UG, int NR>
__device__ __forceinline__ void token_sums(const float *tbl, uint64_t cw, int L, int g, float (&s)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) s[r] = 0.0f;
    for (int d = 0; d < L; ++d) {
        const uint32_t c = (uint32_t)(cw >> (8 * d)) & 255u;
        const f32x4 *row = reinterpret_cast<const f32x4 *>(tbl + (size_t)(d * 256 + (int)c) * UG + 4 * g);
#pragma unroll
        for (int hh = 0; hh < NR / 4; ++hh) {
            const f32x4 v = row[4 * hh];
            s[4 * hh + 0] += v[0];
            s[4 * hh + 1] += v[1];
            s[4 * hh + 2] += v[2];
            s[4 * hh + 3] += v[3];
        }
    }
}

// ---------------------------------------------------------------------- table
// One wave per (padded user, depth): log-softmax over the V codes for raw logits;
// codes >= V and users >= U get 0.
__global__ __launch_bounds__(256) void k_score_table(ScoreDev a) {
    const int lane = threadIdx.x & 63;
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int UG = a.ug, L = a.L, V = a.V;
    if (wid >= a.groups * UG * L) return;
    const int d = wid % L, uu = wid / L;
    const int grp = uu / UG, row = uu % UG;
    const bool user = uu < a.U;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = lane * 4 + e;
        x[e] = (user && c < V) ? a.table_in[((size_t)uu * L + d) * V + c] : 0.0f;
    }
    if (a.kind == TCB_TABLE_LOGITS && user) {
        float m = kNegInf;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (lane * 4 + e < V) m = fmaxf(m, x[e]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (lane * 4 + e < V) sum += expf(x[e] - m);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
        const float lse = m + logf(sum);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (lane * 4 + e < V) x[e] -= lse;
    }
    float *out = a.table + ((size_t)grp * L + d) * 256 * UG + row;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[(size_t)(lane * 4 + e) * UG] = x[e];
}

// ---------------------------------------------------------------------- scan
template <bool WIDE, int KS, bool LSE>
__global__ __launch_bounds__(kScanThreads) void k_score_scan(ScoreDev a) {
    constexpr int UG = WIDE ? kScoreUGWide : kScoreUGNarrow;
    constexpr int NH = UG / 16;                       // 16-user halves of the group
    constexpr int NR = 4 * NH;                        // (user, SID) values per lane and tile
    constexpr int KA = KS > 0 ? KS : 1;
    constexpr int TPB = kScoreBlock / kScoreGroup;    // tiles (groups) per block
    __shared__ f32x4 tbl4[kScoreTableFloats / 4];
    __shared__ float2 part[kScanWaves][32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, g = lane >> 4;
    const int grp = blockIdx.y, L = a.L;
    const int64_t n = a.n, NG = (n + kScoreGroup - 1) / kScoreGroup, NB = (n + kScoreBlock - 1) / kScoreBlock;
    {
        const int nf4 = UG * L * 64;
        const f32x4 *src = reinterpret_cast<const f32x4 *>(a.table) + (size_t)grp * nf4;
        for (int i = tid; i < nf4; i += kScanThreads) tbl4[i] = src[i];
    }
    const float *tbl = reinterpret_cast<const float *>(tbl4);
    u32x4 av[NH][KA];
    if constexpr (KS > 0) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            const int user = grp * UG + 16 * hh + j;
            load_rows<KS>(a.user_vec, user, user < a.U, g, av[hh], false);
        }
    }
    float lm[NR], ls[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        lm[r] = kNegInf;
        ls[r] = 0.0f;
    }
    __syncthreads();
    const float w = a.w;
    float *gmax = a.gmax + (size_t)grp * NG * UG;
    float *bmax = a.bmax + (size_t)grp * NB * UG;
    const int wr = 16 * (j >> 2) + 4 * g + (j & 3);   // the user row whose maxima lane j < NR stores

    for (int64_t blk = (int64_t)blockIdx.x * kScanWaves + wave; blk < NB; blk += (int64_t)gridDim.x * kScanWaves) {
        float bm[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) bm[r] = kNegInf;
        uint64_t cw[2];
        u32x4 bv[2][KA];
        auto load_tile = [&](int t, int slot) {
            const int64_t leaf = blk * kScoreBlock + t * kScoreGroup + j;
            const bool valid = leaf < n;
            cw[slot] = valid ? load_codes<WIDE>(a.codes, leaf) : 0ull;
            if constexpr (KS > 0) load_rows<KS>(a.emb, leaf, valid, g, bv[slot], true);
        };
        auto tile = [&](int t, int slot) {
            const int64_t grp_id = blk * TPB + t;
            float s[NR];
            token_sums<UG, NR>(tbl, cw[slot], L, g, s);
            if constexpr (KS > 0) {
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    const f32x4 acc = sim_tile<KS>(av[hh], bv[slot]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[4 * hh + e] = fmaf(w, acc[e], s[4 * hh + e]);
                }
            }
            if (grp_id * kScoreGroup + j >= n) {
#pragma unroll
                for (int r = 0; r < NR; ++r) s[r] = kNegInf;
            }
            float gm[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) gm[r] = row16_max(s[r]);
            float v = gm[0];
#pragma unroll
            for (int r = 1; r < NR; ++r) v = j == r ? gm[r] : v;
            if (j < NR && grp_id < NG) gmax[grp_id * UG + wr] = v;
#pragma unroll
            for (int r = 0; r < NR; ++r) bm[r] = fmaxf(bm[r], gm[r]);
            if constexpr (LSE) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const float M = fmaxf(lm[r], gm[r]);
                    if (M > lm[r]) {
                        ls[r] *= exp2_fast(kLog2e * (lm[r] - M));
                        lm[r] = M;
                    }
                    if (M != kNegInf) ls[r] += exp2_fast(kLog2e * (s[r] - M));
                }
            }
        };
        load_tile(0, 0);
#pragma unroll 1
        for (int t = 0; t < TPB; t += 2) {
            load_tile(t + 1, 1);
            tile(t, 0);
            if (t + 2 < TPB) load_tile(t + 2, 0);
            tile(t + 1, 1);
        }
        float v = bm[0];
#pragma unroll
        for (int r = 1; r < NR; ++r) v = j == r ? bm[r] : v;
        if (j < NR) bmax[blk * UG + wr] = v;
    }

    if constexpr (LSE) {
        // the 16 lanes of a DPP row hold the same users: butterfly over them, then the
        // waves in order
#pragma unroll
        for (int r = 0; r < NR; ++r) {
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const float m2 = __shfl_xor(lm[r], o, 64), s2 = __shfl_xor(ls[r], o, 64);
                lse_merge(lm[r], ls[r], m2, s2);
            }
        }
        if (j == 0) {
#pragma unroll
            for (int r = 0; r < NR; ++r) part[wave][16 * (r >> 2) + 4 * g + (r & 3)] = make_float2(lm[r], ls[r]);
        }
        __syncthreads();
        if (tid < UG) {
            float m = part[0][tid].x, s = part[0][tid].y;
            for (int wv = 1; wv < kScanWaves; ++wv) lse_merge(m, s, part[wv][tid].x, part[wv][tid].y);
            float *o = a.lse_part + (((size_t)grp * gridDim.x + blockIdx.x) * UG + tid) * 2;
            o[0] = m;
            o[1] = s;
        }
    }
}

// ---------------------------------------------------------------------- select
constexpr int kSelWaves = kSelectThreads / 64;

struct SelSmem {
    uint32_t hist[256];
    uint32_t wcount[kSelWaves];
    uint32_t st[4];
};

// Exclusive count of set flags before this thread, over the workgroup; total in *total.
__device__ __forceinline__ uint32_t block_count_before(bool f, SelSmem &S, uint32_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t b = __ballot(f);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
    if (lane == 0) S.wcount[wave] = (uint32_t)__popcll(b);
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const uint32_t c = S.wcount[w];
        before += w < wave ? c : 0u;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + below;
}

// Exact top-k of n keys (a larger key is better; equal keys: the lower position first,
// 1 <= k <= n): writes the chosen positions, ascending, to out[0 .. k).
template <class Key>
__device__ void select_top(int k, int n, const Key &key, uint32_t *out, SelSmem &S) {
    const int tid = threadIdx.x, lane = tid & 63;
    uint32_t prefix = 0u, mask = 0u;
    uint32_t rem = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kSelectThreads) S.hist[i] = 0u;
        __syncthreads();
        for (int i = tid; i < n; i += kSelectThreads) {
            const uint32_t kv = key(i);
            if ((kv & mask) == prefix) atomicAdd(&S.hist[(kv >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l owns digits 255 - 4l ... 252 - 4l: counts from the top digit down
            uint32_t c[4], sum = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                c[e] = S.hist[255 - 4 * lane - e];
                sum += c[e];
            }
            uint32_t incl = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = (uint32_t)__shfl_up((int)incl, o, 64);
                if (lane >= o) incl += y;
            }
            const uint32_t excl = incl - sum;
            if (excl < rem && incl >= rem) {
                uint32_t cum = excl;
                bool done = false;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (!done && cum + c[e] >= rem) {
                        S.st[0] = (uint32_t)(255 - 4 * lane - e);
                        S.st[1] = cum;
                        done = true;
                    }
                    if (!done) cum += c[e];
                }
            }
        }
        __syncthreads();
        const uint32_t digit = S.st[0], above = S.st[1];
        rem -= above;
        prefix |= digit << shift;
        mask |= 255u << shift;
        __syncthreads();
    }
    // prefix is the k-th best key; take every key above it and the first rem equal to it
    uint32_t eq_seen = 0u, taken = 0u;
    for (int base = 0; base < n; base += kSelectThreads) {
        const int i = base + tid;
        const uint32_t kv = i < n ? key(i) : 0u;
        const bool eq = i < n && kv == prefix, gt = i < n && kv > prefix;
        uint32_t eq_tot, take_tot;
        const uint32_t eq_rank = eq_seen + block_count_before(eq, S, eq_tot);
        const bool take = gt || (eq && eq_rank < rem);
        const uint32_t pos = taken + block_count_before(take, S, take_tot);
        if (take && pos < (uint32_t)k) out[pos] = (uint32_t)i;
        eq_seen += eq_tot;
        taken += take_tot;
    }
    __syncthreads();
}

template <bool WIDE, int KS>
__global__ __launch_bounds__(kSelectThreads) void k_score_select(ScoreDev a) {
    constexpr int UG = WIDE ? kScoreUGWide : kScoreUGNarrow;
    constexpr int KA = KS > 0 ? KS : 1;
    constexpr int MK = TCB_SCORE_MAX_K;
    __shared__ float val[kScoreCand];
    __shared__ uint32_t listA[MK], listB[MK];
    __shared__ uint64_t sortk[MK];
    __shared__ SelSmem S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, g = lane >> 4;
    const int u = blockIdx.x, grp = u / UG, row = u % UG, L = a.L;
    const int64_t n = a.n, NG = (n + kScoreGroup - 1) / kScoreGroup, NB = (n + kScoreBlock - 1) / kScoreBlock;
    const int K = a.K;

    // 1. the best K blocks by their best score
    const float *bm = a.bmax + (size_t)grp * NB * UG + row;
    const int nA = (int)NB, kA = min(K, nA);
    select_top(kA, nA, [&](int i) { return f2ord(bm[(size_t)i * UG]); }, listA, S);

    // 2. the best K groups inside them
    const float *gm = a.gmax + (size_t)grp * NG * UG + row;
    const int nB = kScoreBlock / kScoreGroup * kA;
    for (int p = tid; p < nB; p += kSelectThreads) {
        const int64_t g = (int64_t)listA[p >> 4] * (kScoreBlock / kScoreGroup) + (p & 15);
        val[p] = g < NG ? gm[(size_t)g * UG] : kNegInf;
    }
    __syncthreads();
    const int kB = min(K, nB);
    select_top(kB, nB, [&](int i) { return f2ord(val[i]); }, listB, S);
    for (int q = tid; q < kB; q += kSelectThreads) {
        const uint32_t p = listB[q];
        listB[q] = listA[p >> 4] * (uint32_t)(kScoreBlock / kScoreGroup) + (p & 15u);
    }
    __syncthreads();

    // 3. rescore the SIDs of those groups: one 16-SID MFMA tile per group; only the
    //    16-user half holding this user is multiplied (its result does not depend on
    //    the other half)
    const int hh_u = row >> 4, g_u = (row >> 2) & 3, e_u = row & 3;
    u32x4 av[KA];
    if constexpr (KS > 0) {
        const int user = grp * UG + 16 * hh_u + j;
        load_rows<KS>(a.user_vec, user, user < a.U, g, av, false);
    }
    const float *tg = a.table + (size_t)grp * L * 256 * UG + row;
    for (int q = wave; q < kB; q += kSelWaves) {
        const int64_t leaf = (int64_t)listB[q] * kScoreGroup + j;
        const bool valid = leaf < n;
        const uint64_t cw = valid ? load_codes<WIDE>(a.codes, leaf) : 0ull;
        float s = 0.0f;
        for (int d = 0; d < L; ++d) s += tg[(size_t)(d * 256 + (int)((cw >> (8 * d)) & 255u)) * UG];
        if constexpr (KS > 0) {
            u32x4 bv[KA];
            load_rows<KS>(a.emb, leaf, valid, g, bv, false);
            const f32x4 acc = sim_tile<KS>(av, bv);
            const float x = e_u == 0 ? acc[0] : e_u == 1 ? acc[1] : e_u == 2 ? acc[2] : acc[3];
            s = fmaf(a.w, x, s);
        }
        if (!valid) s = kNegInf;
        if (g == g_u) val[q * kScoreGroup + j] = s;
    }
    __syncthreads();

    // 4. the best K SIDs, then sorted by (score desc, SID asc)
    const int nC = kScoreGroup * kB;
    const int kC = (int)min((int64_t)K, n);
    select_top(kC, nC, [&](int i) { return f2ord(val[i]); }, listA, S);
    int P2 = 1;
    while (P2 < kC) P2 <<= 1;
    for (int i = tid; i < P2; i += kSelectThreads) {
        uint64_t key = ~0ull;
        if (i < kC) {
            const uint32_t p = listA[i];
            const uint32_t leaf = listB[p >> 4] * (uint32_t)kScoreGroup + (p & 15u);
            key = ((uint64_t)(~f2ord(val[p])) << 32) | leaf;
        }
        sortk[i] = key;
    }
    __syncthreads();
    for (int size = 2; size <= P2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < P2 / 2; i += kSelectThreads) {
                const int lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
                const bool up = (lo & size) == 0;
                const uint64_t x = sortk[lo], y = sortk[hi];
                if ((x > y) == up) {
                    sortk[lo] = y;
                    sortk[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < K; i += kSelectThreads) {
        int32_t leaf = -1, item = -1;
        float sc = kNegInf;
        if (i < kC) {
            const uint64_t key = sortk[i];
            leaf = (int32_t)(uint32_t)key;
            sc = ord2f(~(uint32_t)(key >> 32));
            item = (int64_t)leaf < n ? a.leaf_item[leaf] : -1;
        }
        a.out_leaf[(size_t)u * K + i] = leaf;
        a.out_score[(size_t)u * K + i] = sc;
        if (a.out_item) a.out_item[(size_t)u * K + i] = item;
    }

    // 5. log-normaliser of the softmax over every valid SID: scan partials in order
    if (a.out_lse && wave == 0) {
        const float *pp = a.lse_part + ((size_t)grp * kScanWGs * UG + row) * 2;
        float m = kNegInf, s = 0.0f;
        for (int b = lane; b < kScanWGs; b += 64) lse_merge(m, s, pp[(size_t)b * UG * 2], pp[(size_t)b * UG * 2 + 1]);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
            lse_merge(m, s, m2, s2);
        }
        if (lane == 0) a.out_lse[u] = m + logf(s);
    }
}

template <bool WIDE, int KS>
hipError_t launch_ks(const ScoreDev &a, hipStream_t s, const hipEvent_t *ev) {
    const dim3 scan_grid(kScanWGs, a.groups);
    if (ev) (void)hipEventRecord(ev[1], s);
    if (a.out_lse)
        hipLaunchKernelGGL((k_score_scan<WIDE, KS, true>), scan_grid, dim3(kScanThreads), 0, s, a);
    else
        hipLaunchKernelGGL((k_score_scan<WIDE, KS, false>), scan_grid, dim3(kScanThreads), 0, s, a);
    if (ev) (void)hipEventRecord(ev[2], s);
    hipLaunchKernelGGL((k_score_select<WIDE, KS>), dim3(a.U), dim3(kSelectThreads), 0, s, a);
    if (ev) (void)hipEventRecord(ev[3], s);
    return hipGetLastError();
}

template <bool WIDE>
hipError_t launch_w(const ScoreDev &a, hipStream_t s, const hipEvent_t *ev) {
    switch (a.user_vec ? a.D / 32 : 0) {
    case 0: return launch_ks<WIDE, 0>(a, s, ev);
    case 1: return launch_ks<WIDE, 1>(a, s, ev);
    case 2: return launch_ks<WIDE, 2>(a, s, ev);
    case 4: return launch_ks<WIDE, 4>(a, s, ev);
    case 8: return launch_ks<WIDE, 8>(a, s, ev);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

ScoreLayout score_layout(int L, int64_t n, int max_users) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const int UG = score_ug(L);
    const size_t groups = (size_t)((max_users + UG - 1) / UG);
    const size_t NG = (size_t)((n + kScoreGroup - 1) / kScoreGroup), NB = (size_t)((n + kScoreBlock - 1) / kScoreBlock);
    ScoreLayout o;
    o.table = 0;
    o.gmax = al(o.table + groups * L * 256 * UG * 4);
    o.bmax = al(o.gmax + groups * NG * UG * 4);
    o.lse = al(o.bmax + groups * NB * UG * 4);
    o.total = al(o.lse + groups * kScanWGs * UG * 8);
    return o;
}

hipError_t launch_score(const ScoreDev &a, hipStream_t s, const hipEvent_t *ev) {
    const int waves = a.groups * a.ug * a.L;
    if (ev) (void)hipEventRecord(ev[0], s);
    hipLaunchKernelGGL(k_score_table, dim3((waves + 3) / 4), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return a.L > 4 ? launch_w<true>(a, s, ev) : launch_w<false>(a, s, ev);
}

}  // namespace tcb
