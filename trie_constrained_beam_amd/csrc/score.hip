// gfx950 kernels of single-pass scoring of every valid SID.
//
// SPRINT summary (method and inference paragraphs): one forward pass gives, per user,
// an L x V table of per-position token distributions and a user vector; each valid SID
// of the catalog's prefix trie is scored by the sum of its tokens' log-probabilities
// plus a SID-level similarity (a table lookup plus one matrix product), the best K are
// kept, and the softmax runs over the valid SIDs only:
//   score(u, s) = sum_d T_u[d][c_d(s)] + w <v_u, e_s>,   lse(u) = log sum_s exp score(u, s)
//
// Four kernels:
//   k_score_scan    one persistent 512-thread workgroup per CU and group of users (32 at
//                   L <= 4). The group's tables, normalised per position when they hold
//                   raw logits, sit in LDS user-minor ([depth][code][user], so a 16-byte
//                   read gives 4 users); each wave streams blocks of
//                   256 SIDs as 16 tiles of 16 (a tile is a group), several tiles of loads
//                   in flight: token sums from LDS, similarities from v_mfma_f32_16x16x32_bf16
//                   (16 users x 16 SIDs x 32 embedding elements per step, two user halves),
//                   SID codes and embeddings read once with nontemporal loads. It writes
//                   the best score of every group and of every block per user, and
//                   per-workgroup (max, sum of exp) partials of the log-normaliser.
//   k_score_pick    one workgroup per user. Ranking is (score desc, SID asc) and groups,
//                   blocks and superblocks (16 blocks) are runs of consecutive SIDs, so the
//                   best K SIDs lie in the best K groups (ranked by their best score, then
//                   by position), those in the best K blocks, and those in the best K
//                   superblocks: if K groups ranked above a SID's group, each would hold a
//                   SID ranked above it. It takes the exact top K of the superblocks, then
//                   of the blocks and of the groups inside them (at most 16384 blocks: the
//                   top K of all blocks directly).
//   k_score_rescore rescores the SIDs of the chosen groups with the very same arithmetic as
//                   the scan (same operands, same MFMA, same order of additions).
//   k_score_final   one workgroup per user: the exact top K of the rescored SIDs, sorted,
//                   and the log-normaliser from the scan's partials.
// Every top-K is a radix selection on order-preserving keys with ties taken in ascending
// position, so the result is deterministic.
#include <mutex>
#include <type_traits>

#include "score_internal.h"

namespace tcb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;
// score of a lane past the last SID in the scan: below any real score, but finite, so
// that it needs no special case in the running sums of exp
constexpr float kPastEnd = -1.0e30f;

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
using CodeWord = typename std::conditional<WIDE, uint64_t, uint32_t>::type;

template <bool WIDE>
__device__ __forceinline__ CodeWord<WIDE> load_codes(const void *codes, int64_t leaf) {
    return __builtin_nontemporal_load(static_cast<const CodeWord<WIDE> *>(codes) + leaf);
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
// level from 0 over LP levels (levels past L hold zero rows and code 0). The LDS row of
// (depth d, code c) starts at (256 d + c) * ST; row 256 LP holds kPastEnd, read at depth 0
// by lanes past the last SID so that their scores come out below every real one without a
// per-value select.
template <int NR, int LP, int ST, class W>
__device__ __forceinline__ void token_sums(const float *tbl, W cw, bool valid, int g, float (&s)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) s[r] = 0.0f;
#pragma unroll
    for (int d = 0; d < LP; ++d) {
        const uint32_t c = (uint32_t)(cw >> (8 * d)) & 255u;
        const int rix = (d == 0 && !valid) ? LP * 256 : d * 256 + (int)c;   // past the end: the -inf row
        const f32x4 *row = reinterpret_cast<const f32x4 *>(tbl + rix * ST + 4 * g);
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

// Maximum over the 16 lanes of a DPP row for each of a lane's NR values (NR = 8 or 4,
// one per user), by a transposed butterfly: each exchange halves the values a lane keeps,
// so 8 values need 4 + 2 + 1 + 1 moves instead of 8 x 4. The pairings are xor 1, xor 2,
// row_half_mirror (i <-> 7 - i) and row_mirror (i <-> 15 - i); the half a lane keeps is
// chosen by c0 = b0^b2, c1 = b1^b2, c2 = b2^b3 (b = bits of its lane in the row), which
// makes every partner hold the same users. Lane j ends with the maximum of register
// reduced_reg(j); lanes j and 15 - j hold the same one.
template <int NR>
__device__ __forceinline__ int reduced_reg(int j) {
    const int b0 = j & 1, b1 = (j >> 1) & 1, b2 = (j >> 2) & 1, b3 = (j >> 3) & 1;
    if constexpr (NR == 8)
        return 4 * (b0 ^ b2) + 2 * (b1 ^ b2) + (b2 ^ b3);
    else
        return 2 * (b0 ^ b2) + (b1 ^ b2);
}

template <int NR>
__device__ __forceinline__ float transposed_max(const float (&v)[NR], int j) {
    const bool c0 = ((j ^ (j >> 2)) & 1) != 0, c1 = (((j >> 1) ^ (j >> 2)) & 1) != 0;
    constexpr int H = NR / 2;
    float w[H];
#pragma unroll
    for (int r = 0; r < H; ++r) {
        const float keep = c0 ? v[r + H] : v[r], send = c0 ? v[r] : v[r + H];
        w[r] = fmaxf(keep, dpp_f<0xB1>(send));                // xor 1
    }
    constexpr int Q = H / 2;
    float x[Q];
#pragma unroll
    for (int r = 0; r < Q; ++r) {
        const float keep = c1 ? w[r + Q] : w[r], send = c1 ? w[r] : w[r + Q];
        x[r] = fmaxf(keep, dpp_f<0x4E>(send));                // xor 2
    }
    float y;
    if constexpr (NR == 8) {
        const bool c2 = (((j >> 2) ^ (j >> 3)) & 1) != 0;
        const float keep = c2 ? x[1] : x[0], send = c2 ? x[0] : x[1];
        y = fmaxf(keep, dpp_f<0x141>(send));                  // row_half_mirror
    } else {
        y = fmaxf(x[0], dpp_f<0x141>(x[0]));
    }
    return fmaxf(y, dpp_f<0x140>(y));                         // row_mirror
}


// ---------------------------------------------------------------------- tables
// the value lane l holds (l wave-uniform)
__device__ __forceinline__ float lane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// The group's tables into LDS, normalised per position for raw logits (log-softmax over
// the V codes); codes >= V and users >= U get 0. The rows (depth, user) are dealt to the
// waves in chunks of 16 consecutive users of one depth (chunk k: depth k mod LP, users
// 16 (k / LP) ...); a wave issues the loads of all its rows at once (lane l holds codes
// l + 64 e), and after normalising writes, per code, each chunk's 16 values as four 16-byte
// pieces of the code's user-minor row (lanes of consecutive codes land in distinct LDS
// banks). Every workgroup computes the same values (the same operations in the same
// order); with `store` it also writes them to the workspace for the selection kernels.
template <int UG, int LP, int ST>
__device__ void load_tables(const ScoreDev &a, int grp, float *tbl, bool store) {
    constexpr int CPW = UG * LP / 16 / kScanWaves;        // chunks per wave
    static_assert(CPW >= 1 && CPW * 16 * kScanWaves == UG * LP, "whole chunks per wave");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int L = a.L, V = a.V;
    float x[CPW][16][4];
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
        const int ch = wave + kScanWaves * k, d = ch % LP, ub = (ch / LP) * 16;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int uu = grp * UG + ub + r;
            const bool user = uu < a.U && d < L;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = lane + 64 * e;
                x[k][r][e] = (user && c < V) ? a.table_in[((size_t)uu * L + d) * V + c] : 0.0f;
            }
        }
    }
    if (a.kind == TCB_TABLE_LOGITS) {
        // each step runs over all 16 rows of a chunk, so that the rows' chains of cross-lane
        // reductions overlap; rows past the last user or depth go through the steps (their
        // values are all 0, so every step stays finite) and keep their zeros
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
            const int ch = wave + kScanWaves * k, d = ch % LP, ub = (ch / LP) * 16;
            float m[16], sum[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                m[r] = kNegInf;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (lane + 64 * e < V) m[r] = fmaxf(m[r], x[k][r][e]);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) m[r] = fmaxf(m[r], dpp_f<0xB1>(m[r]));
#pragma unroll
            for (int r = 0; r < 16; ++r) m[r] = fmaxf(m[r], dpp_f<0x4E>(m[r]));
#pragma unroll
            for (int r = 0; r < 16; ++r) m[r] = fmaxf(m[r], dpp_f<0x141>(m[r]));
#pragma unroll
            for (int r = 0; r < 16; ++r) m[r] = fmaxf(m[r], dpp_f<0x140>(m[r]));
#pragma unroll
            for (int r = 0; r < 16; ++r)
                m[r] = fmaxf(fmaxf(lane_f(m[r], 0), lane_f(m[r], 16)), fmaxf(lane_f(m[r], 32), lane_f(m[r], 48)));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sum[r] = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (lane + 64 * e < V) sum[r] += exp2_fast((x[k][r][e] - m[r]) * kLog2e);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[r] += dpp_f<0xB1>(sum[r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[r] += dpp_f<0x4E>(sum[r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[r] += dpp_f<0x141>(sum[r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[r] += dpp_f<0x140>(sum[r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float t = (lane_f(sum[r], 0) + lane_f(sum[r], 16)) + (lane_f(sum[r], 32) + lane_f(sum[r], 48));
                const bool live = grp * UG + ub + r < a.U && d < L;
                const float lse = live ? m[r] + __builtin_amdgcn_logf(t) * kLn2 : 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (lane + 64 * e < V) x[k][r][e] -= lse;
            }
        }
    }
    f32x4 *t4 = reinterpret_cast<f32x4 *>(tbl);
    f32x4 *g4 = reinterpret_cast<f32x4 *>(a.table + (size_t)grp * L * 256 * UG);
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
        const int ch = wave + kScanWaves * k, d = ch % LP, ub = (ch / LP) * 16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = d * 256 + lane + 64 * e;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = {x[k][4 * q][e], x[k][4 * q + 1][e], x[k][4 * q + 2][e], x[k][4 * q + 3][e]};
                t4[(c * ST + ub) / 4 + q] = v;
                if (store && d < L) g4[((size_t)c * UG + ub) / 4 + q] = v;
            }
        }
    }
    for (int i = threadIdx.x; i < ST; i += kScanThreads) tbl[LP * 256 * ST + i] = kPastEnd;
}

// ---------------------------------------------------------------------- scan
template <bool WIDE, int KS, bool LSE>
__global__ __launch_bounds__(kScanThreads) void k_score_scan(ScoreDev a) {
    constexpr int UG = WIDE ? kScoreUGWide : kScoreUGNarrow;
    constexpr int NH = UG / 16;                       // 16-user halves of the group
    constexpr int NR = 4 * NH;                        // (user, SID) values per lane and tile
    constexpr int KA = KS > 0 ? KS : 1;
    constexpr int TPB = kScoreBlock / kScoreGroup;    // tiles (groups) per block
    constexpr int PD = KS == 0 ? 8 : (KS <= 2 ? 4 : 2);   // tiles of loads in flight per wave
    static_assert(TPB % PD == 0, "whole rounds of the load pipeline per block");
    static_assert(TPB % 4 == 0, "a block's group maxima are stored 4 at a time");
    __shared__ f32x4 tbl4[kScoreTableFloats / 4];
    __shared__ float2 part[kScanWaves][32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, g = lane >> 4;
    constexpr int LP = WIDE ? 8 : 4;                  // levels, padded
    constexpr int ST = WIDE ? kScoreStrideWide : kScoreStrideNarrow;
    const int grp = blockIdx.y;
    const int n = (int)a.n, NB = (n + kScoreBlock - 1) / kScoreBlock;
    float *tbl = reinterpret_cast<float *>(tbl4);
    // the user vectors and the first tiles' loads do not depend on the tables: they are
    // issued first and arrive while the tables are built
    u32x4 av[NH][KA];
    if constexpr (KS > 0) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
            const int user = grp * UG + 16 * hh + j;
            load_rows<KS>(a.user_vec, user, user < a.U, g, av[hh], false);
        }
    }
    // this wave's tiles: its blocks first, first + stride, ... taken 16 tiles each, as one
    // sequence, so loads run PD tiles ahead across block ends; past the end they read the
    // last SID again (a valid address) and the results are masked
    const int first = (int)blockIdx.x * kScanWaves + wave, stride = (int)gridDim.x * kScanWaves;
    const int ntile = first < NB ? ((NB - 1 - first) / stride + 1) * TPB : 0;
    auto tile_first = [&](int q) { return (first + (q / TPB) * stride) * kScoreBlock + (q % TPB) * kScoreGroup; };
    CodeWord<WIDE> cw[PD];
    u32x4 bv[PD][KA];
    auto load_tile = [&](int q, int slot) {
        int leaf = tile_first(q) + j;
        leaf = leaf < n ? leaf : n - 1;
        cw[slot] = load_codes<WIDE>(a.codes, leaf);
        if constexpr (KS > 0) load_rows<KS>(a.emb, leaf, true, g, bv[slot], true);
    };
#pragma unroll
    for (int q = 0; q < PD - 1; ++q) load_tile(q, q);
    load_tables<UG, LP, ST>(a, grp, tbl, blockIdx.x == 0);
    // log-normaliser partials: per lane and register a reference rl (in log2 units) and
    // the sum ls of 2^(x log2 e - rl) over the scores x seen; the reference is the first
    // score, raised (and the sum rescaled) when a score exceeds it by more than 2^64
    float rl[NR], ls[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        rl[r] = kNegInf;
        ls[r] = 0.0f;
    }
    __syncthreads();
    const float w = a.w;
    float *gmax = a.gmax + (size_t)grp * NB * UG * (kScoreBlock / kScoreGroup);
    // after the transposed reduction lane j holds register ru of its row's users
    const int ru = reduced_reg<NR>(j);
    const int wr = 16 * (ru >> 2) + 4 * g + (ru & 3);        // ... i.e. this user row of the group
    const bool writer = j < NR;                                // these lanes hold distinct users
    float *bmax = a.bmax + ((size_t)grp * UG + wr) * NB;

    // one block (16 tiles) per round, unrolled, so that a lane keeps its user's 16 group
    // maxima in registers and stores them as 64 contiguous bytes at the block end
#pragma unroll 1
    for (int q0 = 0; q0 < ntile; q0 += TPB) {
        float gv[TPB];
#pragma unroll
        for (int q = 0; q < TPB; ++q) {
            load_tile(q0 + q + PD - 1, (q + PD - 1) % PD);
            const int f = tile_first(q0 + q);
            float s[NR];
            token_sums<NR, LP, ST>(tbl, cw[q % PD], f + j < n, g, s);
            if constexpr (KS > 0) {
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    const f32x4 acc = sim_tile<KS>(av[hh], bv[q % PD]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[4 * hh + e] = fmaf(w, acc[e], s[4 * hh + e]);
                }
            }
            if constexpr (LSE) {
                float t[NR], mx = kNegInf;
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    t[r] = fmaf(s[r], kLog2e, -rl[r]);
                    mx = fmaxf(mx, t[r]);
                }
                if (mx > 64.0f) {                                // first scores, or a rare jump
#pragma unroll
                    for (int r = 0; r < NR; ++r)
                        if (t[r] > 0.0f) {
                            ls[r] *= exp2_fast(-t[r]);
                            rl[r] = s[r] * kLog2e;
                            t[r] = 0.0f;
                        }
                }
#pragma unroll
                for (int r = 0; r < NR; ++r) ls[r] += exp2_fast(t[r]);
            }
            gv[q] = transposed_max<NR>(s, j);
        }
        // block end: [block][user][group in block] and the block's maximum per user
        const int blk = tile_first(q0) / kScoreBlock;
        float bmx = gv[0];
#pragma unroll
        for (int q = 1; q < TPB; ++q) bmx = fmaxf(bmx, gv[q]);
        if (writer) {
            f32x4 *dst = reinterpret_cast<f32x4 *>(gmax + ((size_t)blk * UG + wr) * TPB);
#pragma unroll
            for (int c = 0; c < TPB / 4; ++c) dst[c] = f32x4{gv[4 * c], gv[4 * c + 1], gv[4 * c + 2], gv[4 * c + 3]};
            bmax[blk] = bmx;
        }
    }

    if constexpr (LSE) {
        // the 16 lanes of a DPP row hold the same users: butterfly over them by DPP (xor 1,
        // xor 2, row_half_mirror, row_mirror), then the waves in order
        float lm[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            lm[r] = rl[r] * kLn2;                              // back to natural-log units
            lse_merge(lm[r], ls[r], dpp_f<0xB1>(lm[r]), dpp_f<0xB1>(ls[r]));
            lse_merge(lm[r], ls[r], dpp_f<0x4E>(lm[r]), dpp_f<0x4E>(ls[r]));
            lse_merge(lm[r], ls[r], dpp_f<0x141>(lm[r]), dpp_f<0x141>(ls[r]));
            lse_merge(lm[r], ls[r], dpp_f<0x140>(lm[r]), dpp_f<0x140>(ls[r]));
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
constexpr int KPT = kScoreCand / kSelectThreads;      // keys per thread in a selection: 8
static_assert(KPT * kSelectThreads == kScoreCand, "whole keys per thread");
static_assert(kScoreCand < 65536, "16-bit halves in the compaction's prefix sum");
constexpr int kDirectKeys = 16;   // block maxima per thread when the pick skips the superblocks
static_assert(kSelectThreads * kDirectKeys < 65536, "16-bit halves in the compaction's prefix sum");

struct SelSmem {
    uint32_t hist[3][256];                  // radix passes rotate through three histograms
    uint32_t wsum[2][kSelWaves];            // and prefix sums through two wave-total rows
    uint32_t mn[kSelWaves], mx[kSelWaves];
};

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {    // lanes with no source, or in masked rows: 0
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, true);
}

// inclusive prefix sum over the 64 lanes of a wave, in lane order, by DPP: shifts within
// each row of 16 lanes, then the last lane of row 0 and 2 added to rows 1 and 3, and the
// last lane of row 1 to rows 2 and 3
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
    x += dpp_u<0x111>(x);            // row_shr:1
    x += dpp_u<0x112>(x);            // row_shr:2
    x += dpp_u<0x114>(x);            // row_shr:4
    x += dpp_u<0x118>(x);            // row_shr:8
    x += dpp_u<0x142, 0xA>(x);       // row_bcast:15
    x += dpp_u<0x143, 0xC>(x);       // row_bcast:31
    return x;
}

__device__ __forceinline__ uint32_t lane_u(uint32_t v, int l) {   // l wave-uniform
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// the value lane (lane ^ J) holds: DPP inside rows of 16 lanes (J = 1, 2, 4, 8), a swizzle
// inside halves of 32 (J = 16), a permute (J = 32)
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    if constexpr (J == 1) {
        return dpp_u<0xB1>(v);                                  // quad_perm [1,0,3,2]
    } else if constexpr (J == 2) {
        return dpp_u<0x4E>(v);                                  // quad_perm [2,3,0,1]
    } else if constexpr (J == 4) {
        const uint32_t from_above = dpp_u<0x104>(v), from_below = dpp_u<0x114>(v);   // row_shl:4, row_shr:4
        return (threadIdx.x & 4) ? from_below : from_above;
    } else if constexpr (J == 8) {
        return dpp_u<0x128>(v);                                 // row_ror:8
    } else if constexpr (J == 16) {
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);   // bitmask mode, xor 16
    } else {
        static_assert(J == 32, "lane distance");
        return (uint32_t)__shfl_xor((int)v, 32, 64);
    }
}

// one compare-exchange step of a bitonic sorting network over the wave's 64 lanes: blocks
// of K lanes are ordered ascending where (lane & K) == 0, descending elsewhere; partners
// are J apart
template <int K, int J>
__device__ __forceinline__ void bitonic_step(uint64_t &x) {
    const uint32_t lo = xor_lane<J>((uint32_t)x), hi = xor_lane<J>((uint32_t)(x >> 32));
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    const int lane = threadIdx.x & 63;
    const bool keep_min = ((lane & J) == 0) == ((lane & K) == 0);
    x = keep_min ? (y < x ? y : x) : (y < x ? x : y);
}
template <int K, int J>
__device__ __forceinline__ void bitonic_merge(uint64_t &x) {
    bitonic_step<K, J>(x);
    if constexpr (J > 1) bitonic_merge<K, J / 2>(x);
}
template <int K>
__device__ __forceinline__ void bitonic_sort(uint64_t &x) {
    if constexpr (K > 2) bitonic_sort<K / 2>(x);
    bitonic_merge<K, K / 2>(x);
}
// the wave's 64 keys (one per lane), sorted ascending across the lanes
__device__ __forceinline__ uint64_t wave_sort(uint64_t x) {
    bitonic_sort<64>(x);
    return x;
}

// Exclusive prefix sum of one value per thread over the workgroup, in thread order;
// total in *total. One barrier: callers alternate `buf`, and consecutive uses of the same
// row are separated by another barrier.
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t v, SelSmem &S, int buf, uint32_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_sum(v);
    if (lane == 63) S.wsum[buf][wave] = incl;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const uint32_t c = S.wsum[buf][w];
        before += w < wave ? c : 0u;
        tot += c;
    }
    total = tot;
    return before + incl - v;
}

// Exact top-k of n <= 65535 keys held in registers (thread t holds positions NK t ... NK t +
// NK - 1; a larger key is better, equal keys: the lower position first; 1 <= k <= n):
// writes the chosen positions, ascending, to out[0 .. k). Radix selection of the k-th
// best key over d = key - (smallest key), 8 bits per pass from the highest bit in which
// the keys differ (so the first pass spreads them over the bins), then one ordered
// compaction (threads own consecutive positions, so two prefix sums place everything).
// One barrier per radix pass: every wave finds the digit itself from the shared
// histogram, and the histograms rotate so that clearing one never races with a read.
template <int NK>
__device__ void select_top(int k, int n, const uint32_t (&kv)[NK], uint32_t *out, SelSmem &S) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p0 = tid * NK;
    for (int i = tid; i < 256; i += kSelectThreads) S.hist[0][i] = 0u;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int e = 0; e < NK; ++e)
        if (p0 + e < n) {
            lo = min(lo, kv[e]);
            hi = max(hi, kv[e]);
        }
    // within each row of 16 lanes (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
    // row_mirror: every lane ends with its row's extremes), then over the four rows
    lo = min(lo, dpp_u<0xB1>(lo));
    hi = max(hi, dpp_u<0xB1>(hi));
    lo = min(lo, dpp_u<0x4E>(lo));
    hi = max(hi, dpp_u<0x4E>(hi));
    lo = min(lo, dpp_u<0x141>(lo));
    hi = max(hi, dpp_u<0x141>(hi));
    lo = min(lo, dpp_u<0x140>(lo));
    hi = max(hi, dpp_u<0x140>(hi));
    lo = min(min(lane_u(lo, 0), lane_u(lo, 16)), min(lane_u(lo, 32), lane_u(lo, 48)));
    hi = max(max(lane_u(hi, 0), lane_u(hi, 16)), max(lane_u(hi, 32), lane_u(hi, 48)));
    if (lane == 0) {
        S.mn[wave] = lo;
        S.mx[wave] = hi;
    }
    __syncthreads();
    lo = S.mn[0];
    hi = S.mx[0];
#pragma unroll
    for (int w = 1; w < kSelWaves; ++w) {
        lo = min(lo, S.mn[w]);
        hi = max(hi, S.mx[w]);
    }
    uint32_t pref = 0u, rem = (uint32_t)k;
    int remaining = hi > lo ? 32 - __clz((int)(hi - lo)) : 0;   // bits of d still undecided
    for (int pass = 0; remaining > 0; ++pass) {
        const int w = min(8, remaining), shift = remaining - w;
        uint32_t *H = S.hist[pass % 3];
        // the next pass's histogram was last read two passes ago, before the previous
        // pass's barrier; this pass's was cleared before it
        for (int i = tid; i < 256; i += kSelectThreads) S.hist[(pass + 1) % 3][i] = 0u;
#pragma unroll
        for (int e = 0; e < NK; ++e) {
            const uint32_t d = kv[e] - lo;
            if (p0 + e < n && (uint32_t)((uint64_t)d >> remaining) == pref)
                atomicAdd(&H[(d >> shift) & ((1u << w) - 1u)], 1u);
        }
        __syncthreads();
        // every wave: lane l owns digits 255 - 4l ... 252 - 4l, counts from the top digit down
        uint32_t c[4], sum = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            c[e] = H[255 - 4 * lane - e];
            sum += c[e];
        }
        const uint32_t incl = wave_incl_sum(sum);
        const uint32_t excl = incl - sum;
        uint32_t digit = 0u, above = 0u;
        if (excl < rem && incl >= rem) {
            uint32_t cum = excl;
            bool done = false;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (!done && cum + c[e] >= rem) {
                    digit = (uint32_t)(255 - 4 * lane - e);
                    above = cum;
                    done = true;
                }
                if (!done) cum += c[e];
            }
        }
        const uint64_t hit = __ballot(excl < rem && incl >= rem);
        const int src = hit ? (int)__builtin_ctzll(hit) : 0;       // exactly one lane holds the digit
        digit = lane_u(digit, src);
        above = lane_u(above, src);
        rem -= above;
        pref = (pref << w) | digit;
        remaining = shift;
    }
    const uint32_t T = lo + pref;     // the k-th best key; take all above it and the first rem equal
    // one prefix sum of (keys above T) | (keys equal to T) << 16 (n < 2^16 keeps the
    // halves apart): a taken key's place is the keys above T before it plus the taken
    // equal keys before it, min(equal keys before it, rem)
    uint32_t n_gt = 0u, n_eq = 0u;
#pragma unroll
    for (int e = 0; e < NK; ++e) {
        const bool valid = p0 + e < n;
        n_gt += (valid && kv[e] > T) ? 1u : 0u;
        n_eq += (valid && kv[e] == T) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t before = block_excl_sum(n_gt | (n_eq << 16), S, 0, tot);
    uint32_t gt_before = before & 0xFFFFu, eq_before = before >> 16;
#pragma unroll
    for (int e = 0; e < NK; ++e) {
        const bool valid = p0 + e < n;
        const bool gt = valid && kv[e] > T, eq = valid && kv[e] == T;
        if (gt || (eq && eq_before < rem)) {
            const uint32_t pos = gt_before + min(eq_before, rem);
            if (pos < (uint32_t)k) out[pos] = (uint32_t)(p0 + e);
        }
        gt_before += gt ? 1u : 0u;
        eq_before += eq ? 1u : 0u;
    }
    __syncthreads();
}

template <bool WIDE>
__global__ __launch_bounds__(kSelectThreads) void k_score_pick(ScoreDev a) {
    constexpr int UG = WIDE ? kScoreUGWide : kScoreUGNarrow;
    constexpr int MK = TCB_SCORE_MAX_K;
    constexpr int SUB = kScoreBlock / kScoreGroup;       // groups per block = blocks per superblock
    static_assert(SUB % KPT == 0, "a thread's keys stay inside one parent");
    __shared__ float sbm[kScoreCand];
    __shared__ uint32_t listA[MK], listB[MK];
    __shared__ SelSmem S;
    const int tid = threadIdx.x, lane = tid & 63;
    const int u = blockIdx.x, grp = u / UG, row = u % UG;
    const int n = (int)a.n, NG = (n + kScoreGroup - 1) / kScoreGroup, NB = (n + kScoreBlock - 1) / kScoreBlock;
    const int NS = (NB + SUB - 1) / SUB;
    const int K = a.K;
    const int p0 = tid * KPT;
    uint32_t kv[KPT];

    const float *bm = a.bmax + ((size_t)grp * UG + row) * NB;
    int kA;
    if (NB <= kSelectThreads * kDirectKeys) {
        // 1-2. few blocks: the best K of all block maxima at once (thread t holds blocks
        //      kDirectKeys t ...)
        uint32_t kb[kDirectKeys];
        const int b0 = tid * kDirectKeys;
        float x[kDirectKeys];
#pragma unroll
        for (int e = 0; e < kDirectKeys; ++e) x[e] = bm[b0 + e < NB ? b0 + e : NB - 1];
#pragma unroll
        for (int e = 0; e < kDirectKeys; ++e) kb[e] = f2ord(b0 + e < NB ? x[e] : kNegInf);
        kA = min(K, NB);
        select_top(kA, NB, kb, listB, S);
    } else {
        // 1. superblock maxima: coalesced reads of this user's block maxima, a maximum
        //    over each row of 16 lanes (16 consecutive blocks), then the best K superblocks
        for (int c = 0; c < NB; c += kSelectThreads * 16) {          // 16 loads in flight per thread
            float x[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int b = c + e * kSelectThreads + tid;
                x[e] = bm[b < NB ? b : NB - 1];
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int b = c + e * kSelectThreads + tid;
                const float m = row16_max(b < NB ? x[e] : kNegInf);
                if ((lane & 15) == 0 && b < NB) sbm[b / SUB] = m;
            }
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < KPT; ++e) kv[e] = f2ord(p0 + e < NS ? sbm[p0 + e] : kNegInf);
        const int kS = min(K, NS);
        select_top(kS, NS, kv, listA, S);

        // 2. the best K blocks inside them
        const int nA = SUB * kS;
        {
            float x[KPT];
            const int sb = (int)listA[min(p0 / SUB, kS - 1)];
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const int b = sb * SUB + (p0 + e) % SUB;
                x[e] = bm[b < NB ? b : NB - 1];
            }
#pragma unroll
            for (int e = 0; e < KPT; ++e) kv[e] = f2ord(sb * SUB + (p0 + e) % SUB < NB ? x[e] : kNegInf);
        }
        kA = min(K, nA);
        select_top(kA, nA, kv, listB, S);
        for (int q = tid; q < kA; q += kSelectThreads) {
            const uint32_t p = listB[q];
            listB[q] = listA[p / SUB] * (uint32_t)SUB + (p % SUB);
        }
        __syncthreads();
    }

    // 3. the best K groups inside those blocks: a block's 16 group maxima of one user are
    //    64 contiguous bytes
    const float *gm = a.gmax + (size_t)grp * NB * UG * SUB + (size_t)row * SUB;
    const int nB = SUB * kA;
    {
        const int blk = (int)listB[min(p0 / SUB, kA - 1)];          // may lie past the last block
        const f32x4 *src = reinterpret_cast<const f32x4 *>(gm + (size_t)min(blk, NB - 1) * UG * SUB + p0 % SUB);
        const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const float v = e < 4 ? x0[e] : x1[e - 4];
            kv[e] = f2ord(blk * SUB + (p0 + e) % SUB < NG && p0 + e < nB ? v : kNegInf);
        }
    }
    const int kB = min(K, nB);
    select_top(kB, nB, kv, listA, S);
    for (int q = tid; q < kB; q += kSelectThreads) {
        const uint32_t p = listA[q];
        a.pick[(size_t)u * MK + q] = (int32_t)(listB[p / SUB] * (uint32_t)SUB + (p % SUB));
    }
    if (tid == 0) a.npick[u] = kB;
}

// 4. rescore the SIDs of the picked groups of one user, spread over kRescoreWGs
//    workgroups per user: one 16-SID MFMA tile per group; only the 16-user half holding
//    this user is multiplied (its result does not depend on the other half), and the token
//    sums add the same table values in the same order as the scan, so every score equals
//    the scan's bit for bit.
template <bool WIDE, int KS>
__global__ __launch_bounds__(kRescoreThreads) void k_score_rescore(ScoreDev a) {
    constexpr int UG = WIDE ? kScoreUGWide : kScoreUGNarrow;
    constexpr int KA = KS > 0 ? KS : 1;
    constexpr int MK = TCB_SCORE_MAX_K;
    constexpr int LP = WIDE ? 8 : 4;
    constexpr int NWV = kRescoreThreads / 64;
    constexpr int RB = KS >= 8 ? 2 : (KS >= 4 ? 4 : 8);   // groups a wave rescores at once
    __shared__ float tcol[LP * 256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, g = lane >> 4;
    const int u = blockIdx.y, grp = u / UG, row = u % UG, L = a.L;
    const int n = (int)a.n;
    const int kB = a.npick[u];
    const int *pick = a.pick + (size_t)u * MK;
    float *cand = a.cand + (size_t)u * kScoreCand;
    const int hh_u = row >> 4, g_u = (row >> 2) & 3, e_u = row & 3;
    const int step = (int)gridDim.x * NWV;
    CodeWord<WIDE> cw[RB];
    u32x4 bv[RB][KA];
    uint32_t leafv[RB];
    // a round's loads need neither the table nor the count kB: entries of pick past kB
    // (left from earlier calls) give SIDs that are clamped into the catalog and dropped
    auto load_round = [&](int q0) {
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const int q = q0 + b * step;
            leafv[b] = (uint32_t)pick[q < MK ? q : MK - 1] * (uint32_t)kScoreGroup + (uint32_t)j;
            const int lc = leafv[b] < (uint32_t)n ? (int)leafv[b] : n - 1;
            cw[b] = load_codes<WIDE>(a.codes, lc);
            if constexpr (KS > 0) load_rows<KS>(a.emb, lc, true, g, bv[b], true);
        }
    };
    // the first round is issued before the table and the count arrive
    const int qs = (int)blockIdx.x * NWV + wave;
    load_round(qs);
    for (int i = tid; i < LP * 256; i += kRescoreThreads)
        tcol[i] = i < L * 256 ? a.table[((size_t)grp * L * 256 + i) * UG + row] : 0.0f;
    u32x4 av[KA];
    if constexpr (KS > 0) {
        const int user = grp * UG + 16 * hh_u + j;
        load_rows<KS>(a.user_vec, user, user < a.U, g, av, false);
    }
    __syncthreads();
    for (int q0 = qs; q0 < kB; q0 += step * RB) {
        if (q0 != qs) load_round(q0);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            float s = 0.0f;
#pragma unroll
            for (int d = 0; d < LP; ++d) s += tcol[d * 256 + (int)((cw[b] >> (8 * d)) & 255u)];
            if constexpr (KS > 0) {
                const f32x4 acc = sim_tile<KS>(av, bv[b]);
                // register e_u by two bit selects: a chain of equality tests is lowered to
                // branches, and a branch taken right after the MFMA was compiled without
                // the wait states its result needs (wrong values seen on gfx950)
                const float lo = (e_u & 1) ? acc[1] : acc[0], hi = (e_u & 1) ? acc[3] : acc[2];
                s = fmaf(a.w, (e_u & 2) ? hi : lo, s);
            }
            const int q = q0 + b * step;
            if (q < kB && g == g_u) cand[q * kScoreGroup + j] = leafv[b] < (uint32_t)n ? s : kNegInf;
        }
    }
}

// 5-6. the best K SIDs of one user, placed by rank under (score desc, SID asc), and the
// log-normaliser of the softmax over every valid SID.
template <bool WIDE>
__global__ __launch_bounds__(kSelectThreads) void k_score_final(ScoreDev a) {
    constexpr int UG = WIDE ? kScoreUGWide : kScoreUGNarrow;
    constexpr int MK = TCB_SCORE_MAX_K;
    __shared__ uint32_t listB[MK];
    __shared__ uint64_t sortk[MK];
    __shared__ SelSmem S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int u = blockIdx.x, grp = u / UG, row = u % UG;
    const int n = (int)a.n;
    const int K = a.K;
    const int p0 = tid * KPT;
    const int kB = a.npick[u];
    const int *pick = a.pick + (size_t)u * MK;
    const float *cand = a.cand + (size_t)u * kScoreCand;
    const int nC = kScoreGroup * kB;
    const int kC = min(K, n);
    uint32_t kv[KPT];
    {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(cand + p0);
        const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
        for (int e = 0; e < KPT; ++e) kv[e] = f2ord(p0 + e < nC ? (e < 4 ? x0[e] : x1[e - 4]) : kNegInf);
    }
    select_top(kC, nC, kv, listB, S);
    for (int i = tid; i < kC; i += kSelectThreads) {
        const uint32_t p = listB[i];
        const uint32_t leaf = (uint32_t)pick[p / kScoreGroup] * (uint32_t)kScoreGroup + (p % kScoreGroup);
        sortk[i] = ((uint64_t)(~f2ord(cand[p])) << 32) | leaf;   // ascending = (score desc, SID asc)
    }
    __syncthreads();
    // place each of the kC keys (distinct: they hold the SID) by its rank: waves 0 .. 7
    // sort 64 keys each in registers, and a key's rank is the number of keys below it in
    // every wave's sorted list (a binary search in LDS per list; in its own list that is
    // its lane)
    {
        const int nlist = (kC + 63) / 64;
        uint64_t me = ~0ull;                          // no real key: the SID is below 2^25
        int32_t item = -1;
        if (wave < nlist) {
            const int i = wave * 64 + lane;
            me = wave_sort(i < kC ? sortk[i] : ~0ull);
            sortk[i] = me;                            // a wave rewrites only the keys it read
            const int32_t leaf = (int32_t)(uint32_t)me;
            if (me != ~0ull && a.out_item && leaf < n) item = a.leaf_item[leaf];   // arrives during the search
        }
        __syncthreads();
        if (wave < nlist) {
            constexpr int NL = MK / 64;
            int pos[NL];
#pragma unroll
            for (int l = 0; l < NL; ++l) pos[l] = 0;
#pragma unroll
            for (int st = 32; st > 0; st >>= 1)
#pragma unroll
                for (int l = 0; l < NL; ++l)
                    if (l < nlist && sortk[l * 64 + pos[l] + st - 1] < me) pos[l] += st;
            uint32_t rank = 0u;
#pragma unroll
            for (int l = 0; l < NL; ++l)
                if (l < nlist) rank += (uint32_t)pos[l] + (sortk[l * 64 + pos[l]] < me ? 1u : 0u);
            if (me != ~0ull) {
                const int32_t leaf = (int32_t)(uint32_t)me;
                a.out_leaf[(size_t)u * K + rank] = leaf;
                a.out_score[(size_t)u * K + rank] = ord2f(~(uint32_t)(me >> 32));
                if (a.out_item) a.out_item[(size_t)u * K + rank] = item;
            }
        }
    }
    for (int i = kC + tid; i < K; i += kSelectThreads) {
        a.out_leaf[(size_t)u * K + i] = -1;
        a.out_score[(size_t)u * K + i] = kNegInf;
        if (a.out_item) a.out_item[(size_t)u * K + i] = -1;
    }
    if (a.out_lse && wave == 0) {
        const float *pp = a.lse_part + ((size_t)grp * kScanWGs * UG + row) * 2;
        static_assert(kScanWGs % 64 == 0, "whole partials per lane");
        float pm[kScanWGs / 64], ps[kScanWGs / 64];
#pragma unroll
        for (int i = 0; i < kScanWGs / 64; ++i) {                 // all loads first, then the merges
            pm[i] = pp[(size_t)(lane + 64 * i) * UG * 2];
            ps[i] = pp[(size_t)(lane + 64 * i) * UG * 2 + 1];
        }
        float m = kNegInf, s = 0.0f;
#pragma unroll
        for (int i = 0; i < kScanWGs / 64; ++i) lse_merge(m, s, pm[i], ps[i]);
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
    if (ev) (void)hipEventRecord(ev[0], s);
    if (a.out_lse)
        hipLaunchKernelGGL((k_score_scan<WIDE, KS, true>), scan_grid, dim3(kScanThreads), 0, s, a);
    else
        hipLaunchKernelGGL((k_score_scan<WIDE, KS, false>), scan_grid, dim3(kScanThreads), 0, s, a);
    if (ev) (void)hipEventRecord(ev[1], s);
    hipLaunchKernelGGL((k_score_pick<WIDE>), dim3(a.U), dim3(kSelectThreads), 0, s, a);
    hipLaunchKernelGGL((k_score_rescore<WIDE, KS>), dim3(kRescoreWGs, a.U), dim3(kRescoreThreads), 0, s, a);
    hipLaunchKernelGGL((k_score_final<WIDE>), dim3(a.U), dim3(kSelectThreads), 0, s, a);
    if (ev) (void)hipEventRecord(ev[2], s);
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
    o.bmax = al(o.gmax + groups * NB * UG * (kScoreBlock / kScoreGroup) * 4);
    o.lse = al(o.bmax + groups * NB * UG * 4);
    o.pick = al(o.lse + groups * kScanWGs * UG * 8);
    o.npick = al(o.pick + (size_t)max_users * TCB_SCORE_MAX_K * 4);
    o.cand = al(o.npick + (size_t)max_users * 4);
    o.total = al(o.cand + (size_t)max_users * kScoreCand * 4);
    (void)NG;
    return o;
}

hipError_t launch_score(const ScoreDev &a, hipStream_t s, const hipEvent_t *ev) {
    return a.L > 4 ? launch_w<true>(a, s, ev) : launch_w<false>(a, s, ev);
}

// The scratch of tcb_score_catalog_static, for callers that cannot allocate: one array per
// GPU the library runs on, held until the process ends. Host code uses only the address
// hipGetSymbolAddress gives for the current device, never the array's name.
static __device__ __align__(256) uint8_t scratch[kStaticScoreScratch];

hipError_t static_score_scratch(void **ptr, size_t *bytes) {
    static std::mutex mu;
    static void *dev_ptr[kMaxScratchDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (dev_ptr[dev] == nullptr) {                    // once per device, with it current
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        dev_ptr[dev] = p;
    }
    *ptr = dev_ptr[dev];
    *bytes = kStaticScoreScratch;
    return hipSuccess;
}

}  // namespace tcb
