// gfx950 kernels of the catalog-constrained wide-beam step.
//
// The step (flashrec 0.1.0, Features > Decoding, "SID constraint"; OneLA summary,
// sections 2.1 and 3.3; SPRINT summary, inference paragraph):
//   for every live row r of a request, with trie node p_r and children K_r,
//     logp_{r,c} = x_{r,c} - (m_r + ln sum_{c' in K_r} exp(x_{r,c'} - m_r)),  c in K_r
//     candidate (r, c) scores s_r + logp_{r,c}
//   the request keeps its best n (beam width) candidates by (score desc, r*256+c asc),
//   in rank order; survivor j records parent r, code c and the child node.
//
// Two kernels per step:
//   expand  one workgroup per tile of kTileRows rows of one request. Each wave64 owns
//           whole rows: lane l holds codes 4l..4l+3, so a row is one coalesced 1 KiB
//           (fp32) or 512 B (bf16) load. The row's child set is a 256-bit mask, read
//           from the dense per-node mask at shallow depths or built in wave-private LDS
//           from the CSR child list deeper down; both give bit-identical results.
//           The masked log-softmax is two wave reductions. The tile then keeps its own
//           best n candidates (exact, by histogram refinement) and records the n-th
//           score, so the merge can discard what no tile-local top-n contains.
//   merge   one workgroup per request: prunes against the largest tile threshold,
//           stages the rest in LDS, finds the exact n-th candidate, orders the
//           survivors by bucketing plus exact in-bucket ranking, and writes the new
//           rows (parent-gather / trie-advance) plus the per-level back-pointers.
// All selection keys are unique (flat index breaks ties) and all float reductions
// have a fixed order, so results are deterministic run to run.
#include "tcb_internal.h"

namespace tcb {
namespace {

// ---------------------------------------------------------------------- helpers
__device__ __forceinline__ uint32_t f2ord(float f) {   // order-preserving, -0 == +0
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord2f(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

// LDS ordering among the lanes of one wave (no workgroup barrier needed)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *part, int *total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) part[w] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        const int p = part[i];
        before += (i < w) ? p : 0;
        tot += p;
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

// ---------------------------------------------------------------------- selection
// Exact k-th best of a set of (order key o, flat f) pairs spread over the threads of a
// workgroup, best = larger o, then smaller f. The active range [lo, hi] of keys is
// narrowed by 1024-bin histograms of the key distance to hi (binned by a shift, so the
// range's extremes always land in different bins and every round makes progress);
// once one key value remains, the same is done on the flat index.
struct SelSmem {
    uint32_t hist[kSelBins];
    int part[16];
    uint32_t lo, hi;
    uint32_t bstar, need;
};

__device__ __forceinline__ int range_shift(uint32_t range) {
    const int bits = 32 - __clz((int)range);          // range >= 1
    return bits > 10 ? bits - 10 : 0;
}

template <int NT>
__device__ __forceinline__ void find_bstar(SelSmem &S, uint32_t need) {
    constexpr int BPT = kSelBins / NT;
    uint32_t loc[BPT];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        loc[i] = S.hist[threadIdx.x * BPT + i];
        sum += (int)loc[i];
    }
    int total;
    const int before = block_excl_scan<NT>(sum, S.part, &total);
    if ((uint32_t)before < need && need <= (uint32_t)(before + sum)) {
        uint32_t c = (uint32_t)before;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            if (c < need && c + loc[i] >= need) {
                S.bstar = threadIdx.x * BPT + i;
                S.need = need - c;
            }
            c += loc[i];
        }
    }
    __syncthreads();
}

// `each(fn)` calls fn(o, f) for every element held by the calling thread. Every
// thread of the workgroup must call this function. Requires 1 <= k <= n.
template <int NT, class Each>
__device__ void block_select(Each each, uint32_t k, SelSmem &S, uint32_t &o_star, uint32_t &f_star,
                             uint32_t *err) {
    const int t = threadIdx.x;
    for (int i = t; i < kSelBins; i += NT) S.hist[i] = 0;
    if (t == 0) {
        S.lo = 0xffffffffu;
        S.hi = 0u;
    }
    __syncthreads();
    {
        uint32_t a = 0xffffffffu, b = 0u;
        each([&](uint32_t o, uint32_t) {
            a = min(a, o);
            b = max(b, o);
        });
        a = wave_min_u(a);
        b = wave_max_u(b);
        if ((t & 63) == 0) {
            atomicMin(&S.lo, a);
            atomicMax(&S.hi, b);
        }
    }
    __syncthreads();
    uint32_t lo = S.lo, hi = S.hi, need = k;
    // phase 1: the key value of the k-th element. Each round keeps one bin, whose key
    // range has at least 10 fewer bits, so 4 rounds always suffice; the cap only turns
    // a logic error into a flagged error instead of a hang.
    for (int round = 0; lo != hi; ++round) {
        if (round >= 8) {
            if (t == 0) atomicOr(err, kErrInternal);
            break;
        }
        const int sh = range_shift(hi - lo);
        each([&](uint32_t o, uint32_t) {
            if (o >= lo && o <= hi) atomicAdd(&S.hist[(hi - o) >> sh], 1u);
        });
        __syncthreads();
        find_bstar<NT>(S, need);
        const uint32_t bs = S.bstar, nn = S.need;
        for (int i = t; i < kSelBins; i += NT) S.hist[i] = 0;
        if (t == 0) {
            S.lo = 0xffffffffu;
            S.hi = 0u;
        }
        __syncthreads();
        uint32_t a = 0xffffffffu, b = 0u;
        each([&](uint32_t o, uint32_t) {
            if (o >= lo && o <= hi && ((hi - o) >> sh) == bs) {
                a = min(a, o);
                b = max(b, o);
            }
        });
        a = wave_min_u(a);
        b = wave_max_u(b);
        if ((t & 63) == 0) {
            atomicMin(&S.lo, a);
            atomicMax(&S.hi, b);
        }
        __syncthreads();
        lo = S.lo;
        hi = S.hi;
        need = nn;
        __syncthreads();
    }
    // phase 2: among elements with key lo, the need-th smallest flat index
    if (t == 0) {
        S.lo = 0xffffffffu;
        S.hi = 0u;
    }
    __syncthreads();
    {
        uint32_t a = 0xffffffffu, b = 0u;
        each([&](uint32_t o, uint32_t f) {
            if (o == lo) {
                a = min(a, f);
                b = max(b, f);
            }
        });
        a = wave_min_u(a);
        b = wave_max_u(b);
        if ((t & 63) == 0) {
            atomicMin(&S.lo, a);
            atomicMax(&S.hi, b);
        }
    }
    __syncthreads();
    uint32_t flo = S.lo, fhi = S.hi;
    __syncthreads();
    for (int round = 0; flo != fhi; ++round) {
        if (round >= 8) {
            if (t == 0) atomicOr(err, kErrInternal);
            break;
        }
        const int sh = range_shift(fhi - flo);
        each([&](uint32_t o, uint32_t f) {
            if (o == lo && f >= flo && f <= fhi) atomicAdd(&S.hist[(f - flo) >> sh], 1u);
        });
        __syncthreads();
        find_bstar<NT>(S, need);
        const uint32_t bs = S.bstar, nn = S.need;
        for (int i = t; i < kSelBins; i += NT) S.hist[i] = 0;
        if (t == 0) {
            S.lo = 0xffffffffu;
            S.hi = 0u;
        }
        __syncthreads();
        uint32_t a = 0xffffffffu, b = 0u;
        each([&](uint32_t o, uint32_t f) {
            if (o == lo && f >= flo && f <= fhi && ((f - flo) >> sh) == bs) {
                a = min(a, f);
                b = max(b, f);
            }
        });
        a = wave_min_u(a);
        b = wave_max_u(b);
        if ((t & 63) == 0) {
            atomicMin(&S.lo, a);
            atomicMax(&S.hi, b);
        }
        __syncthreads();
        flo = S.lo;
        fhi = S.hi;
        need = nn;
        __syncthreads();
    }
    o_star = lo;
    f_star = flo;
}

__device__ __forceinline__ bool key_le(uint32_t o, uint32_t f, uint32_t o_star, uint32_t f_star) {
    return o > o_star || (o == o_star && f <= f_star);
}

// ---------------------------------------------------------------------- candidates
struct alignas(16) Cand {
    float score;
    uint32_t flat;       // r * 256 + c, r = parent's rank in the request
    int32_t node;        // child node id
    uint32_t pad;
};

// ---------------------------------------------------------------------- row logits
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int DT, bool VEC>
__device__ __forceinline__ void load_row(const void *logits, int64_t ld, int slot, int lane, int V,
                                         float x[4]) {
    if constexpr (VEC) {
        if constexpr (DT == TCB_F32) {
            const f32x4 *p = reinterpret_cast<const f32x4 *>(
                static_cast<const float *>(logits) + (size_t)slot * (size_t)ld);
            const f32x4 v = __builtin_nontemporal_load(p + lane);
            x[0] = v[0];
            x[1] = v[1];
            x[2] = v[2];
            x[3] = v[3];
        } else {
            const u32x2 *p = reinterpret_cast<const u32x2 *>(
                static_cast<const uint16_t *>(logits) + (size_t)slot * (size_t)ld);
            const u32x2 v = __builtin_nontemporal_load(p + lane);
            x[0] = __uint_as_float(v[0] << 16);
            x[1] = __uint_as_float(v[0] & 0xffff0000u);
            x[2] = __uint_as_float(v[1] << 16);
            x[3] = __uint_as_float(v[1] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 4 * lane + q;
            float v = 0.0f;
            if (c < V) {
                if constexpr (DT == TCB_F32)
                    v = static_cast<const float *>(logits)[(size_t)slot * (size_t)ld + c];
                else
                    v = __uint_as_float((uint32_t) static_cast<const uint16_t *>(
                                            logits)[(size_t)slot * (size_t)ld + c] << 16);
            }
            x[q] = v;
        }
    }
}

// Child set of node n as a 256-bit mask (8 wave-uniform words) plus the first child id.
// Returns false if n is not a node of depth `level` (corrupt state).
__device__ __forceinline__ bool row_children(const TrieDev &T, uint32_t n, int level, int lane,
                                             uint32_t *wmask, uint32_t m[8], uint32_t &cb) {
    if (n < T.off[level] || n >= T.off[level + 1]) return false;
    cb = T.child_begin[n];
    if (level < T.mask_depths) {
#pragma unroll
        for (int w = 0; w < 8; ++w) m[w] = T.mask[(size_t)n * 8 + w];
    } else {
        const uint32_t ce = T.child_begin[n + 1];
        if (lane < 8) wmask[lane] = 0u;
        wave_lds_sync();
        for (uint32_t p = cb + lane; p < ce; p += 64) {
            const uint32_t c = T.child_code[p];
            atomicOr(&wmask[c >> 5], 1u << (c & 31));
        }
        wave_lds_sync();
#pragma unroll
        for (int w = 0; w < 8; ++w) m[w] = __builtin_amdgcn_readfirstlane(wmask[w]);
        wave_lds_sync();
    }
    return true;
}

// ---------------------------------------------------------------------- expand
// Per-thread candidate store: kRowsPerWave rows x 4 codes.
constexpr int kE = kRowsPerWave * 4;

template <int DT, int NORM, bool VEC>
__global__ __launch_bounds__(kExpandThreads) void k_expand(TrieDev T, WaveDev W, int par,
                                                           const void *__restrict__ logits, int64_t ld) {
    __shared__ uint32_t s_wmask[kTileWaves][8];
    __shared__ SelSmem S;

    const int req = blockIdx.x / W.MT;
    const int lt = blockIdx.x - req * W.MT;
    const ReqRec rec = W.rec[req];
    if (rec.status != kReqActive || rec.level >= T.L) return;
    const int r0 = lt * kTileRows;
    if (r0 >= rec.rows) return;
    const int level = rec.level;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int V = T.V;

    // issue every row's state and logits loads first
    int rr[kRowsPerWave];
    int32_t nd[kRowsPerWave];
    float sr[kRowsPerWave];
    float x[kRowsPerWave][4];
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
        rr[j] = r0 + j * kTileWaves + wave;
        nd[j] = -1;
        sr[j] = 0.0f;
        x[j][0] = x[j][1] = x[j][2] = x[j][3] = 0.0f;
        if (rr[j] < rec.rows) {
            const int slot = rec.base + rr[j];
            nd[j] = W.node[par][slot];
            sr[j] = W.score[par][slot];
            load_row<DT, VEC>(logits, ld, slot, lane, V, x[j]);
        }
    }

    uint32_t co[kE];     // order keys of this lane's candidates
    int32_t cn[kE];      // child node ids
    uint32_t valid = 0u;
    bool bad_value = false;
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
        if (rr[j] >= rec.rows) continue;                       // wave-uniform
        const uint32_t n = (uint32_t)__builtin_amdgcn_readfirstlane(nd[j]);
        uint32_t m[8], cb = 0;
        if (!row_children(T, n, level, lane, s_wmask[wave], m, cb)) {
            if (lane == 0) atomicOr(W.err, kErrBadNode);
            continue;
        }
        // this lane's 4 codes: word lane>>3, bits (lane&7)*4 .. +3
        const int wl = lane >> 3, sh = (lane & 7) * 4;
        uint32_t below = 0u, word = 0u;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            below += (w < wl) ? (uint32_t)__popc(m[w]) : 0u;
            word = (w == wl) ? m[w] : word;
        }
        const uint32_t bits4 = (word >> sh) & 0xFu;
        const uint32_t rank0 = below + (uint32_t)__popc(word & ((1u << sh) - 1u));

        if (W.validate) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (4 * lane + q < V && !isfinite(x[j][q])) bad_value = true;
        }
        // masked log-softmax: max and sum over the support, fixed reduction order
        float mx = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool in = (NORM == TCB_NORM_CHILDREN) ? ((bits4 >> q) & 1u) : (4 * lane + q < V);
            if (in) mx = fmaxf(mx, x[j][q]);
        }
        mx = wave_max_f(mx);
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool in = (NORM == TCB_NORM_CHILDREN) ? ((bits4 >> q) & 1u) : (4 * lane + q < V);
            if (in) sum += expf(x[j][q] - mx);
        }
        sum = wave_sum_f(sum);
        const float lse = mx + logf(sum);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = j * 4 + q;
            const float cand = sr[j] + (x[j][q] - lse);
            co[e] = f2ord(cand);
            cn[e] = (int32_t)(cb + rank0 + (uint32_t)__popc(bits4 & ((1u << q) - 1u)));
            valid |= ((bits4 >> q) & 1u) << e;
        }
    }
    if (bad_value) atomicOr(W.err, kErrNonFinite);

    auto flat_of = [&](int e) -> uint32_t {
        return (uint32_t)rr[e >> 2] * 256u + (uint32_t)(4 * lane + (e & 3));
    };
    auto each = [&](auto fn) {
#pragma unroll
        for (int e = 0; e < kE; ++e)
            if ((valid >> e) & 1u) fn(co[e], flat_of(e));
    };

    int total;
    block_excl_scan<kExpandThreads>(__popc(valid), S.part, &total);
    const uint32_t width = (uint32_t)rec.width;
    uint32_t thr = 0u;
    if ((uint32_t)total > width) {
        uint32_t o_star, f_star;
        block_select<kExpandThreads>(each, width, S, o_star, f_star, W.err);
#pragma unroll
        for (int e = 0; e < kE; ++e)
            if (!key_le(co[e], flat_of(e), o_star, f_star)) valid &= ~(1u << e);
        thr = o_star;
    }
    const int mine = __popc(valid);
    const int off = block_excl_scan<kExpandThreads>(mine, S.part, &total);
    Cand *out = reinterpret_cast<Cand *>(W.cand) + ((size_t)req * W.MT + lt) * W.CAPT;
    int i = off;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        if ((valid >> e) & 1u) {
            Cand c;
            c.score = ord2f(co[e]);
            c.flat = flat_of(e);
            c.node = cn[e];
            c.pad = 0u;
            out[i++] = c;
        }
    }
    if (threadIdx.x == 0) {
        W.tile_count[req * W.MT + lt] = total;
        W.tile_thr[req * W.MT + lt] = thr;
    }
}

// ---------------------------------------------------------------------- merge
struct MergeSmem {
    float s[kMergeCap];
    uint32_t f[kMergeCap];
    int32_t node[kMergeCap];
    uint32_t order[TCB_MAX_WIDTH];
    uint32_t bin_cnt[kSortBins];
    uint32_t bin_start[kSortBins];
    uint32_t bin_cur[kSortBins];
    int32_t tcnt[kMaxTilesPerReq];
    SelSmem sel;
    uint32_t thr, n, n_all, omax;
};

__global__ __launch_bounds__(kMergeThreads) void k_merge(TrieDev T, WaveDev W, int par) {
    __shared__ MergeSmem M;
    constexpr int NT = kMergeThreads;
    const int req = blockIdx.x;
    const int t = threadIdx.x;
    const ReqRec rec = W.rec[req];
    if (rec.status != kReqActive) return;
    const int nxt = par ^ 1;
    if (rec.level >= T.L) {   // finished, awaiting finalize: carry its rows over
        for (int r = t; r < rec.rows; r += NT) {
            W.node[nxt][rec.base + r] = W.node[par][rec.base + r];
            W.score[nxt][rec.base + r] = W.score[par][rec.base + r];
        }
        return;
    }
    const int ntile = (rec.rows + kTileRows - 1) / kTileRows;
    if (t == 0) {
        M.thr = 0u;
        M.n = 0u;
        M.n_all = 0u;
        M.omax = 0u;
    }
    for (int i = t; i < kSortBins; i += NT) {
        M.bin_cnt[i] = 0u;
        M.bin_cur[i] = 0u;
    }
    __syncthreads();
    for (int i = t; i < ntile; i += NT) {
        const int c = W.tile_count[req * W.MT + i];
        M.tcnt[i] = c;
        atomicAdd(&M.n_all, (uint32_t)c);
        atomicMax(&M.thr, W.tile_thr[req * W.MT + i]);
    }
    __syncthreads();
    const uint32_t thr = M.thr;
    const uint32_t n_all = M.n_all;
    const uint32_t k = min((uint32_t)rec.width, n_all);
    const Cand *cand = reinterpret_cast<const Cand *>(W.cand) + (size_t)req * W.MT * W.CAPT;
    const int CAPT = W.CAPT;

    // stage candidates at or above the largest tile threshold (wave-aggregated append)
    constexpr int U = 8;
    for (int tb = 0; tb < ntile; tb += U) {
        for (int i0 = 0; i0 < CAPT; i0 += NT) {
            Cand c[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int tile = tb + u;
                const int i = i0 + t;
                ok[u] = tile < ntile && i < M.tcnt[tile < ntile ? tile : 0];
                if (ok[u]) c[u] = cand[(size_t)tile * CAPT + i];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool pass = ok[u] && f2ord(c[u].score) >= thr;
                const uint64_t bal = __ballot(pass);
                uint32_t wbase = 0;
                if ((t & 63) == 0 && bal) wbase = atomicAdd(&M.n, (uint32_t)__popcll(bal));
                wbase = __shfl(wbase, 0, 64);
                if (pass) {
                    const uint32_t p = wbase + (uint32_t)__popcll(bal & ((1ull << (t & 63)) - 1ull));
                    if (p < (uint32_t)kMergeCap) {
                        M.s[p] = c[u].score;
                        M.f[p] = c[u].flat;
                        M.node[p] = c[u].node;
                    }
                }
            }
        }
    }
    __syncthreads();
    uint32_t n = M.n;
    uint32_t o_star = 0u, f_star = 0xffffffffu;       // default: keep everything staged
    const bool did_select = n > k;
    if (n > (uint32_t)kMergeCap) {
        // too many survivors of the pruning for LDS: select straight from global memory,
        // then stage exactly the k selected candidates
        if (t == 0) atomicOr(W.err, kInfoMergeSpill);
        auto each_g = [&](auto fn) {
            for (int tile = 0; tile < ntile; ++tile)
                for (int i = t; i < M.tcnt[tile]; i += NT) {
                    const Cand c = cand[(size_t)tile * CAPT + i];
                    const uint32_t o = f2ord(c.score);
                    if (o >= thr) fn(o, c.flat);
                }
        };
        block_select<NT>(each_g, k, M.sel, o_star, f_star, W.err);
        if (t == 0) M.n = 0u;
        __syncthreads();
        for (int tile = 0; tile < ntile; ++tile)
            for (int i0 = 0; i0 < M.tcnt[tile]; i0 += NT) {
                const int i = i0 + t;
                bool pass = false;
                Cand c{};
                if (i < M.tcnt[tile]) {
                    c = cand[(size_t)tile * CAPT + i];
                    const uint32_t o = f2ord(c.score);
                    pass = o >= thr && key_le(o, c.flat, o_star, f_star);
                }
                const uint64_t bal = __ballot(pass);
                uint32_t wbase = 0;
                if ((t & 63) == 0 && bal) wbase = atomicAdd(&M.n, (uint32_t)__popcll(bal));
                wbase = __shfl(wbase, 0, 64);
                if (pass) {
                    const uint32_t p = wbase + (uint32_t)__popcll(bal & ((1ull << (t & 63)) - 1ull));
                    M.s[p] = c.score;
                    M.f[p] = c.flat;
                    M.node[p] = c.node;
                }
            }
        __syncthreads();
        n = M.n;
    } else if (n > k) {
        auto each_l = [&](auto fn) {
            for (uint32_t e = t; e < n; e += NT) fn(f2ord(M.s[e]), M.f[e]);
        };
        block_select<NT>(each_l, k, M.sel, o_star, f_star, W.err);
    }
    if (t == 0 && n < k) atomicOr(W.err, kErrInternal);

    // order the k selected: buckets by key distance to the best, then exact in-bucket rank
    {
        uint32_t b = 0u;
        for (uint32_t e = t; e < n; e += NT) {
            const uint32_t o = f2ord(M.s[e]);
            if (key_le(o, M.f[e], o_star, f_star)) b = max(b, o);
        }
        b = wave_max_u(b);
        if ((t & 63) == 0) atomicMax(&M.omax, b);
    }
    __syncthreads();
    const uint32_t omax = M.omax;
    // smallest selected key: the k-th key after a selection, else the minimum staged key
    uint32_t olo = o_star;
    if (!did_select) {
        if (t == 0) M.sel.lo = 0xffffffffu;
        __syncthreads();
        uint32_t a = 0xffffffffu;
        for (uint32_t e = t; e < n; e += NT) a = min(a, f2ord(M.s[e]));
        a = wave_min_u(a);
        if ((t & 63) == 0) atomicMin(&M.sel.lo, a);
        __syncthreads();
        olo = M.sel.lo;
    }
    const int bsh = (omax > olo) ? range_shift(omax - olo) : 0;
    for (uint32_t e = t; e < n; e += NT) {
        const uint32_t o = f2ord(M.s[e]);
        if (key_le(o, M.f[e], o_star, f_star)) atomicAdd(&M.bin_cnt[(omax - o) >> bsh], 1u);
    }
    __syncthreads();
    {
        constexpr int BPT = kSortBins / NT;
        uint32_t loc[BPT];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            loc[i] = M.bin_cnt[t * BPT + i];
            sum += (int)loc[i];
        }
        int total;
        int before = block_excl_scan<NT>(sum, M.sel.part, &total);
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            M.bin_start[t * BPT + i] = (uint32_t)before;
            before += (int)loc[i];
        }
    }
    __syncthreads();
    for (uint32_t e = t; e < n; e += NT) {
        const uint32_t o = f2ord(M.s[e]);
        if (key_le(o, M.f[e], o_star, f_star)) {
            const uint32_t bin = (omax - o) >> bsh;
            const uint32_t p = M.bin_start[bin] + atomicAdd(&M.bin_cur[bin], 1u);
            M.order[p] = e;
        }
    }
    __syncthreads();
    const int S = W.S;
    const int level = rec.level;
    const uint32_t kk = min(k, n);        // equal unless the invariant above failed
    for (uint32_t p = t; p < kk; p += NT) {
        const uint32_t e = M.order[p];
        if (e >= n) continue;
        const uint32_t o = f2ord(M.s[e]), f = M.f[e];
        const uint32_t bin = (omax - o) >> bsh;
        const uint32_t st = M.bin_start[bin], en = st + M.bin_cnt[bin];
        uint32_t rank = st;
        for (uint32_t q = st; q < en; ++q) {
            const uint32_t e2 = M.order[q];
            const uint32_t o2 = f2ord(M.s[e2]), f2 = M.f[e2];
            rank += (o2 > o || (o2 == o && f2 < f)) ? 1u : 0u;
        }
        const int slot = rec.base + (int)rank;
        W.node[nxt][slot] = M.node[e];
        W.score[nxt][slot] = M.s[e];
        W.parent_slot[slot] = rec.base + (int)(f >> 8);
        W.hist[(size_t)level * S + slot] = f;             // (r << 8) | c
    }
    if (t == 0) {
        W.rec[req].rows = (int32_t)kk;
        W.rec[req].level = level + 1;
    }
}

// ---------------------------------------------------------------------- small kernels
__global__ void k_clear_wave(WaveDev W) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < W.R) {
        ReqRec r{};
        W.rec[i] = r;
    }
    if (i < W.R * W.MT) {
        W.tile_count[i] = 0;
        W.tile_thr[i] = 0u;
    }
    if (i == 0) *W.err = 0u;
}

__global__ void k_init(WaveDev W, int par, InitBatch b) {
    const int i = threadIdx.x;
    if (i >= b.n) return;
    ReqRec r{};
    r.base = b.base[i];
    r.width = b.width[i];
    r.rows = 1;
    r.level = 0;
    r.status = kReqActive;
    W.rec[b.req[i]] = r;
    W.node[par][b.base[i]] = 0;        // the root
    W.score[par][b.base[i]] = 0.0f;
}

__global__ void k_finalize(TrieDev T, WaveDev W, int par, FinBatch fb, uint8_t *sids, float *scores,
                           int64_t *items, int32_t *counts) {
    const int i = blockIdx.x;
    if (i >= fb.n) return;
    const int req = fb.req[i];
    const size_t orow = (size_t)fb.out_row[i];
    const ReqRec rec = W.rec[req];
    const int L = T.L;
    const uint32_t leaf0 = T.off[L], leaf1 = T.off[L + 1];
    for (int j = threadIdx.x; j < W.Bmax; j += blockDim.x) {
        const size_t out = orow * (size_t)W.Bmax + (size_t)j;
        if (j < rec.rows) {
            const int slot = rec.base + j;
            const uint32_t node = (uint32_t)W.node[par][slot];
            int64_t item = -1;
            if (node >= leaf0 && node < leaf1) item = T.leaf_item[node - leaf0];
            else atomicOr(W.err, kErrBadNode);
            uint32_t r = (uint32_t)j;
            for (int lv = L - 1; lv >= 0; --lv) {
                if (r >= (uint32_t)rec.width) {      // corrupt back-pointer: never read past the request
                    atomicOr(W.err, kErrBadNode);
                    break;
                }
                const uint32_t h = W.hist[(size_t)lv * W.S + rec.base + r];
                sids[out * L + lv] = (uint8_t)(h & 255u);
                r = h >> 8;
            }
            scores[out] = W.score[par][slot];
            items[out] = item;
        } else {
            for (int lv = 0; lv < L; ++lv) sids[out * L + lv] = 0;
            scores[out] = -INFINITY;
            items[out] = -1;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        counts[orow] = rec.rows;
        W.rec[req].status = kReqFree;
    }
}

__global__ void k_export_req(WaveDev W, int32_t *rows, int32_t *level) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= W.R) return;
    const ReqRec r = W.rec[i];
    if (rows) rows[i] = r.status == kReqActive ? r.rows : 0;
    if (level) level[i] = r.level;
}

}  // namespace

// ---------------------------------------------------------------------- launchers
hipError_t launch_clear_wave(const WaveDev &w, hipStream_t s) {
    const int n = w.R * w.MT > w.R ? w.R * w.MT : w.R;
    hipLaunchKernelGGL(k_clear_wave, dim3((n + 255) / 256), dim3(256), 0, s, w);
    return hipGetLastError();
}

hipError_t launch_init(const WaveDev &w, int par, const InitBatch &b, hipStream_t s) {
    hipLaunchKernelGGL(k_init, dim3(1), dim3(InitBatch::kMax), 0, s, w, par, b);
    return hipGetLastError();
}

template <int DT, int NORM, bool VEC>
static void launch_expand_t(const TrieDev &t, const WaveDev &w, int par, int n_req, const void *logits,
                            int64_t ld, hipStream_t s) {
    hipLaunchKernelGGL((k_expand<DT, NORM, VEC>), dim3(n_req * w.MT), dim3(kExpandThreads), 0, s, t, w,
                       par, logits, ld);
}

hipError_t launch_expand(const TrieDev &t, const WaveDev &w, int par, int n_req, const void *logits,
                         int64_t ld, int dtype, hipStream_t s) {
    if (n_req <= 0) return hipSuccess;
    const bool vec = t.V == 256 && (ld % 4) == 0 &&
                     ((uintptr_t)logits % (dtype == TCB_F32 ? 16 : 8)) == 0;
    const bool lvl = w.norm == TCB_NORM_LEVEL;
    if (dtype == TCB_F32) {
        if (vec) lvl ? launch_expand_t<TCB_F32, TCB_NORM_LEVEL, true>(t, w, par, n_req, logits, ld, s)
                     : launch_expand_t<TCB_F32, TCB_NORM_CHILDREN, true>(t, w, par, n_req, logits, ld, s);
        else lvl ? launch_expand_t<TCB_F32, TCB_NORM_LEVEL, false>(t, w, par, n_req, logits, ld, s)
                 : launch_expand_t<TCB_F32, TCB_NORM_CHILDREN, false>(t, w, par, n_req, logits, ld, s);
    } else {
        if (vec) lvl ? launch_expand_t<TCB_BF16, TCB_NORM_LEVEL, true>(t, w, par, n_req, logits, ld, s)
                     : launch_expand_t<TCB_BF16, TCB_NORM_CHILDREN, true>(t, w, par, n_req, logits, ld, s);
        else lvl ? launch_expand_t<TCB_BF16, TCB_NORM_LEVEL, false>(t, w, par, n_req, logits, ld, s)
                 : launch_expand_t<TCB_BF16, TCB_NORM_CHILDREN, false>(t, w, par, n_req, logits, ld, s);
    }
    return hipGetLastError();
}

hipError_t launch_merge(const TrieDev &t, const WaveDev &w, int par, int n_req, hipStream_t s) {
    if (n_req <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_merge, dim3(n_req), dim3(kMergeThreads), 0, s, t, w, par);
    return hipGetLastError();
}

hipError_t launch_finalize(const TrieDev &t, const WaveDev &w, int par, const FinBatch &b, uint8_t *sids,
                           float *scores, int64_t *items, int32_t *counts, hipStream_t s) {
    hipLaunchKernelGGL(k_finalize, dim3(b.n), dim3(256), 0, s, t, w, par, b, sids, scores, items, counts);
    return hipGetLastError();
}

hipError_t launch_export_req(const WaveDev &w, int32_t *rows, int32_t *level, hipStream_t s) {
    hipLaunchKernelGGL(k_export_req, dim3((w.R + 255) / 256), dim3(256), 0, s, w, rows, level);
    return hipGetLastError();
}

}  // namespace tcb

namespace tcb {
hipError_t launch_expand_lmhead(const TrieDev &, const WaveDev &, int, int, const void *, int64_t, int,
                                const void *, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace tcb
