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
//           The masked log-softmax is two wave reductions. Candidates are counted in
//           request-wide score bins (distance below the request's best row score,
//           which no candidate can exceed); the tile keeps the bins down to the one
//           holding its own n-th best, a superset of its top-n, and writes the bin
//           counts of what it kept.
//   merge   one workgroup per request: sums the tiles' bin counts to find the bin
//           b* of the request's n-th candidate before reading any candidate, stages
//           only bins <= b* in LDS grouped by bin, ranks each by counting the better
//           members of its bin, and writes the new rows (parent-gather / trie-advance)
//           plus the per-level back-pointers.
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

// ---------------------------------------------------------------------- expand
// Per-thread candidate store: kRowsPerWave rows x 4 codes.
constexpr int kE = kRowsPerWave * 4;

__device__ __forceinline__ uint32_t score_bin(float sref, float s) {
    const float d = (sref - s) * kHistRes;
    return d < (float)(kHistBins - 1) ? (uint32_t)d : (uint32_t)(kHistBins - 1);
}

template <int DT, int NORM, bool VEC>
__global__ __launch_bounds__(kExpandThreads) void k_expand(TrieDev T, WaveDev W, int par,
                                                           const void *__restrict__ logits, int64_t ld) {
    static_assert(kExpandThreads == kHistBins, "one histogram bin per thread");
    __shared__ uint32_t s_wmask[kTileWaves][kRowsPerWave][8];
    __shared__ uint32_t s_hist[kHistBins];
    __shared__ SelSmem S;
    __shared__ uint32_t s_bstar;

    const int req = blockIdx.x / W.MT;
    const int lt = blockIdx.x - req * W.MT;
    const ReqRec rec = W.rec[req];
    if (rec.status != kReqActive || rec.level >= T.L) return;
    const int r0 = lt * kTileRows;
    if (r0 >= rec.rows) return;
    const int level = rec.level;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int V = T.V;
    const float sref = W.score[par][rec.base];      // best row of the request (rank order)
    s_hist[tid] = 0u;
    if (tid == 0) s_bstar = kHistBins - 1;

    // 1. state and logits of this wave's rows, all issued before any use
    int rr[kRowsPerWave];
    bool live[kRowsPerWave];
    int32_t nd[kRowsPerWave];
    float sr[kRowsPerWave];
    float x[kRowsPerWave][4];
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
        rr[j] = r0 + j * kTileWaves + wave;
        live[j] = rr[j] < rec.rows;
        nd[j] = -1;
        sr[j] = 0.0f;
        x[j][0] = x[j][1] = x[j][2] = x[j][3] = 0.0f;
        if (live[j]) {
            const int slot = rec.base + rr[j];
            nd[j] = W.node[par][slot];
            sr[j] = W.score[par][slot];
            load_row<DT, VEC>(logits, ld, slot, lane, V, x[j]);
        }
    }
    // 2. trie: child range (and the dense child mask at shallow depths) of every row
    const bool dense = level < T.mask_depths;
    const uint32_t lo_id = T.off[level], hi_id = T.off[level + 1];
    bool ok[kRowsPerWave];
    uint32_t cb[kRowsPerWave], ce[kRowsPerWave], m[kRowsPerWave][8];
    bool bad_node = false;
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
        ok[j] = false;
        cb[j] = ce[j] = 0u;
#pragma unroll
        for (int w = 0; w < 8; ++w) m[j][w] = 0u;
        if (!live[j]) continue;                                   // wave-uniform
        const uint32_t n = (uint32_t)__builtin_amdgcn_readfirstlane(nd[j]);
        if (n < lo_id || n >= hi_id) {
            bad_node = true;
            continue;
        }
        ok[j] = true;
        cb[j] = T.child_begin[n];
        if (dense) {
#pragma unroll
            for (int w = 0; w < 8; ++w) m[j][w] = T.mask[(size_t)n * 8 + w];
        } else {
            ce[j] = T.child_begin[n + 1];
        }
    }
    if (bad_node && lane == 0) atomicOr(W.err, kErrBadNode);
    // 3. deeper down: each row's CSR child list becomes a mask in wave-private LDS
    if (!dense) {
        uint32_t cc[kRowsPerWave][4];
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t p = cb[j] + (uint32_t)(lane + 64 * q);
                cc[j][q] = (ok[j] && p < ce[j]) ? (uint32_t)T.child_code[p] : 0xffffffffu;
            }
        if (lane < 8) {
#pragma unroll
            for (int j = 0; j < kRowsPerWave; ++j) s_wmask[wave][j][lane] = 0u;
        }
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (cc[j][q] != 0xffffffffu) atomicOr(&s_wmask[wave][j][cc[j][q] >> 5], 1u << (cc[j][q] & 31));
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < kRowsPerWave; ++j)
#pragma unroll
            for (int w = 0; w < 8; ++w) m[j][w] = __builtin_amdgcn_readfirstlane(s_wmask[wave][j][w]);
    }

    // 4. masked log-softmax and the candidates of this lane's 4 codes of each row
    uint32_t co[kE];     // order keys
    int32_t cn[kE];      // child node ids
    uint32_t valid = 0u;
    bool bad_value = false;
    const int wl = lane >> 3, sh = (lane & 7) * 4;   // this lane's codes: word wl, bits sh..sh+3
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            co[j * 4 + q] = 0u;
            cn[j * 4 + q] = 0;
        }
        if (!ok[j]) continue;                                     // wave-uniform
        uint32_t below = 0u, word = 0u;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            below += (w < wl) ? (uint32_t)__popc(m[j][w]) : 0u;
            word = (w == wl) ? m[j][w] : word;
        }
        const uint32_t bits4 = (word >> sh) & 0xFu;
        const uint32_t rank0 = below + (uint32_t)__popc(word & ((1u << sh) - 1u));
        if (W.validate) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (4 * lane + q < V && !isfinite(x[j][q])) bad_value = true;
        }
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
            co[e] = f2ord(sr[j] + (x[j][q] - lse));
            cn[e] = (int32_t)(cb[j] + rank0 + (uint32_t)__popc(bits4 & ((1u << q) - 1u)));
            valid |= ((bits4 >> q) & 1u) << e;
        }
    }
    if (bad_value) atomicOr(W.err, kErrNonFinite);

    auto flat_of = [&](int e) -> uint32_t {
        return (uint32_t)rr[e >> 2] * 256u + (uint32_t)(4 * lane + (e & 3));
    };

    // 5. histogram of the tile's candidates over the request-wide score bins
    __syncthreads();
    {
        uint32_t over = 0u;
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            if ((valid >> e) & 1u) {
                const uint32_t b = score_bin(sref, ord2f(co[e]));
                if (b < (uint32_t)(kHistBins - 1)) atomicAdd(&s_hist[b], 1u);
                else ++over;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) over += (uint32_t)__shfl_xor((int)over, o, 64);
        if (lane == 0 && over) atomicAdd(&s_hist[kHistBins - 1], over);
    }
    __syncthreads();
    // 6. boundary bin of the tile: where the count from the best bin reaches n_i
    const uint32_t width = (uint32_t)rec.width;
    const uint32_t h = s_hist[tid];
    int total;
    const int before = block_excl_scan<kExpandThreads>((int)h, S.part, &total);
    if ((uint32_t)total > width && (uint32_t)before < width && width <= (uint32_t)before + h) s_bstar = (uint32_t)tid;
    __syncthreads();
    const uint32_t bstar = s_bstar;
    uint32_t keep = 0u;
#pragma unroll
    for (int e = 0; e < kE; ++e)
        if (((valid >> e) & 1u) && score_bin(sref, ord2f(co[e])) <= bstar) keep |= 1u << e;
    int kept;
    int off = block_excl_scan<kExpandThreads>(__popc(keep), S.part, &kept);
    const bool exact = kept > W.CAPT;
    if (exact) {
        // the boundary bin is too full (e.g. many exact ties): keep exactly the tile's top n_i
        auto each = [&](auto fn) {
#pragma unroll
            for (int e = 0; e < kE; ++e)
                if ((valid >> e) & 1u) fn(co[e], flat_of(e));
        };
        uint32_t o_star, f_star;
        block_select<kExpandThreads>(each, width, S, o_star, f_star, W.err);
        keep = 0u;
#pragma unroll
        for (int e = 0; e < kE; ++e)
            if (((valid >> e) & 1u) && key_le(co[e], flat_of(e), o_star, f_star)) keep |= 1u << e;
        off = block_excl_scan<kExpandThreads>(__popc(keep), S.part, &kept);
        s_hist[tid] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kE; ++e)
            if ((keep >> e) & 1u) atomicAdd(&s_hist[score_bin(sref, ord2f(co[e]))], 1u);
        __syncthreads();
    }
    // 7. emit the kept candidates and their bin counts
    Cand *out = reinterpret_cast<Cand *>(W.cand) + ((size_t)req * W.MT + lt) * W.CAPT;
    int i = off;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        if ((keep >> e) & 1u) {
            Cand c;
            c.score = ord2f(co[e]);
            c.flat = flat_of(e);
            c.node = cn[e];
            c.pad = 0u;
            out[i++] = c;
        }
    }
    const uint32_t hk = exact ? s_hist[tid] : ((uint32_t)tid <= bstar ? h : 0u);
    W.tile_hist[((size_t)req * W.MT + lt) * kHistBins + tid] = (uint16_t)hk;
    if (tid == 0) W.tile_count[req * W.MT + lt] = kept;
}

// ---------------------------------------------------------------------- merge
// One workgroup per request. The tiles' bin counts give the request's boundary bin
// b* before any candidate is read; only candidates in bins <= b* are staged, already
// grouped by bin, and each finds its rank by counting the better members of its bin.
struct MergeSmem {
    float s[kMergeCap];
    uint32_t f[kMergeCap];
    int32_t node[kMergeCap];
    uint32_t ghist[kHistBins];
    uint32_t gstart[kHistBins];
    uint32_t cursor[kHistBins];
    int32_t tcnt[kMaxTilesPerReq];
    SelSmem sel;
    uint32_t bstar, n, o_star, f_star;
};

constexpr int kBigBin = 1024;   // boundary bins larger than this use the exact selection

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
    const float sref = W.score[par][rec.base];
    const int CAPT = W.CAPT;
    const Cand *cand = reinterpret_cast<const Cand *>(W.cand) + (size_t)req * W.MT * CAPT;
    const uint16_t *th = W.tile_hist + (size_t)req * W.MT * kHistBins;

    // request-wide bin counts = sum of the tiles' counts
    uint32_t h = 0u;
    if (t < kHistBins) {
        M.cursor[t] = 0u;
        int tile = 0;
        for (; tile + 4 <= ntile; tile += 4) {
            const uint32_t a = th[(size_t)(tile + 0) * kHistBins + t];
            const uint32_t b = th[(size_t)(tile + 1) * kHistBins + t];
            const uint32_t c = th[(size_t)(tile + 2) * kHistBins + t];
            const uint32_t d = th[(size_t)(tile + 3) * kHistBins + t];
            h += a + b + c + d;
        }
        for (; tile < ntile; ++tile) h += th[(size_t)tile * kHistBins + t];
        M.ghist[t] = h;
    }
    if (t < ntile) M.tcnt[t] = W.tile_count[req * W.MT + t];
    if (t == 0) {
        M.bstar = kHistBins - 1;
        M.n = 0u;
    }
    int total;
    const int before = block_excl_scan<NT>((int)h, M.sel.part, &total);
    const uint32_t k = min((uint32_t)rec.width, (uint32_t)total);
    if (t < kHistBins) {
        M.gstart[t] = (uint32_t)before;
        if ((uint32_t)before < k && k <= (uint32_t)before + h) M.bstar = (uint32_t)t;
    }
    __syncthreads();
    const uint32_t bstar = M.bstar;
    const uint32_t cbefore = M.gstart[bstar], cnt_b = M.ghist[bstar];
    const uint32_t staged = cbefore + cnt_b;
    const uint32_t need = k - cbefore;          // members of b* that survive
    const int S = W.S;
    const int level = rec.level;

    auto write_row = [&](uint32_t rank, float score, uint32_t flat, int32_t node) {
        const int slot = rec.base + (int)rank;
        W.node[nxt][slot] = node;
        W.score[nxt][slot] = score;
        W.parent_slot[slot] = rec.base + (int)(flat >> 8);
        W.hist[(size_t)level * S + slot] = flat;               // (r << 8) | c
    };

    if (staged <= (uint32_t)kMergeCap) {
        // stage bins <= b*, grouped by bin
        constexpr int U = 8;
        for (int tb = 0; tb < ntile; tb += U) {
            for (int i0 = 0; i0 < CAPT; i0 += NT) {
                Cand c[U];
                bool okc[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int tile = tb + u, i = i0 + t;
                    okc[u] = tile < ntile && i < M.tcnt[tile < ntile ? tile : 0];
                    if (okc[u]) c[u] = cand[(size_t)tile * CAPT + i];
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (!okc[u]) continue;
                    const uint32_t b = score_bin(sref, c[u].score);
                    if (b <= bstar) {
                        const uint32_t p = M.gstart[b] + atomicAdd(&M.cursor[b], 1u);
                        if (p < staged) {          // holds by construction; never write past it
                            M.s[p] = c[u].score;
                            M.f[p] = c[u].flat;
                            M.node[p] = c[u].node;
                        }
                    }
                }
            }
        }
        __syncthreads();
        // a very full boundary bin: find its need-th member exactly first
        const bool big = cnt_b > (uint32_t)kBigBin && need < cnt_b;
        uint32_t o_star = 0u, f_star = 0xffffffffu;
        if (big) {
            auto each_b = [&](auto fn) {
                for (uint32_t p = cbefore + t; p < staged; p += NT) fn(f2ord(M.s[p]), M.f[p]);
            };
            block_select<NT>(each_b, need, M.sel, o_star, f_star, W.err);
        }
        for (uint32_t p = t; p < staged; p += NT) {
            const float sc = M.s[p];
            const uint32_t o = f2ord(sc), fl = M.f[p];
            const uint32_t b = score_bin(sref, sc);
            if (b == bstar && big && !key_le(o, fl, o_star, f_star)) continue;
            const uint32_t st = M.gstart[b], en = st + M.ghist[b];
            uint32_t r = 0u;
            for (uint32_t q = st; q < en; ++q) {
                const uint32_t o2 = f2ord(M.s[q]), f2 = M.f[q];
                r += (o2 > o || (o2 == o && f2 < fl)) ? 1u : 0u;
            }
            if (b < bstar || r < need) write_row(st + r, sc, fl, M.node[p]);
        }
    } else {
        // spill: select straight from the tiles' buffers, then rank the k survivors
        if (t == 0) atomicOr(W.err, kInfoMergeSpill);
        auto each_g = [&](auto fn) {
            for (int tile = 0; tile < ntile; ++tile)
                for (int i = t; i < M.tcnt[tile]; i += NT) {
                    const Cand c = cand[(size_t)tile * CAPT + i];
                    if (score_bin(sref, c.score) <= bstar) fn(f2ord(c.score), c.flat);
                }
        };
        uint32_t o_star, f_star;
        block_select<NT>(each_g, k, M.sel, o_star, f_star, W.err);
        for (int tile = 0; tile < ntile; ++tile)
            for (int i = t; i < M.tcnt[tile]; i += NT) {
                const Cand c = cand[(size_t)tile * CAPT + i];
                const uint32_t o = f2ord(c.score);
                if (score_bin(sref, c.score) <= bstar && key_le(o, c.flat, o_star, f_star)) {
                    const uint32_t p = atomicAdd(&M.n, 1u);
                    if (p < (uint32_t)kMergeCap) {
                        M.s[p] = c.score;
                        M.f[p] = c.flat;
                        M.node[p] = c.node;
                    }
                }
            }
        __syncthreads();
        const uint32_t n = min(M.n, (uint32_t)kMergeCap);
        if (t == 0 && M.n != k) atomicOr(W.err, kErrInternal);
        for (uint32_t p = t; p < n; p += NT) {
            const uint32_t o = f2ord(M.s[p]), fl = M.f[p];
            uint32_t r = 0u;
            for (uint32_t q = 0; q < n; ++q) {
                const uint32_t o2 = f2ord(M.s[q]), f2 = M.f[q];
                r += (o2 > o || (o2 == o && f2 < fl)) ? 1u : 0u;
            }
            write_row(r, M.s[p], fl, M.node[p]);
        }
    }
    if (t == 0) {
        W.rec[req].rows = (int32_t)k;
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
    if (i < W.R * W.MT) W.tile_count[i] = 0;
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
