// gfx950 device code of the catalog-constrained wide-beam step, shared by the
// translation units that instantiate it (kernels.hip and the tile_*.hip files, each of
// which compiles one logits type / sampling variant of the tile kernel).
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
//   k_tile   workgroup = a tile of 64 consecutive rows of one request. 16 lanes per
//            row (one DPP row), 16 codes per lane: a row is one coalesced 1 KiB (fp32)
//            or 512 B (bf16) load. The child set is a 256-bit mask, read from the
//            trie's per-node masks or, at depths stored without them, built in LDS from
//            the CSR child list (bit-identical results). Masked log-softmax with DPP
//            reductions inside the 16-lane row. Candidates are binned request-wide; a
//            per-lane sample bounds the tile's n-th best so that only a few candidates
//            need exact treatment; the tile keeps every bin down to the one where its own
//            count reaches n (a superset of its top-n) and writes them as 16-byte
//            records grouped by bin, plus its cumulative bin counts.
//   k_merge  one workgroup per request: sums the tiles' cumulative counts to find the
//            bin b* of the request's n-th candidate, stages only bins <= b* in LDS, ranks
//            each candidate by counting the better members of its own bin, and writes the
//            new rows (parent-gather / trie-advance) and the back-pointers.
// The tiles of a request and its merge run on one XCD (workgroups are dealt to the 8
// XCDs round-robin), so the candidates pass through that XCD's L2.
// Selection keys are unique (the flat index breaks score ties) and every float
// reduction has a fixed order, so results are deterministic run to run.
#pragma once

#include "tcb_internal.h"

namespace tcb {
namespace {

// ---------------------------------------------------------------------- helpers
__device__ __forceinline__ uint32_t f2ord(float f) {   // order-preserving, -0 == +0
    const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool key_better(uint32_t o, uint32_t f, uint32_t o2, uint32_t f2) {
    return o > o2 || (o == o2 && f < f2);     // (score desc, flat asc)
}
__device__ __forceinline__ bool key_le(uint32_t o, uint32_t f, uint32_t o_star, uint32_t f_star) {
    return o > o_star || (o == o_star && f <= f_star);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bin = min(kBins - 1, floor(max(0, (sref - s) * kBinRes))). The fma rounds
// kBinRes * sref - kBinRes * s once, which equals kBinRes * fl(sref - s) exactly
// (kBinRes is a power of two), so every caller bins identically.
__device__ __forceinline__ uint32_t score_bin(float sref, float s) {
    const float d = fmaf(s, -kBinRes, sref * kBinRes);
    return (uint32_t)__builtin_amdgcn_fmed3f(d, 0.0f, (float)(kBins - 1));
}

// DPP moves within a row of 16 lanes; every reduction below leaves the result in all
// 16 lanes of the row (the butterfly pairs are symmetric, so the values are bitwise equal).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF,
                                                                 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;    // row_half_mirror: lane i <-> 7-i within 8
constexpr int kMirror = 0x140;        // row_mirror: lane i <-> 15-i within 16

__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<kQuadXor1>(v));
    v = fmaxf(v, dpp_f<kQuadXor2>(v));
    v = fmaxf(v, dpp_f<kHalfMirror>(v));
    v = fmaxf(v, dpp_f<kMirror>(v));
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<kQuadXor1>(v);
    v += dpp_f<kQuadXor2>(v);
    v += dpp_f<kHalfMirror>(v);
    v += dpp_f<kMirror>(v);
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
// Inclusive scan over the 64 lanes of a wave with DPP: shifts inside each row of 16
// lanes, then the last lane of a row is broadcast into the following rows.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += dpp_u<0x111, 0xF>(x);   // row_shr:1
    x += dpp_u<0x112, 0xF>(x);   // row_shr:2
    x += dpp_u<0x114, 0xF>(x);   // row_shr:4
    x += dpp_u<0x118, 0xF>(x);   // row_shr:8
    x += dpp_u<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_u<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// smallest value over the 16 lanes of a row (in all 16 lanes)
__device__ __forceinline__ uint32_t row16_min_u(uint32_t v) {
    v = min(v, dpp_u<kQuadXor1, 0xF>(v));
    v = min(v, dpp_u<kQuadXor2, 0xF>(v));
    v = min(v, dpp_u<kHalfMirror, 0xF>(v));
    v = min(v, dpp_u<kMirror, 0xF>(v));
    return v;
}

// Phase trace (diagnostics): thread 0 records the real-time clock (100 MHz) when its
// workgroup passes mark i; mark 0 records the XCD. A uniform test of a kernel argument when
// tracing is off.
__device__ __forceinline__ void trace_mark(const WaveDev &W, int i) {
    if (W.trace != nullptr && threadIdx.x == 0) {
        uint64_t v;
        if (i == 0) v = 1u + (__builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 15u);  // HW_REG_XCC_ID
        else v = wall_clock64();
        W.trace[(size_t)blockIdx.x * kTraceSlots + i] = v;
    }
}

// LDS ordering among the lanes of one wave (no workgroup barrier needed)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive scan of one value per thread over a workgroup of NT threads.
template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t *part) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) part[w] = x;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) before += (i < w) ? part[i] : 0u;
    __syncthreads();
    return before + x;
}

// ---------------------------------------------------------------------- exact selection
// The k-th best of a set of (order key o, flat f) pairs spread over the threads of a
// workgroup (best = larger o, then smaller f). The active key range [lo, hi] shrinks by
// 1024-bin histograms of the distance to hi (binned by a shift, so the range's extremes
// fall in different bins and every round makes progress); once one key value is left,
// the same is done on the flat index. Used only where ties defeat the score bins.
struct SelSmem {
    uint32_t hist[kSelBins];
    uint32_t part[kWaves];
    uint32_t lo, hi, bstar, need;
};

__device__ __forceinline__ int range_shift(uint32_t range) {
    const int bits = 32 - __clz((int)range);          // range >= 1
    return bits > 10 ? bits - 10 : 0;
}

template <int NT>
__device__ __forceinline__ void find_bstar(SelSmem &S, uint32_t need) {
    static_assert(kSelBins == NT, "one selection bin per thread");
    const uint32_t h = S.hist[threadIdx.x];
    const uint32_t incl = block_incl_scan<NT>(h, S.part);
    if (incl - h < need && need <= incl) {
        S.bstar = threadIdx.x;
        S.need = need - (incl - h);
    }
    __syncthreads();
}

template <int NT, class Each>
__device__ void block_select(Each each, uint32_t k, SelSmem &S, uint32_t &o_star, uint32_t &f_star,
                             uint32_t *err) {
    const int t = threadIdx.x;
    auto reset = [&]() {
        S.hist[t] = 0u;
        if (t == 0) {
            S.lo = 0xffffffffu;
            S.hi = 0u;
        }
    };
    auto minmax = [&](uint32_t a, uint32_t b) {
        a = wave_min_u(a);
        b = wave_max_u(b);
        if ((t & 63) == 0) {
            atomicMin(&S.lo, a);
            atomicMax(&S.hi, b);
        }
    };
    reset();
    __syncthreads();
    {
        uint32_t a = 0xffffffffu, b = 0u;
        each([&](uint32_t o, uint32_t) {
            a = min(a, o);
            b = max(b, o);
        });
        minmax(a, b);
    }
    __syncthreads();
    uint32_t lo = S.lo, hi = S.hi, need = k;
    __syncthreads();
    // phase 1: the key value of the k-th element (4 rounds suffice; the cap turns a
    // logic error into a flagged error instead of a hang)
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
        __syncthreads();
        reset();
        __syncthreads();
        uint32_t a = 0xffffffffu, b = 0u;
        each([&](uint32_t o, uint32_t) {
            if (o >= lo && o <= hi && ((hi - o) >> sh) == bs) {
                a = min(a, o);
                b = max(b, o);
            }
        });
        minmax(a, b);
        __syncthreads();
        lo = S.lo;
        hi = S.hi;
        need = nn;
        __syncthreads();
    }
    // phase 2: among elements with key lo, the need-th smallest flat index
    reset();
    __syncthreads();
    {
        uint32_t a = 0xffffffffu, b = 0u;
        each([&](uint32_t o, uint32_t f) {
            if (o == lo) {
                a = min(a, f);
                b = max(b, f);
            }
        });
        minmax(a, b);
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
        __syncthreads();
        reset();
        __syncthreads();
        uint32_t a = 0xffffffffu, b = 0u;
        each([&](uint32_t o, uint32_t f) {
            if (o == lo && f >= flo && f <= fhi && ((f - flo) >> sh) == bs) {
                a = min(a, f);
                b = max(b, f);
            }
        });
        minmax(a, b);
        __syncthreads();
        flo = S.lo;
        fhi = S.hi;
        need = nn;
        __syncthreads();
    }
    o_star = lo;
    f_star = flo;
}

// ---------------------------------------------------------------------- row layout
// Lane j (0..15) of a row's 16-lane group holds element e = i*CW + q (chunk i, q < CW)
// = code i*(256/CH) + j*CW + q, so every load instruction of the group reads one
// contiguous 256-byte piece of the row.
template <int DT>
struct Lay;
template <>
struct Lay<TCB_F32> {
    static constexpr int CH = 4, CW = 4;
};
template <>
struct Lay<TCB_BF16> {
    static constexpr int CH = 2, CW = 8;
};
constexpr int kElems = 16;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ int code_of(int e, int j) {
    constexpr int CW = Lay<DT>::CW, SPAN = 256 / Lay<DT>::CH;
    return (e / CW) * SPAN + j * CW + (e % CW);
}

template <int DT, bool VEC>
__device__ __forceinline__ void load_row(const void *logits, int64_t ld, int slot, int j, int V,
                                         float (&x)[kElems]) {
    if constexpr (VEC) {
        if constexpr (DT == TCB_F32) {
            const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(logits) +
                                                             (size_t)slot * (size_t)ld);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = __builtin_nontemporal_load(p + 16 * i + j);
                x[4 * i + 0] = v[0];
                x[4 * i + 1] = v[1];
                x[4 * i + 2] = v[2];
                x[4 * i + 3] = v[3];
            }
        } else {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(logits) +
                                                             (size_t)slot * (size_t)ld);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const u32x4 v = __builtin_nontemporal_load(p + 16 * i + j);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    x[8 * i + 2 * w] = __uint_as_float(v[w] << 16);
                    x[8 * i + 2 * w + 1] = __uint_as_float(v[w] & 0xffff0000u);
                }
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            const int c = code_of<DT>(e, j);
            float v = 0.0f;
            if (c < V) {
                if constexpr (DT == TCB_F32)
                    v = static_cast<const float *>(logits)[(size_t)slot * (size_t)ld + c];
                else
                    v = __uint_as_float(
                        (uint32_t) static_cast<const uint16_t *>(logits)[(size_t)slot * (size_t)ld + c] << 16);
            }
            x[e] = v;
        }
    }
}

// A row's logits as loaded (16-byte pieces), before widening to fp32: loading into these and
// widening only where the values are used keeps a load issued early from being waited on
// at once (a widening inside a branch would make the branch join wait for it).
template <int DT>
struct RawRow;
template <>
struct RawRow<TCB_F32> {
    f32x4 v[4];
};
template <>
struct RawRow<TCB_BF16> {
    u32x4 v[2];
};
template <int DT>
__device__ __forceinline__ void load_row_raw(const void *logits, int64_t ld, int slot, int j, RawRow<DT> &raw) {
    if constexpr (DT == TCB_F32) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(logits) + (size_t)slot * (size_t)ld);
#pragma unroll
        for (int i = 0; i < 4; ++i) raw.v[i] = __builtin_nontemporal_load(p + 16 * i + j);
    } else {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(logits) + (size_t)slot * (size_t)ld);
#pragma unroll
        for (int i = 0; i < 2; ++i) raw.v[i] = __builtin_nontemporal_load(p + 16 * i + j);
    }
}
template <int DT>
__device__ __forceinline__ void widen_row(const RawRow<DT> &raw, float (&x)[kElems]) {
    if constexpr (DT == TCB_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[4 * i + 0] = raw.v[i][0];
            x[4 * i + 1] = raw.v[i][1];
            x[4 * i + 2] = raw.v[i][2];
            x[4 * i + 3] = raw.v[i][3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                x[8 * i + 2 * w] = __uint_as_float(raw.v[i][w] << 16);
                x[8 * i + 2 * w + 1] = __uint_as_float(raw.v[i][w] & 0xffff0000u);
            }
    }
}

// Only the chunks of a row whose bit in `chunks` is set (16-byte pieces, as load_row reads
// them); the others stay 0. Used where a row's children touch few of its sectors.
template <int DT>
__device__ __forceinline__ void load_row_chunks(const void *logits, int64_t ld, int slot, int j, uint32_t chunks,
                                                float (&x)[kElems]) {
    if constexpr (DT == TCB_F32) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(logits) + (size_t)slot * (size_t)ld);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if ((chunks >> i) & 1u) {
                const f32x4 v = __builtin_nontemporal_load(p + 16 * i + j);
                x[4 * i + 0] = v[0];
                x[4 * i + 1] = v[1];
                x[4 * i + 2] = v[2];
                x[4 * i + 3] = v[3];
            }
    } else {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(logits) + (size_t)slot * (size_t)ld);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            if ((chunks >> i) & 1u) {
                const u32x4 v = __builtin_nontemporal_load(p + 16 * i + j);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    x[8 * i + 2 * w] = __uint_as_float(v[w] << 16);
                    x[8 * i + 2 * w + 1] = __uint_as_float(v[w] & 0xffff0000u);
                }
            }
    }
}

// ---------------------------------------------------------------------- children-only lm_head
// flashrec 0.1.0, Features > Decoding: the head is evaluated only over the SID range, and
// the trie is used dense or sparse by depth. Where a row has about one child, the logits
// of its other codes are never used (they are masked off), so the tile computes only
//     x[c] = sum_h hidden[slot][h] * W[level][c][h]      for each child code c of the row
// (bf16 operands widened exactly, fp32 sums). A wave takes its 4 rows' (row, child) pairs
// one at a time, rows in order and each row's children lowest code first, and all 64 lanes
// share each pair: lane l sums the products of the rows' 16-byte pieces l, l + 64, ...
// (8 elements each, in element order), then the 64 lane sums are added in a fixed order
// (a DPP butterfly within each 16-lane row, then across rows), so a logit does not depend
// on the launch and every lane holds the same value; the lane owning the code keeps it in
// x. One pair's operand loads are all in flight at once (4 pieces of each operand per lane
// at H = 2048). tv: the lane's codes that are children (bit e <-> code code_of(e, j)); g:
// the lane's row in the wave; slot: the slot of the lane's row.
__device__ __forceinline__ float dot8_bf16(const u32x4 &a, const u32x4 &b, float acc) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        acc = fmaf(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), acc);
        acc = fmaf(__uint_as_float(a[w] & 0xffff0000u), __uint_as_float(b[w] & 0xffff0000u), acc);
    }
    return acc;
}

constexpr int kHeadBatch = 4;                               // pieces of each operand per lane per load round

template <int DT>
__device__ __forceinline__ void head_children(const StepHead &hd, int slot, int level, int g, int j, uint32_t tv,
                                              float (&x)[kElems]) {
    const int lane = (int)(threadIdx.x & 63u);
    const uint16_t *wl = hd.weight + (size_t)level * 256 * (size_t)hd.H;
    const int pieces = hd.H >> 3;                           // 16-byte pieces of a row
    uint32_t rem = tv;
#pragma unroll 1
    for (int gg = 0; gg < 4; ++gg) {
        const u32x4 *hp = reinterpret_cast<const u32x4 *>(
            hd.hidden + (size_t)__builtin_amdgcn_readlane(slot, 16 * gg) * (size_t)hd.ld);
#pragma unroll 1
        while (true) {
            const int e0 = rem ? __builtin_ctz(rem) : 0;
            const uint32_t mine = rem ? (uint32_t)code_of<DT>(e0, j) : 256u;
            // row gg's next child code (256: none left), the same in every lane
            const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)row16_min_u(mine), 16 * gg);
            if (c >= 256u) break;
            const u32x4 *wp = reinterpret_cast<const u32x4 *>(wl + (size_t)c * (size_t)hd.H);
            float acc = 0.0f;
#pragma unroll 1
            for (int p0 = 0; p0 < pieces; p0 += 64 * kHeadBatch) {
                u32x4 hv[kHeadBatch], wv[kHeadBatch];
#pragma unroll
                for (int i = 0; i < kHeadBatch; ++i) {
                    const int p = min(p0 + 64 * i + lane, pieces - 1);   // past the row: read, not summed
                    hv[i] = __builtin_nontemporal_load(hp + p);
                    wv[i] = wp[p];
                }
#pragma unroll
                for (int i = 0; i < kHeadBatch; ++i)
                    if (p0 + 64 * i + lane < pieces) acc = dot8_bf16(hv[i], wv[i], acc);
            }
            acc = row16_sum(acc);
            acc += __shfl_xor(acc, 16, 64);
            acc += __shfl_xor(acc, 32, 64);
            if (g == gg && mine == c) {
#pragma unroll
                for (int e = 0; e < kElems; ++e)
                    if (e == e0) x[e] = acc;
                rem &= rem - 1u;
            }
        }
    }
}

// ---------------------------------------------------------------------- shared memory
struct alignas(16) MergeSmem {
    uint64_t key[kMergeCap];                       // staged entries' keys (merge_key): larger is better
    float s[kMergeCap];
    uint32_t f[kMergeCap];
    int32_t n[kMergeCap];
    float phi[kMergeCap];
    uint32_t G[kBins];                             // request-wide cumulative kept count
    uint32_t cur[kBins];                           // staging cursors
    uint32_t toff[kMaxTilesPerReq + 1];            // staged entries before each tile
    uint32_t bstar, cnt, pad[2];
};

// ---------------------------------------------------------------------- merge
// New row `rank` of request ra (in the request's other row buffers) and its back-pointer.
__device__ __forceinline__ void write_new_row(const WaveDev &W, const ReqArg ra, uint32_t rank, float score,
                                              uint32_t flat, int32_t node, float phi) {
    if (rank >= (uint32_t)ra.width()) return;         // cannot happen; never write past the request
    const int slot = ra.base() + (int)rank, np = ra.par() ^ 1;
    W.node[np][slot] = node;
    W.score[np][slot] = score;
    W.phi[np][slot] = phi;
    W.parent_slot[slot] = ra.base() + (int)(flat >> 8);
    W.hist[(size_t)ra.level() * W.S + slot] = flat;   // (r << 8) | c
}

// The request's record for the next step: k rows one level deeper, in the other buffers.
__device__ __forceinline__ void write_next_record(const WaveDev &W, int q, const ReqArg ra, int rp, uint32_t k) {
    if (threadIdx.x == 0) {
        ReqRec nr{};
        nr.base = ra.base();
        nr.width = ra.width();
        nr.rows = (int32_t)k;
        nr.level = ra.level() + 1;
        nr.status = kReqActive;
        nr.par = ra.par() ^ 1;
        W.rec[rp ^ 1][q] = nr;
    }
}

// An entry's selection key as one 64-bit word, larger = better: the order-preserving score
// above, the complemented flat index below (a lower flat index wins a tie).
__device__ __forceinline__ uint64_t merge_key(float s, uint32_t f) {
    return ((uint64_t)f2ord(s) << 32) | (uint64_t)(~f);
}

// Entries p < staged of M are grouped by bin (bin b at [G[b - 1], min(G[b], staged)),
// G[-1] = 0), each with its merge_key in M.key: an entry's rank is the entries of better bins
// plus the better members of its own bin. emit(rank, p, s, f) is called for every entry;
// ranks below k are the new rows.
template <class Emit>
__device__ __forceinline__ void rank_staged(const MergeSmem &M, const uint32_t *G, uint32_t staged, float sref,
                                            Emit emit) {
    constexpr int U = kMergeCap / kThreads;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t p = (uint32_t)(threadIdx.x + u * kThreads);
        if (p < staged) {
            const float s = M.s[p];
            const uint32_t f = M.f[p];
            const uint64_t key = M.key[p];
            const uint32_t b = score_bin(sref, s);
            const uint32_t st = b ? G[b - 1] : 0u, en = min(G[b], staged);
            uint32_t r = 0u, i = st;
            for (; i + 4u <= en; i += 4u)
                r += (M.key[i] > key ? 1u : 0u) + (M.key[i + 1] > key ? 1u : 0u) + (M.key[i + 2] > key ? 1u : 0u) +
                     (M.key[i + 3] > key ? 1u : 0u);
            for (; i < en; ++i) r += M.key[i] > key ? 1u : 0u;
            emit(st + r, p, s, f);
        }
    }
}

// ---------------------------------------------------------------------- finishing requests
// With StepFin set, the step that brings a request to depth L also does what k_finalize
// does: the request's beams, best first, go to row q of the outputs and both of its
// records become free.
__device__ __forceinline__ bool finishes(const TrieDev &T, const StepFin &F, const ReqArg ra) {
    return F.sids != nullptr && ra.level() + 1 == T.L;
}

// Whether `node` is a depth-L node (li: its leaf index); a node that is neither that nor
// the unconstrained wave's off-catalog -1 sets kErrBadNode.
__device__ __forceinline__ bool leaf_index(const TrieDev &T, const WaveDev &W, int32_t node, uint32_t &li) {
    const uint32_t leaf0 = T.off[T.L], leaf1 = T.off[T.L + 1];
    li = (uint32_t)node - leaf0;
    if ((uint32_t)node >= leaf0 && (uint32_t)node < leaf1) return true;
    if (!(W.norm == TCB_NORM_OPEN && node == -1)) atomicOr(W.err, kErrBadNode);
    return false;
}

__device__ __forceinline__ int64_t item_of(const TrieDev &T, const WaveDev &W, int32_t node) {
    uint32_t li;
    return leaf_index(T, W, node, li) ? (int64_t)T.leaf_item[li] : (int64_t)-1;
}

// Output entry `rank` of finished request q: codes c_0 .. c_{L-2} from pfx (byte t holds
// c_t), then c; the summed log-probability and the catalog item.
__device__ __forceinline__ void write_final_row(const StepFin &F, int L, int Bmax, int q, uint32_t rank,
                                                uint64_t pfx, uint32_t c, float phi, int64_t item) {
    const size_t out = (size_t)q * (size_t)Bmax + rank;
    uint8_t *sp = F.sids + out * (size_t)L;
    const uint64_t codes = pfx | ((uint64_t)c << (8 * (L - 1)));
    if (L == 4 && ((uintptr_t)sp & 3u) == 0) {          // one store where the row is aligned
        *reinterpret_cast<uint32_t *>(sp) = (uint32_t)codes;
    } else if (L == 8 && ((uintptr_t)sp & 7u) == 0) {
        *reinterpret_cast<uint64_t *>(sp) = codes;
    } else {
        for (int t = 0; t < L; ++t) sp[t] = (uint8_t)(codes >> (8 * t));
    }
    F.scores[out] = phi;
    F.items[out] = item;
}

// Codes of the request's row r at its current depth, walked back through the per-level
// back-pointers in memory; a pointer past the request's width sets kErrBadNode.
__device__ __forceinline__ uint64_t walk_prefix(const WaveDev &W, const ReqArg ra, uint32_t r) {
    uint64_t pfx = 0;
    for (int t = ra.level() - 1; t >= 0; --t) {
        if (r >= (uint32_t)ra.width()) {
            atomicOr(W.err, kErrBadNode);
            break;
        }
        const uint32_t h = W.hist[(size_t)t * W.S + ra.base() + r];
        pfx |= (uint64_t)(h & 255u) << (8 * t);
        r = h >> 8;
    }
    return pfx;
}

// New row `rank` of a finishing request: its output entry (the request is released, so no
// row state is written).
__device__ __forceinline__ void write_finished_row(const TrieDev &T, const WaveDev &W, const StepFin &F, int q,
                                                   const ReqArg ra, uint32_t rank, float s, uint32_t f,
                                                   int32_t node, float phi) {
    (void)s;
    if (rank < (uint32_t)ra.width())
        write_final_row(F, T.L, W.Bmax, q, rank, walk_prefix(W, ra, f >> 8), f & 255u, phi, item_of(T, W, node));
}

// The output entries past the request's k beams, its count, and its free records (in
// place of write_next_record). The record this step read keeps its row count (rows_in),
// so a relaunch of the step's kernels reads the same input.
__device__ __forceinline__ void finish_request(const TrieDev &T, const WaveDev &W, const StepFin &F, int q,
                                               const ReqArg ra, int rp, int rows_in, uint32_t k) {
    const int L = T.L;
    for (int j = (int)k + (int)threadIdx.x; j < W.Bmax; j += (int)blockDim.x) {
        const size_t out = (size_t)q * (size_t)W.Bmax + (size_t)j;
        for (int t = 0; t < L; ++t) F.sids[out * L + t] = 0;
        F.scores[out] = -INFINITY;
        F.items[out] = -1;
    }
    if (threadIdx.x == 0) {
        F.counts[q] = (int32_t)k;
        ReqRec fr{};
        fr.base = ra.base();
        fr.width = ra.width();
        fr.rows = (int32_t)k;
        fr.level = L;
        fr.status = kReqFree;
        fr.par = ra.par() ^ 1;
        W.rec[rp ^ 1][q] = fr;
        fr.rows = rows_in;
        W.rec[rp][q] = fr;
    }
}

// One workgroup per request (k_merge). Every tile's kept candidates are in its region
// of the candidate records grouped by bin, with its cumulative kept counts in tcum.
// Hs (or nullptr): LDS for the back-pointers of up to kThreads rows when the request finishes
// in this step, so that its beams' codes are walked on chip.
// out.row(rank, s, f, node, phi) takes each new row (rank < k) and out.done(k) the count,
// except for a finishing request, whose rows and records are written here.
template <class Out>
__device__ __forceinline__ void merge_request(const TrieDev &T, const WaveDev &W, const StepFin &F, int q,
                                              const ReqArg ra, int rp, MergeSmem &M, SelSmem &sel,
                                              uint32_t (*Hs)[kThreads], const Out &out) {
    const int tid = threadIdx.x;
    const int MT = W.MT, CAPT = W.CAPT;
    const int cpar = ra.level() & 1;                  // the buffers the step's tiles wrote
    const uint16_t *tc = W.tcum[cpar] + (size_t)q * MT * kBins;
    const size_t reg0 = (size_t)q * MT * CAPT;
    // the live-row count (how many tiles wrote counts), the best row's score and the
    // tiles' counts are all loaded at once: the counts of every tile the request could
    // have are read and those past the live tiles are dropped
    const bool fresh = ra.level() == 0;                // the initial state: one row, the root, score 0
    const int rows_ld = W.rec[rp][q].rows;             // read unconditionally (no branch join waits)
    const float sref_ld = W.score[ra.par()][ra.base()];
    const int rows = fresh ? 1 : rows_ld;
    const float sref = fresh ? 0.0f : sref_ld;
    const int tmax = (ra.rmax() + kTileRows - 1) / kTileRows;
    const bool fin = finishes(T, F, ra);
    // a finishing request: every row's back-pointers of all levels are loaded at once
    // (ahead of the counts) and stored in LDS, where the beams' codes are walked later
    const bool fin_lds = fin && Hs != nullptr && ra.rmax() <= kThreads;
    constexpr int kH = TCB_MAX_L - 1;
    uint32_t hh[kH];
    if (fin_lds && tid < ra.rmax()) {
#pragma unroll
        for (int t = 0; t < kH; ++t)
            if (t < ra.level()) hh[t] = W.hist[(size_t)t * W.S + ra.base() + tid];
    }

    // 1. request-wide cumulative kept counts and the boundary bin b*
    const int ntile = (rows + kTileRows - 1) / kTileRows;
    uint32_t g = 0u;
    uint32_t a8[8];                                   // this bin's counts of tiles 0..7
    for (int jt = 0; jt < tmax; jt += 8) {
        uint32_t a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] = (jt + u < tmax) ? tc[(size_t)(jt + u) * kBins + tid] : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            a[u] = (jt + u < ntile) ? a[u] : 0u;
            g += a[u];
            if (jt == 0) a8[u] = a[u];
        }
    }
    M.G[tid] = g;
    M.cur[tid] = 0u;
    trace_mark(W, 8);                                 // the counts have arrived
    if (fin_lds && tid < ra.rmax()) {
#pragma unroll
        for (int t = 0; t < kH; ++t)
            if (t < ra.level()) Hs[t][tid] = hh[t];
    }
    if (tid == 0) {
        M.bstar = kBins - 1;
        M.cnt = 0u;
        M.toff[0] = 0u;
    }
    __syncthreads();
    const uint32_t Ktot = M.G[kBins - 1];
    const uint32_t k = min((uint32_t)ra.width(), Ktot);
    // the bin of the request's k-th candidate; the thread holding it also knows how many
    // entries of each tile are staged (tcum_j[b*]) when the request has at most 8 tiles
    if (g >= k && (tid == 0 || M.G[tid - 1] < k)) {
        M.bstar = (uint32_t)tid;
        if (ntile <= 8) {
            uint32_t acc = 0u;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                acc += a8[u];
                if (u < ntile) M.toff[u + 1] = acc;
            }
        }
    }
    __syncthreads();
    const uint32_t bs = M.bstar;
    const uint32_t staged = M.G[bs];
    if (ntile > 8) {                                  // more tiles: read tcum_j[b*] again
        if (tid < 64) {
            const uint32_t c = tid < ntile ? (uint32_t)tc[(size_t)tid * kBins + bs] : 0u;
            const uint32_t incl = wave_incl_scan(c);
            if (tid < ntile) M.toff[tid + 1] = incl;
        }
        __syncthreads();
    }

    auto tile_of = [&](uint32_t p) {                  // largest tile j with toff[j] <= p
        int lo = 0, hi = ntile - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (M.toff[mid] <= p) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };
    auto cand_index = [&](uint32_t p) {
        const int jt = tile_of(p);
        return reg0 + (size_t)jt * CAPT + (p - M.toff[jt]);
    };


    if (staged <= (uint32_t)kMergeCap) {
        // 2. stage bins <= b* grouped by bin (each tile's first tcum_j[b*] entries)
        constexpr int U = kMergeCap / kThreads;
        float sc[U], ph[U];
        uint32_t fl[U], pos[U];
        int32_t nd[U];
        int32_t it[U];                                // finishing request: the candidates' catalog items
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t p = (uint32_t)(tid + u * kThreads);
            nd[u] = 0;
            if (p < staged) {
                const Cand c = W.cand[cpar][cand_index(p)];
                sc[u] = c.s;
                fl[u] = c.f;
                nd[u] = c.n;
                ph[u] = c.phi;
            }
        }
        uint32_t leafm = 0u;                          // bit u: entry u's node is a depth-L node
        if (fin_lds) {
            // issued now, used after the ranking; unconditional (a non-leaf reads item 0), so
            // that no branch join makes the binning below wait for them
            const uint32_t leaf0 = T.off[T.L], nleaf = T.off[T.L + 1] - leaf0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t p = (uint32_t)(tid + u * kThreads);
                const uint32_t li = (uint32_t)nd[u] - leaf0;
                const bool leaf = p < staged && li < nleaf;
                leafm |= (leaf ? 1u : 0u) << u;
                it[u] = T.leaf_item[leaf ? li : 0u];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t p = (uint32_t)(tid + u * kThreads);
            pos[u] = 0u;
            if (p < staged) {
                const uint32_t b = score_bin(sref, sc[u]);
                pos[u] = (b ? M.G[b - 1] : 0u) + atomicAdd(&M.cur[b], 1u);
                if (b <= bs && pos[u] < staged) {     // holds by construction
                    M.s[pos[u]] = sc[u];
                    M.f[pos[u]] = fl[u];
                    M.key[pos[u]] = merge_key(sc[u], fl[u]);
                    M.n[pos[u]] = nd[u];
                    M.phi[pos[u]] = ph[u];
                } else {
                    atomicOr(W.err, kErrInternal);
                    pos[u] = staged;
                }
            }
        }
        __syncthreads();
        trace_mark(W, 9);                             // staged
        // 3. rank = members of better bins + better members of the own bin
        if (fin_lds) {
            // each entry's rank goes to LDS (over its node id, which its staging thread
            // holds), and the staging thread writes the row: it holds the item loaded above
            rank_staged(M, M.G, staged, sref, [&](uint32_t rank, uint32_t p, float, uint32_t) {
                M.n[p] = (int32_t)rank;
            });
            __syncthreads();
            trace_mark(W, 11);                        // ranked (k_merge)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t p = (uint32_t)(tid + u * kThreads);
                if (p < staged && pos[u] < staged) {
                    const uint32_t rank = (uint32_t)M.n[pos[u]];
                    if (rank < k) {
                        uint64_t pfx = 0;
                        uint32_t r = fl[u] >> 8;
                        for (int t = ra.level() - 1; t >= 0; --t) {
                            if (r >= (uint32_t)ra.rmax()) {   // rows of every depth are below rmax
                                atomicOr(W.err, kErrBadNode);
                                break;
                            }
                            const uint32_t h = Hs[t][r];
                            pfx |= (uint64_t)(h & 255u) << (8 * t);
                            r = h >> 8;
                        }
                        const bool leaf = (leafm >> u) & 1u;
                        if (!leaf && !(W.norm == TCB_NORM_OPEN && nd[u] == -1)) atomicOr(W.err, kErrBadNode);
                        int32_t item = it[u];
                        asm volatile("" : "+v"(item));   // keeps its widening (and the wait) here
                        write_final_row(F, T.L, W.Bmax, q, rank, pfx, fl[u] & 255u, ph[u],
                                        leaf ? (int64_t)item : (int64_t)-1);
                    }
                }
            }
        } else if (fin) {
            rank_staged(M, M.G, staged, sref, [&](uint32_t rank, uint32_t p, float s, uint32_t f) {
                if (rank < k) write_finished_row(T, W, F, q, ra, rank, s, f, M.n[p], M.phi[p]);
            });
        } else {
            rank_staged(M, M.G, staged, sref, [&](uint32_t rank, uint32_t p, float s, uint32_t f) {
                if (rank < k) out.row(rank, s, f, M.n[p], M.phi[p]);
            });
        }
    } else {
        // exact path (massive ties around b*): select the k-th key over the tiles'
        // buffers, gather exactly k survivors, rank them by counting
        if (tid == 0) atomicOr(W.err, kInfoMergeSpill);
        auto each = [&](auto fn) {
            for (uint32_t p = tid; p < staged; p += kThreads) {
                const Cand c = W.cand[cpar][cand_index(p)];
                fn(f2ord(c.s), c.f);
            }
        };
        uint32_t o_star, f_star;
        block_select<kThreads>(each, k, sel, o_star, f_star, W.err);
        for (uint32_t p = tid; p < staged; p += kThreads) {
            const Cand c = W.cand[cpar][cand_index(p)];
            if (key_le(f2ord(c.s), c.f, o_star, f_star)) {
                const uint32_t pos = atomicAdd(&M.cnt, 1u);
                if (pos < (uint32_t)kMergeCap) {
                    M.s[pos] = c.s;
                    M.f[pos] = c.f;
                    M.n[pos] = c.n;
                    M.phi[pos] = c.phi;
                }
            }
        }
        __syncthreads();
        const uint32_t n = min(M.cnt, (uint32_t)kMergeCap);
        if (tid == 0 && M.cnt != k) atomicOr(W.err, kErrInternal);
        for (uint32_t p = tid; p < n; p += kThreads) {
            const uint32_t o = f2ord(M.s[p]), f = M.f[p];
            uint32_t r = 0u;
            for (uint32_t qq = 0; qq < n; ++qq) r += key_better(f2ord(M.s[qq]), M.f[qq], o, f) ? 1u : 0u;
            if (fin) write_finished_row(T, W, F, q, ra, r, M.s[p], f, M.n[p], M.phi[p]);
            else out.row(r, M.s[p], f, M.n[p], M.phi[p]);
        }
    }
    if (fin) finish_request(T, W, F, q, ra, rp, rows, k);
    else out.done(k);
    trace_mark(W, 10);                                // ranked, rows issued
}

// Where k_merge puts a request's new rows: the row buffers and the next record.
struct RowsToMemory {
    const WaveDev &W;
    ReqArg ra;
    int q, rp;
    __device__ void row(uint32_t rank, float s, uint32_t f, int32_t n, float phi) const {
        write_new_row(W, ra, rank, s, f, n, phi);
    }
    __device__ void done(uint32_t k) const { write_next_record(W, q, ra, rp, k); }
};

// Rows of one tile of the next step, taken from the previous step's merge (FuseRows), with
// their child sets when the window merge has loaded them (info true).
struct FuseRows {
    int32_t node[kTileRows];
    float score[kTileRows], phi[kTileRows];
    RowInfo ri[kTileRows];
    float sref;                                       // the best new row's key
    uint32_t info;                                    // ri holds the rows' child sets
    // window merge: per source tile, its first staged entry and the staged entries before it
    // (window bins), its entries of the first bin and their offsets
    uint32_t wst[kMaxTilesPerReq], woff[kMaxTilesPerReq + 1];
    uint32_t wfirst[kMaxTilesPerReq], foff[kMaxTilesPerReq + 1];
    uint32_t blo, bhi, bfirst, nfirst, glo, k;
};

// The previous step's merge inside a tile of the next step: every tile of the request
// merges, writes the rows of its own window [64 tile, 64 tile + 64) to the row buffers and
// keeps them in LDS; tile 0 writes the record.
struct RowsToTile {
    const WaveDev &W;
    ReqArg ra;                                        // the request at the merged step
    int q, rp, tile;
    FuseRows &Z;
    uint32_t &k_out;
    __device__ void row(uint32_t rank, float s, uint32_t f, int32_t n, float phi) const {
        const uint32_t i = rank - (uint32_t)(tile * kTileRows);
        if (i < (uint32_t)kTileRows) {
            Z.node[i] = n;
            Z.score[i] = s;
            Z.phi[i] = phi;
            write_new_row(W, ra, rank, s, f, n, phi);
        }
        if (rank == 0u) Z.sref = s;
    }
    __device__ void done(uint32_t k) const {
        k_out = k;
        if (tile == 0) write_next_record(W, q, ra, rp, k);
    }
};


// The child set of internal node `n` at depth `level` (RowInfo): its child range and, at
// depths stored with masks, its mask (elsewhere the mask of row 0 is read and ignored: the
// image always holds one). Unconditional loads only, so no branch join waits for them.
__device__ __forceinline__ RowInfo load_row_info(const TrieDev &T, uint32_t n, int level) {
    RowInfo ri;
    ri.cb = T.child_begin[n];
    ri.ce = T.child_begin[n + 1];
    const bool dense = level < T.mask_depths;
    const uint4 *m = reinterpret_cast<const uint4 *>(T.mask + (size_t)(dense ? n : 0u) * 8);
    const uint4 a = m[0], b = m[1];
    ri.mask[0] = a.x; ri.mask[1] = a.y; ri.mask[2] = a.z; ri.mask[3] = a.w;
    ri.mask[4] = b.x; ri.mask[5] = b.y; ri.mask[6] = b.z; ri.mask[7] = b.w;
    ri.pad[0] = ri.pad[1] = 0u;
    return ri;
}

// The previous step's merge inside tile `tile` of the next step, for this tile's rows only:
// the rows of ranks [64 tile, 64 tile + 64) lie in the score bins b_lo .. b_hi, so only the
// candidates of those bins are staged (plus those of the request's first non-empty bin, for
// the best row's key). Staged entries are grouped by bin in LDS (a bin's group starts at the
// kept entries of the window's better bins), and an entry's rank is the kept entries of
// better bins plus the better entries of its own bin. The child sets of the staged
// candidates are loaded while they are ranked. Rows go to Z and to the row buffers; tile 0
// writes the request's record. Returns false (nothing written) when the window would stage
// more than kWinCap entries (massive ties); the caller then merges the whole request.
// pa: the request as its previous step saw it; rpp: the record buffer that step read.
// issue(): called once where this tile has rows (right after the counts have arrived): the
// caller's own loads go there, behind the counts and ahead of the candidates, since a wait
// for a load also waits for every load issued before it (the candidates are waited on
// about when the caller's loads would have arrived anyway).
template <class Issue>
__device__ __forceinline__ bool window_merge(const TrieDev &T, const WaveDev &W, int q, const ReqArg pa, int rpp,
                                             int tile, MergeSmem &M, FuseRows &Z, Issue issue) {
    const int tid = threadIdx.x;
    const int MT = W.MT, CAPT = W.CAPT;
    const int cpar = pa.level() & 1;                  // the buffers the previous step's tiles wrote
    const uint16_t *tc = W.tcum[cpar] + (size_t)q * MT * kBins;
    const size_t reg0 = (size_t)q * MT * CAPT;
    const bool fresh = pa.level() == 0;
    const int tmax = (pa.rmax() + kTileRows - 1) / kTileRows;
    // 1. request-wide cumulative counts (thread = bin); the first 8 tiles' own counts stay
    //    in registers for the staging ranges. Every load of this phase is issued at once and
    //    unconditionally (indices clamped to the request's tiles), values dropped after
    const int rows_ld = W.rec[rpp][q].rows;
    const float sref_ld = W.score[pa.par()][pa.base()];
    uint32_t a8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a8[u] = tc[(size_t)min(u, tmax - 1) * kBins + tid];
    if (tid == 0) Z.info = 0u;
    const int rows = fresh ? 1 : rows_ld;
    const float sref = fresh ? 0.0f : sref_ld;
    const int ntile = min((rows + kTileRows - 1) / kTileRows, tmax);
    uint32_t g = 0u;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        a8[u] = u < ntile ? a8[u] : 0u;
        g += a8[u];
    }
    for (int jt = 8; jt < ntile; ++jt) g += tc[(size_t)jt * kBins + tid];   // beams wider than 512
    auto tile_count = [&](int jt) {                   // this bin's cumulative count in tile jt
        return jt < 8 ? a8[jt & 7] : (uint32_t)tc[(size_t)jt * kBins + tid];
    };
    M.G[tid] = g;
    M.cur[tid] = 0u;                                  // per-bin cursors of the grouping
    trace_mark(W, 8);                                 // the counts have arrived
    __syncthreads();
    const uint32_t Ktot = M.G[kBins - 1];
    const uint32_t k = min((uint32_t)pa.width(), Ktot);
    const uint32_t lo = (uint32_t)(tile * kTileRows);
    if (lo >= k) {                                    // no row of this tile survives (never tile 0: k >= 1)
        if (tile == 0) write_next_record(W, q, pa, rpp, k);
        if (tid == 0) Z.k = k;
        return true;
    }
    issue();
    const uint32_t hi = min(lo + (uint32_t)kTileRows, k) - 1u;
    const uint32_t gprev = tid ? M.G[tid - 1] : 0u;
    const uint32_t gnext = tid + 1 < kBins ? M.G[tid + 1] : 0xFFFFFFFFu;
    // each bin's thread finds its roles at once: the bins holding ranks lo (b_lo) and hi
    // (b_hi), the bin before b_lo, and the first non-empty bin; per source tile they record
    // the tile's own cumulative counts there (the window is [count at b_lo - 1, count at
    // b_hi) of each tile; the first bin's entries are the first ones of each tile)
    if (gprev <= lo && lo < g) {
        Z.blo = (uint32_t)tid;
        Z.glo = gprev;
    }
    // (the first 8 tiles' counts from registers, unrolled; wider beams read the rest again)
    auto put = [&](uint32_t *dst) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (u < ntile) dst[u] = a8[u];
        for (int jt = 8; jt < ntile; ++jt) dst[jt] = tile_count(jt);
    };
    if (gprev <= hi && hi < g) {
        Z.bhi = (uint32_t)tid;
        put(Z.woff + 1);                              // end offsets, turned into lengths below
    }
    if (g <= lo && lo < gnext) put(Z.wst);
    if (lo < M.G[0] && tid < ntile) Z.wst[tid] = 0u;  // b_lo = 0
    if (gprev == 0u && g > 0u) {
        Z.bfirst = (uint32_t)tid;
        Z.nfirst = g;
        put(Z.wfirst);
    }
    __syncthreads();
    trace_mark(W, 11);                                // window bins found
    const uint32_t blo = Z.blo, bfirst = Z.bfirst, glo = Z.glo;
    if (tid < 64) {                                   // lengths -> exclusive offsets (one wave)
        const uint32_t len = tid < ntile ? Z.woff[tid + 1] - Z.wst[tid] : 0u;
        const uint32_t incl = wave_incl_scan(len);
        const uint32_t flen = tid < ntile ? Z.wfirst[tid] : 0u;
        const uint32_t fincl = wave_incl_scan(flen);
        if (tid < ntile) {
            Z.woff[tid + 1] = incl;
            Z.foff[tid + 1] = fincl;
        }
        if (tid == 0) {
            Z.woff[0] = 0u;
            Z.foff[0] = 0u;
        }
    }
    __syncthreads();
    trace_mark(W, 12);                                // staging offsets
    const uint32_t nwin = Z.woff[ntile];
    const uint32_t nfirst = bfirst < blo ? Z.nfirst : 0u;   // first-bin entries staged after the window
    const uint32_t nst = nwin + nfirst;               // >= 1: rank lo lies in the window
    // 2. stage: entry p < nwin from the window, then the first bin's entries of every tile
    //    (they lie at the start of each tile's region). The load is issued by every thread
    //    (index clamped into the staged range), so the caller's loads follow it at one point
    const bool staged = (uint32_t)tid < nst;
    const uint32_t p = min((uint32_t)tid, nst - 1u);
    const bool inwin = p < nwin;
    const uint32_t pp = inwin ? p : p - nwin;
    int jw = 0, jf = 0;                               // the source tile of entry p
#pragma unroll
    for (int u = 1; u < 8; ++u) {
        jw += (u < ntile && Z.woff[u] <= pp) ? 1 : 0;
        jf += (u < ntile && Z.foff[u] <= pp) ? 1 : 0;
    }
    for (int u = 8; u < ntile; ++u) {
        jw += Z.woff[u] <= pp ? 1 : 0;
        jf += Z.foff[u] <= pp ? 1 : 0;
    }
    const int jt = inwin ? jw : jf;
    const uint32_t at = inwin ? Z.wst[jw] + (pp - Z.woff[jw]) : pp - Z.foff[jf];
    const Cand c = W.cand[cpar][reg0 + (size_t)jt * CAPT + min(at, (uint32_t)CAPT - 1u)];
    if (nst > (uint32_t)kWinCap) return false;
    // the candidate's child set, loaded now and used only if the entry is one of this
    // tile's rows; loaded unconditionally (another node of the depth stands in for a
    // candidate off the depth), so that no branch join makes the staging below wait for it
    const int level = pa.level() + 1;
    const bool want = inwin && (uint32_t)c.n >= T.off[level] && (uint32_t)c.n < T.off[level + 1];
    RowInfo ri = load_row_info(T, want ? (uint32_t)c.n : T.off[level], level);
    const uint32_t b = score_bin(sref, c.s);
    // grouped by bin: bin b's entries start after the window's entries of better bins
    uint64_t *gk = reinterpret_cast<uint64_t *>(M.n);
    const uint64_t key = ((uint64_t)f2ord(c.s) << 32) | (uint64_t)(~c.f);   // larger: better
    const uint32_t gb = b ? M.G[b - 1] : 0u;          // kept entries of better bins
    uint32_t st = 0u, en = 0u;
    if (staged) {
        st = inwin ? gb - glo : nwin;
        en = inwin ? M.G[b] - glo : nwin + nfirst;
        gk[st + atomicAdd(&M.cur[b], 1u)] = key;
    }
    trace_mark(W, 13);                                // thread 0's candidate arrived and grouped
    __syncthreads();
    trace_mark(W, 9);                                 // staged
    // 3. ranks
    if (staged) {
        uint32_t r = gb;
        uint32_t i = st;
        for (; i + 4u <= en; i += 4u)
            r += (gk[i] > key ? 1u : 0u) + (gk[i + 1] > key ? 1u : 0u) + (gk[i + 2] > key ? 1u : 0u) +
                 (gk[i + 3] > key ? 1u : 0u);
        for (; i < en; ++i) r += gk[i] > key ? 1u : 0u;
        if (r == 0u) Z.sref = c.s;
        if (inwin && r >= lo && r <= hi) {
            const uint32_t w = r - lo;
            Z.node[w] = c.n;
            Z.score[w] = c.s;
            Z.phi[w] = c.phi;
            if (want) Z.ri[w] = ri;
            else Z.ri[w] = RowInfo{};
            write_new_row(W, pa, r, c.s, c.f, c.n, c.phi);
        }
    }
    if (tile == 0) write_next_record(W, q, pa, rpp, k);
    if (tid == 0) {
        Z.k = k;
        Z.info = 1u;
    }
    trace_mark(W, 10);                                // ranked, rows issued
    return true;
}

// ---------------------------------------------------------------------- tile kernel
// Per tile of 64 rows: masked log-softmax, then a superset of the tile's top-n.
//   rows  lane j of a row's 16-lane group takes 16 of its codes and their bits of the
//         row's 256-bit child mask (read from the trie's per-node masks, or built in LDS
//         from the CSR child list at depths that have none: both give the same bits).
//   pick  1. prefilter (at depths whose nodes have many children on average; elsewhere
//            every candidate goes to step 2): the best candidate of each lane is one
//            sample; the bin b_L where the samples' count reaches n bounds the tile's
//            n-th best from below, so a candidate in a bin > b_L cannot make the
//            request's top-n either. b_L becomes a score threshold (with a margin far
//            above the rounding error), so the test costs one compare per candidate;
//         2. the survivors are binned exactly from registers (a wave skips an element
//            slot none of its lanes needs): the histogram atomics give every survivor its
//            place within its bin, the scan gives the bins' offsets, and the tile writes
//            every bin down to the one where its count reaches n (a superset of its
//            top-n) grouped by bin, with its cumulative bin counts.
//   If that keeps more than the tile's region holds (massive ties), an exact selection
//   over all candidates keeps exactly the tile's top-n instead.
struct TileSmem {
    uint32_t cmask[kWaves][kRowsPerWave][8];       // child masks built from CSR lists
    uint32_t h1[kBins];                            // bins of the lanes' best candidates
    uint32_t h2[kBins];                            // survivors' bins, then inclusive cumulative
    uint32_t p1[kWaves], p2[kWaves];               // wave totals of the two scans
    uint32_t bL, bt, tot, pad;
};

// inclusive scan over the 16 lanes of each DPP row
__device__ __forceinline__ uint32_t row16_incl_scan(uint32_t x) {
    x += dpp_u<0x111, 0xF>(x);   // row_shr:1
    x += dpp_u<0x112, 0xF>(x);   // row_shr:2
    x += dpp_u<0x114, 0xF>(x);   // row_shr:4
    x += dpp_u<0x118, 0xF>(x);   // row_shr:8
    return x;
}
__device__ __forceinline__ uint32_t row16_sum_u(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kQuadXor1, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kQuadXor2, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kHalfMirror, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kMirror, 0xF, 0xF, false);
    return v;
}
// Sum of the totals of waves 0..w-1 (part[] holds each wave's total; w is uniform).
__device__ __forceinline__ uint32_t waves_before(const uint32_t *part, int w) {
    const int lane = threadIdx.x & 63;
    uint32_t v = lane < kWaves ? part[lane] : 0u;
    v = row16_incl_scan(v);
    return w ? (uint32_t)__builtin_amdgcn_readlane((int)v, w - 1) : 0u;
}

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): one output for state x.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
// The uniform draw of child `code` of the beam at local rank `rank`:
// u = (hash >> 40 + 1/2) / 2^24 from a counter-based hash keyed by (seed, request,
// level, rank, code). u needs 25 significant bits, so it is formed in double (near
// u = 1 a float's rounding alone would move -log u by a relative 2^-24 / (1 - u)).
// The child's Gumbel noise is -log(-log u).
__device__ __forceinline__ double noise_uniform(uint64_t seed_hash, uint32_t q, uint32_t level, uint32_t rank,
                                                uint32_t code) {
    const uint64_t key = seed_hash ^ ((uint64_t)q << 40) ^ ((uint64_t)level << 32) ^ ((uint64_t)rank << 8) ^ code;
    return ((double)(splitmix64(key) >> 40) + 0.5) * (1.0 / 16777216.0);
}
// Key of a child whose perturbed score lies delta below its siblings' maximum z, the
// maximum being conditioned to equal the parent's key pk (stochastic beam search, Kool,
// van Hoof and Welling, ICML 2019):
//   key = -log(exp(-pk) - exp(-z) + exp(-(z - delta))) = pk - log1p(exp(pk - z) expm1(delta)),
// evaluated as pk - softplus(pk - z + log expm1(delta)). Near the maximum the key moves
// by about exp(pk - z) times delta, so delta is formed in float64 by the caller.
__device__ __forceinline__ float conditioned_key(float pk, float pk_minus_z, float delta) {
    if (!(delta > 0.0f)) return pk;                    // the maximum itself (and exact ties)
    const float lem = delta < 1.0f ? logf(expm1f(delta)) : delta + log1pf(-expf(-delta));
    const float w = pk_minus_z + lem;
    return pk - (fmaxf(w, 0.0f) + log1pf(expf(-fabsf(w))));
}
__device__ __forceinline__ double row16_max_d(double v) {
    auto step = [](double a, auto dpp) {
        const uint64_t u = __builtin_bit_cast(uint64_t, a);
        const uint32_t lo = (uint32_t)dpp((int)(uint32_t)u), hi = (uint32_t)dpp((int)(uint32_t)(u >> 32));
        return fmax(a, __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo));
    };
    v = step(v, [](int x) { return __builtin_amdgcn_update_dpp(0, x, kQuadXor1, 0xF, 0xF, false); });
    v = step(v, [](int x) { return __builtin_amdgcn_update_dpp(0, x, kQuadXor2, 0xF, 0xF, false); });
    v = step(v, [](int x) { return __builtin_amdgcn_update_dpp(0, x, kHalfMirror, 0xF, 0xF, false); });
    v = step(v, [](int x) { return __builtin_amdgcn_update_dpp(0, x, kMirror, 0xF, 0xF, false); });
    return v;
}

// log-sum-exp of a row from its maximum and its sum of exp(x - max)
__device__ __forceinline__ float row_lse(float mx, float sum) {
    return mx + __builtin_amdgcn_logf(sum) * kLn2;
}

// Masked log-softmax (sampled steps: of x / T) of one row held by a 16-lane group (lane j
// holds the elements e of codes code_of(e, j)) and the keys of its candidates: codes
// outside the support count as -inf. valid: this lane's candidates; ok: the row's node is
// valid (the LEVEL support is every code of a valid row). On return x[e] is candidate e's
// key (-inf off the candidates), ph[e] its log-probability (sampled steps) and lbest the
// lane's best key. The 16 lanes of the group call it together (DPP reductions).
template <int DT, int NORM, bool SAMPLE>
__device__ __forceinline__ void score_row(const StepReqs &R, int q, int level, int r, int j, int V, bool ok,
                                          uint32_t valid, float sr, float pr, float (&x)[kElems],
                                          float (&ph)[SAMPLE ? kElems : 1], float &lbest) {
    float lse = 0.0f;
    uint32_t sup = valid;
    if constexpr (NORM == TCB_NORM_LEVEL) {
        sup = 0u;
#pragma unroll
        for (int e = 0; e < kElems; ++e) sup |= (ok && code_of<DT>(e, j) < V) ? (1u << e) : 0u;
    }
    if constexpr (!SAMPLE) {
#pragma unroll
        for (int e = 0; e < kElems; ++e) x[e] = ((sup >> e) & 1u) ? x[e] : -INFINITY;
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < kElems; ++e) mx = fmaxf(mx, x[e]);
        float lm = mx;                            // this lane's best candidate logit
        if constexpr (NORM == TCB_NORM_LEVEL) {
            lm = -INFINITY;
#pragma unroll
            for (int e = 0; e < kElems; ++e) lm = fmaxf(lm, ((valid >> e) & 1u) ? x[e] : -INFINITY);
        }
        mx = row16_max(mx);
        const float mxl = mx * kLog2e;
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < kElems; ++e) sum += __builtin_amdgcn_exp2f(fmaf(x[e], kLog2e, -mxl));
        lse = row_lse(mx, row16_sum(sum));
        lbest = sr + (lm - lse);
        // from here on x[e] is the candidate's score (-inf off the child set)
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            float sc = sr + (x[e] - lse);
            if constexpr (NORM == TCB_NORM_LEVEL) sc = ((valid >> e) & 1u) ? sc : -INFINITY;
            x[e] = sc;
        }
    } else {
        // the same log-softmax of x / T, leaving x unscaled
        const float it = R.inv_temp;
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < kElems; ++e) mx = fmaxf(mx, ((sup >> e) & 1u) ? x[e] * it : -INFINITY);
        mx = row16_max(mx);
        const float mxl = mx * kLog2e;
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < kElems; ++e)
            sum += __builtin_amdgcn_exp2f(fmaf(((sup >> e) & 1u) ? x[e] * it : -INFINITY, kLog2e, -mxl));
        sum = row16_sum(sum);
        lse = mx + __builtin_amdgcn_logf(sum) * kLn2;
        // Gumbel top-k without replacement over SIDs (stochastic beam search): child c
        // draws g_c = phi_c + Gumbel noise = (pr - lse) + t_c, t_c = x_c / T + Gumbel;
        // its key is g_c conditioned on the siblings' maximum z equalling the row's key.
        // t_c and the gap t* - t_c are formed in float64 from the unscaled logit.
        // From here on x[e] is the child's key.
        const uint64_t sh = splitmix64(R.seed);
        auto t_of = [&](int e) -> double {
            const double u = noise_uniform(sh, (uint32_t)q, (uint32_t)level, (uint32_t)r,
                                           (uint32_t)code_of<DT>(e, j));
            return (double)x[e] * R.inv_temp_d - log(-log(u));
        };
        double tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            ph[e] = pr + (x[e] * it - lse);
            if ((valid >> e) & 1u) tmax = fmax(tmax, t_of(e));
        }
        tmax = row16_max_d(tmax);
        const float pz = (float)((double)sr - (double)pr + (double)lse - tmax);   // pk - z
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            float key = -INFINITY;
            if ((valid >> e) & 1u) key = conditioned_key(sr, pz, (float)(tmax - t_of(e)));
            x[e] = key;
            lbest = fmaxf(lbest, key);
        }
    }
}

// The work of one tile (request ql of the launch, tile `tile`); it returns early where the
// tile has nothing to do (every return is uniform over the workgroup). With MERGE (the
// request's only tile) the kept candidates go to LDS and the tile ranks them and writes
// the request's new rows itself, returning true; it returns false where k_merge's work
// (from the records in memory) is still to do.
// With FUSE, a request whose previous step left its merge pending does that merge first
// (M and Z: its staging and this tile's rows).
// HEAD: an lm_head step; requests with the sparse-head flag get their rows' children's
// logits from head_children (after the child sets are known) instead of from `logits`.
template <int DT, int NORM, bool VEC, bool SAMPLE, bool MERGE, bool FUSE, bool HEAD = false>
__device__ __forceinline__ bool tile_work(const TrieDev &T, const WaveDev &W, int rp, const StepReqs &R,
                                          const void *__restrict__ logits, int64_t ld, int ql, int tile,
                                          TileSmem &A, SelSmem &sel, MergeSmem *M, FuseRows *Z) {
    constexpr int CH = Lay<DT>::CH, CW = Lay<DT>::CW, SPAN = 256 / CH;
    static_assert(CH * CW == kElems && (SPAN / CW) * 8 <= 256, "row layout");
    static_assert(!HEAD || (VEC && !SAMPLE && NORM == TCB_NORM_CHILDREN), "in-tile head: children, 16-byte rows");

    const int tid = threadIdx.x;
    const int MT = W.MT;
    const int q = R.q0 + ql;
    const ReqArg ra = R.r[ql];
    if (!ra.step()) {
        if (tile == 0 && tid == 0) W.rec[rp ^ 1][q] = W.rec[rp][q];   // not stepped: carried over
        return false;
    }
    if (tile * kTileRows >= ra.rmax()) return false;          // past any row the request can have

    trace_mark(W, 0);
    trace_mark(W, 1);                                 // started
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 4, j = lane & 15;
    const int level = ra.level(), cp = ra.par(), base = ra.base();
    const int rt = wave * kRowsPerWave + g;                   // row within the tile
    const int r = tile * kTileRows + rt;                       // local rank in the request
    const int V = T.V;
    const uint32_t width = (uint32_t)ra.width();
    A.h1[tid] = 0u;
    A.h2[tid] = 0u;
    if (tid == 0) {
        A.bL = kBins - 1;
        A.bt = kBins - 1;
        A.tot = 0u;
    }

    // 1. row state and logits, all issued at once: the live-row count arrives with the
    //    rows, which are read for every row the request can have and dropped if dead. A
    //    request's first step starts from its initial state (one row: the root, score 0),
    //    which is not read back, so the step needs no earlier initialising kernel
    const bool fresh = level == 0;
    const bool in_range = r < ra.rmax();
    int32_t nd = -1;
    float sr = 0.0f, pr = 0.0f;                        // the row's key and (sampled) log-probability
    float x[kElems];
#pragma unroll
    for (int e = 0; e < kElems; ++e) x[e] = 0.0f;
    // lm_head rows whose children's logits this tile computes (none are read)
    const bool head_rows = HEAD && ra.sparse_head();
    // at depths with few children per row the logits wait for the trie and only the
    // 16-byte pieces holding a child are read (the rest is masked off either way)
    const bool gather = VEC && ra.gather() && !head_rows;
    // the row's logits, unless they wait for the trie (gather): issued unconditionally with
    // 16-byte pieces (a row past the request's bound reads its last possible row, dropped)
    const int slot_c = base + min(r, ra.rmax() - 1);
    RawRow<DT> raw;
    auto issue_logits = [&]() {
        if constexpr (VEC) {
            if (!head_rows) {
                // the empty asm pins the loads here: their address would otherwise let the
                // compiler hoist them to the kernel's start, ahead of the merge's loads
                int sl = slot_c;
                asm volatile("" : "+v"(sl));
                load_row_raw<DT>(logits, ld, sl, j, raw);
            }
        }
    };
    // a step that first does the previous merge issues them behind the merge's loads, with
    // no branch around them (such a step never gathers: its rows' nodes come from the merge)
    if (!(FUSE && ra.pending()) && !gather) issue_logits();
    int rows;
    float sref;                                       // best row of the request
    // the row's child set, where it came with the row (from the previous step's merge in
    // this kernel, or stored by a first step): this lane's mask words and the child range
    const bool dense_depth = level < T.mask_depths;
    bool have_info = false;
    uint32_t mw[CH], icb = 0u, ice = 0u;
#pragma unroll
    for (int i = 0; i < CH; ++i) mw[i] = 0u;
    if (FUSE && ra.pending()) {
        // the previous step's merge: a row's logits do not depend on it (they are indexed
        // by slot), so they were issued first; the row state then comes from the merge
        if (!VEC && in_range) load_row<DT, VEC>(logits, ld, base + r, j, V, x);
        const ReqArg pa = ra.prev_step();
        if (!window_merge(T, W, q, pa, rp ^ 1, tile, *M, *Z, issue_logits)) {
            uint32_t k = 0u;
            merge_request(T, W, StepFin{}, q, pa, rp ^ 1, *M, sel, nullptr, RowsToTile{W, pa, q, rp ^ 1, tile, *Z, k});
            if (tid == 0) Z->k = k;
        }
        __syncthreads();
        trace_mark(W, 2);                             // previous merge done
        rows = (int)Z->k;
        sref = Z->sref;
        have_info = Z->info != 0u;
        if (r < rows) {
            nd = Z->node[rt];
            sr = Z->score[rt];
            if constexpr (SAMPLE) pr = Z->phi[rt];
            if (have_info) {
#pragma unroll
                for (int i = 0; i < CH; ++i) mw[i] = Z->ri[rt].mask[(i * SPAN + j * CW) >> 5];
                icb = Z->ri[rt].cb;
                ice = Z->ri[rt].ce;
            }
        }
    } else {
        // the row state, loaded unconditionally with the logits (a fresh request's first step
        // uses its known initial state instead; rows past the bound are dropped)
        const int rows_ld = W.rec[rp][q].rows;
        const float sref_ld = W.score[cp][base];
        const int32_t nd_ld = W.node[cp][slot_c];
        const float sr_ld = W.score[cp][slot_c];
        float pr_ld = 0.0f;
        if constexpr (SAMPLE) pr_ld = W.phi[cp][slot_c];
        have_info = ra.rows_info();
        if (have_info) {
            const RowInfo *ri = W.rinfo + slot_c;
            if (dense_depth) {
#pragma unroll
                for (int i = 0; i < CH; ++i) mw[i] = ri->mask[(i * SPAN + j * CW) >> 5];
            }
            icb = ri->cb;
            ice = ri->ce;
        }
        if (!VEC && in_range) load_row<DT, VEC>(logits, ld, slot_c, j, V, x);
        rows = fresh ? 1 : rows_ld;
        sref = fresh ? 0.0f : sref_ld;
        if (in_range) {
            nd = fresh ? 0 : nd_ld;
            sr = fresh ? 0.0f : sr_ld;
            if constexpr (SAMPLE) pr = fresh ? 0.0f : pr_ld;
        }
    }
    if (tile * kTileRows >= rows) return false;              // a tile with no live row
    const bool live = r < rows;
    const bool wave_live = tile * kTileRows + wave * kRowsPerWave < rows;

    // 2. the row's node: first child id and this lane's child bits (chunk i holds the
    //    CW codes i * SPAN + j * CW ...), from the child set that came with the row or
    //    from the trie
    const uint32_t lo_id = T.off[level], hi_id = T.off[level + 1];
    bool ok = false;
    uint32_t cb = 0u, ce = 0u;
    uint32_t bits[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) bits[i] = 0u;
    if (live) {
        const uint32_t n = (uint32_t)nd;
        if (n >= lo_id && n < hi_id) {
            ok = true;
            if (have_info) {
                cb = icb;
                ce = ice;
                if (dense_depth) {
#pragma unroll
                    for (int i = 0; i < CH; ++i) {
                        const int c0 = i * SPAN + j * CW;
                        bits[i] = (mw[i] >> (c0 & 31)) & ((1u << CW) - 1u);
                    }
                }
            } else {
                cb = T.child_begin[n];
                if (dense_depth) {
#pragma unroll
                    for (int i = 0; i < CH; ++i) {
                        const int c0 = i * SPAN + j * CW;
                        bits[i] = (T.mask[(size_t)n * 8 + (c0 >> 5)] >> (c0 & 31)) & ((1u << CW) - 1u);
                    }
                } else {
                    ce = T.child_begin[n + 1];
                }
            }
        } else if (j == 0 && !(NORM == TCB_NORM_OPEN && nd == -1)) {   // -1: off the catalog (open)
            atomicOr(W.err, kErrBadNode);
        }
    }
    if (!dense_depth && wave_live) {
        // no stored mask at this depth: build the row's 256-bit mask in LDS
        uint32_t *cm = A.cmask[wave][g];
        if (j < 8) cm[j] = 0u;
        wave_lds_sync();
        if (ok) {
            for (uint32_t a = (cb & ~3u) + 4u * (uint32_t)j; a < ce; a += 64u) {
                const uint32_t wv = *reinterpret_cast<const uint32_t *>(T.child_code + a);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t idx = a + (uint32_t)k;
                    if (idx >= cb && idx < ce) {
                        const uint32_t c = (wv >> (8 * k)) & 255u;
                        atomicOr(&cm[c >> 5], 1u << (c & 31));
                    }
                }
            }
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c0 = i * SPAN + j * CW;
            bits[i] = ok ? (cm[c0 >> 5] >> (c0 & 31)) & ((1u << CW) - 1u) : 0u;
        }
    }
    if constexpr (VEC) {
        if (!gather && !head_rows) widen_row<DT>(raw, x);   // the logits issued at the start
    }
    if constexpr (HEAD) {
        if (head_rows) {
            uint32_t kids = 0u;
#pragma unroll
            for (int i = 0; i < CH; ++i) kids |= bits[i] << (i * CW);
            head_children<DT>(R.hd, slot_c, level, g, j, kids, x);
        }
    }
    if (gather && live) {
        uint32_t chunks = 0u;
#pragma unroll
        for (int i = 0; i < CH; ++i) chunks |= (bits[i] != 0u ? 1u : 0u) << i;
        load_row_chunks<DT>(logits, ld, base + r, j, chunks, x);
    }
    if (W.validate && live) {
        bool bad = false;
#pragma unroll
        for (int e = 0; e < kElems; ++e)
            if (code_of<DT>(e, j) < V && !isfinite(x[e])) bad = true;
        if (bad) atomicOr(W.err, kErrNonFinite);
    }
    uint32_t tv = 0u;                                 // this lane's codes that are trie children
#pragma unroll
    for (int i = 0; i < CH; ++i) tv |= bits[i] << (i * CW);
    uint32_t valid = tv;                              // this lane's candidates
    if constexpr (NORM == TCB_NORM_OPEN) {            // no constraint: every code of a live row
        valid = 0u;
#pragma unroll
        for (int e = 0; e < kElems; ++e) valid |= (live && code_of<DT>(e, j) < V) ? (1u << e) : 0u;
    }

    // 3. masked log-softmax and the candidates' keys
    trace_mark(W, 14);                                // logits in registers, child bits known
    float lbest = -INFINITY;
    float ph[SAMPLE ? kElems : 1];                    // sampled steps: the candidates' log-probabilities
    if (wave_live) {
        score_row<DT, NORM, SAMPLE>(R, q, level, r, j, V, ok, valid, sr, pr, x, ph, lbest);
    } else {
#pragma unroll
        for (int e = 0; e < kElems; ++e) x[e] = -INFINITY;
    }

    // 4. prefilter (at depths with many children per row): histogram of the lanes' best
    //    candidates, bin b_L where it reaches n. Elsewhere every candidate is binned exactly.
    trace_mark(W, 15);                                // keys computed (wave 0)
    __syncthreads();                                  // the zeroed histograms are visible
    trace_mark(W, 3);                                 // rows loaded, trie read, log-softmax done
    uint32_t bL = kBins - 1;
    if (ra.prefilter()) {
        if (valid) atomicAdd(&A.h1[score_bin(sref, lbest)], 1u);
        __syncthreads();
        const uint32_t h = A.h1[tid];
        const uint32_t incl = wave_incl_scan(h);
        if (lane == 63) A.p1[wave] = incl;
        __syncthreads();
        const uint32_t C = waves_before(A.p1, wave) + incl;
        if (C >= width && C - h < width) A.bL = (uint32_t)tid;
        __syncthreads();
        bL = A.bL;
        trace_mark(W, 4);                             // prefilter bound
    }

    // 5.-6. survivors and their exact bins. A candidate in a bin <= b_L scores above
    //    ts = sref - (b_L + 1) / kBinRes less the bin arithmetic's rounding; the margin
    //    covers that many times over (extra survivors are binned exactly and cut at b_t).
    //    Each element slot is one branch the wave skips when none of its lanes needs it;
    //    all of a lane's atomics are issued before any result is used.
    uint32_t bn[kElems], wb[kElems];
#pragma unroll
    for (int e = 0; e < kElems; ++e) {
        bn[e] = kBins;                                // not a survivor
        wb[e] = 0u;
    }
    if (bL < (uint32_t)(kBins - 1)) {
        const float ts = sref - (float)(bL + 1u) * (1.0f / kBinRes);
        const float thr = ts - (1.0f / 65536.0f) * (1.0f + 2.0f * fabsf(sref) + fabsf(ts));
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            if (x[e] >= thr) {                        // -inf off the child set never passes
                const uint32_t b = score_bin(sref, x[e]);
                bn[e] = b;
                wb[e] = atomicAdd(&A.h2[b], 1u);
            }
        }
    } else {                                          // fewer samples than n: every candidate
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            if ((valid >> e) & 1u) {
                const uint32_t b = score_bin(sref, x[e]);
                bn[e] = b;
                wb[e] = atomicAdd(&A.h2[b], 1u);
            }
        }
    }
    __syncthreads();
    uint32_t C;
    {
        const uint32_t h = A.h2[tid];
        const uint32_t incl = wave_incl_scan(h);
        if (lane == 63) A.p2[wave] = incl;
        __syncthreads();
        C = waves_before(A.p2, wave) + incl;
        if (C >= width && C - h < width) A.bt = (uint32_t)tid;
        A.h2[tid] = C;                                // this thread's bin only
    }
    __syncthreads();
    trace_mark(W, 5);                                 // binned and scanned
    const uint32_t bt = A.bt;
    const uint32_t kept = A.h2[bt];
    const int CAPT = W.CAPT;
    const size_t reg = ((size_t)q * MT + tile) * (size_t)CAPT;

    // child node ids: byte i of rk holds the rank, among the row's children, of the
    // lane's first code in chunk i (a 16-lane scan of per-chunk child counts; every
    // partial sum stays below 256, so the bytes never carry); node(e) = first child id
    // + that rank + the lane's children in the chunk below element e
    uint32_t rk;
    {
        uint32_t pc = 0u;
#pragma unroll
        for (int i = 0; i < CH; ++i) pc |= (uint32_t)__popc(bits[i]) << (8 * i);
        const uint32_t excl = row16_incl_scan(pc) - pc;
        const uint32_t tot = row16_sum_u(pc);
        rk = excl + tot * 0x01010100u;               // byte i: children before chunk i
    }
    const uint32_t flat0 = (uint32_t)r * 256u + (uint32_t)j * CW;
    auto flat_of = [&](int e) -> uint32_t { return flat0 + (uint32_t)((e / CW) * SPAN + e % CW); };
    auto node_of = [&](int e) -> int32_t {
        const uint32_t below = tv & ((1u << e) - (1u << (e & ~(CW - 1))));
        const int32_t n = (int32_t)(cb + ((rk >> (8 * (e / CW))) & 255u) + (uint32_t)__popc(below));
        if constexpr (NORM == TCB_NORM_OPEN) return ((tv >> e) & 1u) ? n : -1;   // -1: off the catalog
        return n;
    };
    // fn(e) for every kept element (one branch per element slot, skipped by a wave with none)
    auto for_kept = [&](auto fn) {
#pragma unroll
        for (int e = 0; e < kElems; ++e)
            if (bn[e] <= bt) fn(e);
    };

    if (kept <= (uint32_t)CAPT) {
        // 7. write bins <= b_t grouped by bin (the bins' offsets are all read first)
        uint32_t at[kElems];
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            at[e] = 0u;
            if (bn[e] != 0u && bn[e] <= bt) at[e] = A.h2[bn[e] - 1];
        }
        if constexpr (MERGE) {
            // the request's only tile: its kept candidates are exactly what k_merge would
            // stage (A.h2 holds the request's cumulative kept counts, b* = b_t), so they are
            // staged in LDS, ranked and written here
            static_assert(kTileCap <= kMergeCap, "a tile's kept candidates fit the merge's staging");
            for_kept([&](int e) {
                const uint32_t dst = at[e] + wb[e];
                if (dst < kept) {
                    M->s[dst] = x[e];
                    M->f[dst] = flat_of(e);
                    M->key[dst] = merge_key(x[e], flat_of(e));
                    M->n[dst] = node_of(e);
                    if constexpr (SAMPLE) M->phi[dst] = ph[e];
                    else M->phi[dst] = x[e];
                } else {
                    atomicOr(W.err, kErrInternal);
                }
            });
            __syncthreads();
            trace_mark(W, 6);                         // staged for the in-tile merge
            const uint32_t k = min(width, kept);
            if (finishes(T, R.fin, ra)) {
                rank_staged(*M, A.h2, kept, sref, [&](uint32_t rank, uint32_t p, float s, uint32_t f) {
                    if (rank < k) write_finished_row(T, W, R.fin, q, ra, rank, s, f, M->n[p], M->phi[p]);
                });
                finish_request(T, W, R.fin, q, ra, rp, rows, k);
            } else {
                rank_staged(*M, A.h2, kept, sref, [&](uint32_t rank, uint32_t p, float s, uint32_t f) {
                    if (rank < k) write_new_row(W, ra, rank, s, f, M->n[p], M->phi[p]);
                });
                write_next_record(W, q, ra, rp, k);
            }
            trace_mark(W, 7);                         // ranked, rows issued
            return true;
        }
        Cand *out = W.cand[level & 1] + reg;
        for_kept([&](int e) {
            const uint32_t dst = at[e] + wb[e];
            if (dst < kept) {
                Cand c;
                c.s = x[e];
                c.f = flat_of(e);
                c.n = node_of(e);
                if constexpr (SAMPLE) c.phi = ph[e];
                else c.phi = x[e];
                out[dst] = c;
            } else {
                atomicOr(W.err, kErrInternal);
            }
        });
        W.tcum[level & 1][((size_t)q * MT + tile) * kBins + tid] = (uint16_t)min(C, kept);
        trace_mark(W, 7);                             // candidates issued
    } else {
        // exact path: keep exactly the tile's top min(n, #candidates)
        if (tid == 0) atomicOr(W.err, kInfoTileExact);
        const uint32_t total = block_incl_scan<kThreads>((uint32_t)__popc(valid), A.p1);
        if (tid == kThreads - 1) A.tot = total;
        A.h2[tid] = 0u;                               // every thread has read kept
        __syncthreads();
        const uint32_t kt = min(width, A.tot);
        // the selection gets copies (a reference to x or the lane's values would keep them
        // in memory on every path when it is not inlined)
        float xe[kElems];
#pragma unroll
        for (int e = 0; e < kElems; ++e) xe[e] = x[e];
        const uint32_t vc = valid, fc = flat0;
        auto each = [xe, vc, fc](auto fn) {
#pragma unroll
            for (int e = 0; e < kElems; ++e)
                if ((vc >> e) & 1u) fn(f2ord(xe[e]), fc + (uint32_t)((e / CW) * SPAN + e % CW));
        };
        uint32_t o_star, f_star;
        block_select<kThreads>(each, kt, sel, o_star, f_star, W.err);
        uint32_t keep = 0u;
#pragma unroll
        for (int e = 0; e < kElems; ++e)
            if (((valid >> e) & 1u) && key_le(f2ord(x[e]), flat_of(e), o_star, f_star))
                keep |= 1u << e;
        uint32_t wbe[kElems];
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            wbe[e] = 0u;
            if ((keep >> e) & 1u) wbe[e] = atomicAdd(&A.h2[score_bin(sref, x[e])], 1u);
        }
        __syncthreads();
        const uint32_t h = A.h2[tid];
        const uint32_t Cx = block_incl_scan<kThreads>(h, A.p1);
        A.h2[tid] = Cx;
        __syncthreads();
        const uint32_t kx = A.h2[kBins - 1];
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            if ((keep >> e) & 1u) {
                const float s = x[e];
                const uint32_t b = score_bin(sref, s);
                const uint32_t dst = (b ? A.h2[b - 1] : 0u) + wbe[e];
                if (dst < kx && dst < (uint32_t)CAPT) {
                    Cand c;
                    c.s = s;
                    c.f = flat_of(e);
                    c.n = node_of(e);
                    if constexpr (SAMPLE) c.phi = ph[e];
                    else c.phi = s;
                    W.cand[level & 1][reg + dst] = c;
                } else {
                    atomicOr(W.err, kErrInternal);
                }
            }
        }
        W.tcum[level & 1][((size_t)q * MT + tile) * kBins + tid] = (uint16_t)Cx;
    }
    return false;
}

// MERGE: every stepped request of the launch has at most kTileRows rows (one tile), so one
// workgroup per request does its tile and then, after a barrier, its merge from the
// records it has just written: no second kernel. Otherwise the tiles of a request are
// dealt to one XCD (workgroups b with the same b mod 8 run on one XCD) and k_merge follows.
// FUSE: requests whose previous merge is pending do it first, in every one of their tiles.
template <int DT, int NORM, bool VEC, bool SAMPLE, bool MERGE, bool FUSE, bool HEAD = false>
__global__ __launch_bounds__(kThreads) void k_tile(TrieDev T, WaveDev W, int rp, StepReqs R,
                                                   const void *__restrict__ logits, int64_t ld) {
    __shared__ TileSmem A;
    __shared__ SelSmem sel;
    if constexpr (MERGE) {
        __shared__ MergeSmem M;
        const int ql = (int)blockIdx.x;
        if (ql >= R.n) return;
        if (tile_work<DT, NORM, VEC, SAMPLE, true, false, HEAD>(T, W, rp, R, logits, ld, ql, 0, A, sel, &M, nullptr))
            return;
        const ReqArg ra = R.r[ql];
        if (!ra.step()) return;                        // carried over by tile_work
        __syncthreads();                               // the tile's records are visible to the workgroup
        merge_request(T, W, R.fin, R.q0 + ql, ra, rp, M, sel, nullptr,     // a tile with no live row, or the exact path
                      RowsToMemory{W, ra, R.q0 + ql, rp});
    } else {
        const int MT = W.MT;
        const int i8 = (int)(blockIdx.x >> 3);
        const int ql = (int)(blockIdx.x & 7u) + 8 * (i8 / MT);  // all tiles of a request on one XCD
        const int tile = i8 % MT;
        if (ql >= R.n) return;
        if constexpr (FUSE) {
            __shared__ MergeSmem M;
            __shared__ FuseRows Z;
            tile_work<DT, NORM, VEC, SAMPLE, false, true, HEAD>(T, W, rp, R, logits, ld, ql, tile, A, sel, &M, &Z);
        } else {
            tile_work<DT, NORM, VEC, SAMPLE, false, false, HEAD>(T, W, rp, R, logits, ld, ql, tile, A, sel, nullptr,
                                                                 nullptr);
        }
    }
}

// ---------------------------------------------------------------------- first step
// A launch whose stepped requests are all at their first step (one row: the root). One
// workgroup of 256 threads per request: lanes 0..15 score the root's row exactly as a tile
// does (same layout and arithmetic, so the rows equal the tile kernel's bit for bit);
// every candidate (at most V <= 256 children) is then ranked by counting the better keys
// in LDS, and the survivors are written in rank order. The root's children are the depth-1
// nodes, so their child sets do not depend on the logits: they are loaded at the start and
// stored with the new rows (WaveDev::rinfo), and the next step reads them with its rows
// instead of waiting on the trie.
struct alignas(16) FirstSmem {
    uint64_t gk[256];                               // candidates' keys grouped by score bin
    uint32_t ord[256];                              // key by code, order-preserving; 0: no candidate
    float key[256], phi[256];
    int32_t node[256];
    RowInfo kid[256];                               // child sets of the depth-1 nodes
    uint32_t bin0[kBins + 1];                       // bin counts, then each bin's first entry
    uint32_t part[4];
    uint32_t cm[8];                                 // the root's mask built from its child list
};

template <int DT, int NORM, bool VEC, bool SAMPLE>
__global__ __launch_bounds__(256) void k_first(TrieDev T, WaveDev W, int rp, StepReqs R,
                                               const void *__restrict__ logits, int64_t ld) {
    constexpr int CH = Lay<DT>::CH, CW = Lay<DT>::CW, SPAN = 256 / CH;
    __shared__ FirstSmem F;
    const int nx = first_xcds(R.n), xb = (int)((blockIdx.x + 7u) & 7u);
    if (xb >= nx) return;                             // a workgroup of a later XCD: nothing to do
    const int ql = (int)(blockIdx.x >> 3) * nx + xb;
    if (ql >= R.n) return;
    const int q = R.q0 + ql;
    const ReqArg ra = R.r[ql];
    const int tid = threadIdx.x;
    if (!ra.step()) {
        if (tid == 0) W.rec[rp ^ 1][q] = W.rec[rp][q];   // not stepped: carried over
        return;
    }
    trace_mark(W, 0);
    trace_mark(W, 1);                                 // started
    const int base = ra.base(), V = T.V, L = T.L;
    const bool fin = finishes(T, R.fin, ra);
    // the child sets of the depth-1 nodes, for the rows the next step will have
    const uint32_t n1 = T.off[1], nk = T.off[2] - T.off[1];
    const bool want_kids = !fin && L > 1 && (uint32_t)tid < nk;
    // issued unconditionally (a stand-in internal node for the others: a depth-1 node, or the
    // root when depth 1 holds the leaves), stored to LDS after the root's row
    const RowInfo ki = load_row_info(T, L > 1 ? n1 + (want_kids ? (uint32_t)tid : 0u) : 0u, 1);
    if (tid < 16) {
        // the root's row, as a tile's 16-lane group holds it
        const int j = tid;
        float x[kElems];
#pragma unroll
        for (int e = 0; e < kElems; ++e) x[e] = 0.0f;
        load_row<DT, VEC>(logits, ld, base, j, V, x);
        const uint32_t cb = T.child_begin[0];
        uint32_t bits[CH];
        if (0 < T.mask_depths) {
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int c0 = i * SPAN + j * CW;
                bits[i] = (T.mask[c0 >> 5] >> (c0 & 31)) & ((1u << CW) - 1u);
            }
        } else {
            const uint32_t ce = T.child_begin[1];
            if (j < 8) F.cm[j] = 0u;
            wave_lds_sync();
            for (uint32_t a = (cb & ~3u) + 4u * (uint32_t)j; a < ce; a += 64u) {
                const uint32_t wv = *reinterpret_cast<const uint32_t *>(T.child_code + a);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t idx = a + (uint32_t)k;
                    if (idx >= cb && idx < ce) {
                        const uint32_t c = (wv >> (8 * k)) & 255u;
                        atomicOr(&F.cm[c >> 5], 1u << (c & 31));
                    }
                }
            }
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int c0 = i * SPAN + j * CW;
                bits[i] = (F.cm[c0 >> 5] >> (c0 & 31)) & ((1u << CW) - 1u);
            }
        }
        if (W.validate) {
            // as the tile kernel reads the row: with sector gathering only the 16-byte
            // pieces that hold a child are read, hence checked
            bool bad = false;
#pragma unroll
            for (int e = 0; e < kElems; ++e)
                if (code_of<DT>(e, j) < V && !isfinite(x[e]) && (!(VEC && ra.gather()) || bits[e / CW] != 0u))
                    bad = true;
            if (bad) atomicOr(W.err, kErrNonFinite);
        }
        uint32_t tv = 0u;
#pragma unroll
        for (int i = 0; i < CH; ++i) tv |= bits[i] << (i * CW);
        uint32_t valid = tv;
        if constexpr (NORM == TCB_NORM_OPEN) {
            valid = 0u;
#pragma unroll
            for (int e = 0; e < kElems; ++e) valid |= code_of<DT>(e, j) < V ? (1u << e) : 0u;
        }
        float ph[SAMPLE ? kElems : 1];
        float lbest = -INFINITY;
        score_row<DT, NORM, SAMPLE>(R, q, 0, 0, j, V, true, valid, 0.0f, 0.0f, x, ph, lbest);
        // child node ids as the tile kernel forms them
        uint32_t pc = 0u;
#pragma unroll
        for (int i = 0; i < CH; ++i) pc |= (uint32_t)__popc(bits[i]) << (8 * i);
        const uint32_t rk = (row16_incl_scan(pc) - pc) + row16_sum_u(pc) * 0x01010100u;
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            const int c = code_of<DT>(e, j);
            const uint32_t below = tv & ((1u << e) - (1u << (e & ~(CW - 1))));
            int32_t n = (int32_t)(cb + ((rk >> (8 * (e / CW))) & 255u) + (uint32_t)__popc(below));
            if constexpr (NORM == TCB_NORM_OPEN) n = ((tv >> e) & 1u) ? n : -1;
            F.ord[c] = ((valid >> e) & 1u) ? f2ord(x[e]) : 0u;   // every code 0..255 is one (e, j)
            F.key[c] = x[e];
            if constexpr (SAMPLE) F.phi[c] = ph[e];
            else F.phi[c] = x[e];
            F.node[c] = n;
        }
    }
    if (want_kids) F.kid[tid] = ki;
    // rank: candidates are grouped by score bin (1 / kBinRes nat below the root's score 0);
    // a candidate's rank is the candidates of better bins plus the better ones of its own
    // bin, by (score desc, code asc)
    for (int i = tid; i <= kBins; i += 256) F.bin0[i] = 0u;
    __syncthreads();
    const uint32_t oo = F.ord[tid];
    const bool cand = oo != 0u;
    uint32_t b = 0u, within = 0u;
    if (cand) {
        b = score_bin(0.0f, F.key[tid]);
        within = atomicAdd(&F.bin0[b], 1u);
    }
    __syncthreads();
    // exclusive offsets of the 1024 bins, 4 per thread
    {
        const uint4 h = reinterpret_cast<const uint4 *>(F.bin0)[tid];
        const uint32_t sum = h.x + h.y + h.z + h.w;
        const uint32_t incl = wave_incl_scan(sum);
        if ((tid & 63) == 63) F.part[tid >> 6] = incl;
        __syncthreads();
        uint32_t before = 0u;
        for (int w = 0; w < (tid >> 6); ++w) before += F.part[w];
        const uint32_t e0 = before + incl - sum;
        reinterpret_cast<uint4 *>(F.bin0)[tid] = make_uint4(e0, e0 + h.x, e0 + h.x + h.y, e0 + h.x + h.y + h.z);
        if (tid == 255) F.bin0[kBins] = before + incl;   // every candidate
    }
    __syncthreads();
    const uint64_t key = ((uint64_t)oo << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)tid);   // larger: better
    const uint32_t st = F.bin0[b];
    if (cand) F.gk[st + within] = key;
    const uint32_t nvalid = F.bin0[kBins];
    __syncthreads();
    trace_mark(W, 6);                                 // scored and grouped
    const uint32_t k = min((uint32_t)ra.width(), nvalid);
    if (cand) {
        const uint32_t en = F.bin0[b + 1];
        uint32_t rank = st;
        for (uint32_t i = st; i < en; ++i) rank += F.gk[i] > key ? 1u : 0u;
        if (rank < k) {
            const int32_t node = F.node[tid];
            if (fin) {
                write_final_row(R.fin, L, W.Bmax, q, rank, 0ull, (uint32_t)tid, F.phi[tid], item_of(T, W, node));
            } else {
                write_new_row(W, ra, rank, F.key[tid], (uint32_t)tid, node, F.phi[tid]);
                // the row's child set (zeros for an unconstrained row off the catalog)
                const bool kid = (uint32_t)node - n1 < nk;
                const uint4 *src = reinterpret_cast<const uint4 *>(&F.kid[kid ? (uint32_t)node - n1 : 0u]);
                uint4 *dst = reinterpret_cast<uint4 *>(W.rinfo + base + (int)rank);
#pragma unroll
                for (int part = 0; part < 3; ++part) {
                    const uint4 v = src[part];        // LDS read, then the choice on values
                    const uint32_t keep = kid ? 0xFFFFFFFFu : 0u;
                    dst[part] = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
                }
            }
        }
    }
    if (fin) finish_request(T, W, R.fin, q, ra, rp, 1, k);
    else write_next_record(W, q, ra, rp, k);
    trace_mark(W, 7);                                 // ranked, rows issued
}

// ---------------------------------------------------------------------- tile launches
template <int DT, int NORM, bool VEC, bool SAMPLE, bool HEAD = false>
void launch_tile_t(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *logits,
                          int64_t ld, int mode, hipStream_t s) {
    const int groups = (R.n + 7) / 8;
    if (mode == kTileFirst) {
        const int nx = first_xcds(R.n);
        hipLaunchKernelGGL((k_first<DT, NORM, VEC, SAMPLE>), dim3(8 * ((R.n + nx - 1) / nx)), dim3(256), 0, s, t, w,
                           rp, R, logits, ld);
    } else if (mode == kTileMerge) {
        hipLaunchKernelGGL((k_tile<DT, NORM, VEC, SAMPLE, true, false, HEAD>), dim3(R.n), dim3(kThreads), 0, s, t, w, rp,
                           R, logits, ld);
    } else if (mode == kTileFuse) {
        hipLaunchKernelGGL((k_tile<DT, NORM, VEC, SAMPLE, false, true, HEAD>), dim3(8 * groups * w.MT), dim3(kThreads), 0,
                           s, t, w, rp, R, logits, ld);
    } else {
        hipLaunchKernelGGL((k_tile<DT, NORM, VEC, SAMPLE, false, false, HEAD>), dim3(8 * groups * w.MT), dim3(kThreads), 0,
                           s, t, w, rp, R, logits, ld);
    }
}

template <int DT, bool SAMPLE, bool VEC>
void launch_tile_v(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *logits,
                          int64_t ld, int merge, hipStream_t s) {
    switch (w.norm) {
    case TCB_NORM_LEVEL: launch_tile_t<DT, TCB_NORM_LEVEL, VEC, SAMPLE>(t, w, rp, R, logits, ld, merge, s); break;
    case TCB_NORM_OPEN: launch_tile_t<DT, TCB_NORM_OPEN, VEC, SAMPLE>(t, w, rp, R, logits, ld, merge, s); break;
    default: launch_tile_t<DT, TCB_NORM_CHILDREN, VEC, SAMPLE>(t, w, rp, R, logits, ld, merge, s); break;
    }
}

template <int DT, bool SAMPLE>
void launch_tile_dt(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *logits,
                           int64_t ld, bool vec, int merge, hipStream_t s) {
    if (vec) launch_tile_v<DT, SAMPLE, true>(t, w, rp, R, logits, ld, merge, s);
    else launch_tile_v<DT, SAMPLE, false>(t, w, rp, R, logits, ld, merge, s);
}

}  // namespace
}  // namespace tcb
