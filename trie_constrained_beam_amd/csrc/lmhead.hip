// SID-range lm_head on the gfx950 matrix cores.
//
// flashrec 0.1.0, Features > Decoding ("SID constraint"): the output head is evaluated
// only over the SID token range, i.e. one [V=256][H] matrix per SID level. For every live
// row (slot) of every stepped request, at that request's level l:
//     x[slot][c] = sum_h hidden[slot][h] * W[l][c][h]       (bf16 inputs, fp32 sums)
// The logits go to an fp32 [max_slots][256] workspace that the tile kernel reads next,
// so the masked log-softmax and selection are the same code as for logits from memory.
// This is the dense head, for depths where rows have many children; where they have about
// one, the tile kernel computes only the children's logits itself (no launch here).
//
// Tiling. A workgroup of 4 waves computes a 64-row x 64-code block with
// v_mfma_f32_16x16x32_bf16 (32 or 16 rows where 64-row blocks would leave CUs idle). The
// block's K range is split across the waves: wave w accumulates the whole 64 x 64 block
// (4 x 4 tiles of 16 x 16, 64 fp32 per lane) over its quarter of K with many K-steps of
// loads in flight (one workgroup per CU leaves each wave a whole SIMD and its register
// file). The loads are row-contiguous (eight lanes read
// 128 bytes of one row: two K-steps, whole 128-byte lines, so each request to L2 carries a
// whole line) and each pair of steps passes through the wave's own LDS stage into the MFMA
// operand layout (lane = row): loading that layout straight from memory touches 16 rows
// per instruction and runs at about a third of the per-CU load rate (measured on gfx950).
// In the stage, 16-byte piece p of row r sits at piece p ^ (r mod 8) of the row, so that
// neither the row-wise writes nor the MFMA-layout reads (8 lanes per LDS pass, 8
// consecutive rows) meet a bank conflict. The four partial blocks are then added through
// LDS in a fixed order (wave 0 + 1 + 2 + 3), so results are deterministic. The four code
// blocks of one row tile are dealt to the same XCD, so the hidden rows they share are read
// from HBM once and then hit that XCD's L2.
//
#include "tcb_internal.h"

namespace tcb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGCodes = 64;                // codes of a block (4 blocks cover V = 256)
constexpr int kGThreads = 256;             // 4 waves, each over a quarter of K
constexpr int kKStep = 32;                 // K of one MFMA

// K-steps per load chunk: two (128 bytes of a row) where the wave's step count is even
template <int NS>
constexpr int lm_group() { return NS > 0 && NS % 2 == 0 ? 2 : 1; }
// byte offset of 16-byte piece p of row r in a stage whose rows hold G K-steps (64 G bytes):
// pieces are permuted within the row by the row's low bits (conflict-free writes and reads)
template <int G>
__device__ __forceinline__ int stage_at(int r, int p) {
    return r * 64 * G + 16 * (p ^ (G == 2 ? (r & 7) : ((r >> 1) & 3)));
}

// NS = K-steps of 32 per wave (H = 4 * 32 * NS); NS = 0: any H % 128 == 0, one step
// of loads in flight. RB = row blocks of 16 per tile (4, 2 or 1) and mt = tiles per request:
// smaller tiles where 64-row tiles would leave CUs idle (a first step, or few rows), so that
// the launch fills the chip and computes fewer dead rows.
template <int NS, int RB>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_lmhead(TrieDev T, WaveDev W, int rp, StepReqs R,
                                                      const uint16_t *__restrict__ hidden, int64_t ld, int H,
                                                      const uint16_t *__restrict__ weight,
                                                      float *__restrict__ out, int mt) {
    constexpr int G = lm_group<NS>();                        // K-steps per load chunk
    constexpr int LPR = 4 * G;                                // lanes per row in a load (16 bytes each)
    constexpr int RPI = 64 / LPR;                             // rows per load instruction
    constexpr int TR = 16 * RB;                               // rows of a tile
    constexpr int NIA = TR / RPI, NIB = kGCodes / RPI;        // load instructions per chunk: rows, codes
    __shared__ f32x4 red[4][RB][4][64];                       // [wave][row blk][code blk][lane]
    __shared__ __attribute__((aligned(16))) uint8_t stage_a[4][TR * 64 * G];       // [wave][row]
    __shared__ __attribute__((aligned(16))) uint8_t stage_b[4][kGCodes * 64 * G];  // [wave][code]
    const int MT = mt;
    const int xcd = (int)(blockIdx.x & 7u), i8 = (int)(blockIdx.x >> 3);
    const int cblk = i8 & 3;                                  // code block 0..3
    const int gt = (i8 >> 2) * 8 + xcd;                       // row tile over (request, tile)
    const int ql = gt / MT, rt = gt - ql * MT;
    if (ql >= R.n) return;
    const ReqArg ra = R.r[ql];
    if (!ra.step() || ra.sparse_head()) return;
    const int r0 = rt * TR;
    if (r0 >= ra.rmax()) return;
    // operand loads are issued for every row the request can have; the live-row count
    // arrives with them and decides which results are stored
    const int rows_bound = ra.rmax(), base = ra.base(), level = ra.level();

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kq = lane >> 4;                // MFMA layout: row l16, k chunk kq
    const int lr = lane / LPR, lc = lane % LPR;               // loads: row lr (+RPI i), 16-byte piece lc
    const int nsteps = NS > 0 ? NS : H / (4 * kKStep);
    const int kw0 = wave * nsteps * kKStep;                   // this wave's first k
    const uint16_t *ag[NIA], *bg[NIB];
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
        const int ar = r0 + RPI * i + lr;                     // rows past the bound read row r0, never stored
        ag[i] = hidden + (size_t)(base + (ar < rows_bound ? ar : r0)) * (size_t)ld + kw0 + 8 * lc;
    }
#pragma unroll
    for (int i = 0; i < NIB; ++i)
        bg[i] = weight + ((size_t)level * 256 + (size_t)cblk * kGCodes + RPI * i + lr) * (size_t)H + kw0 + 8 * lc;
    uint8_t *sa = stage_a[wave], *sb = stage_b[wave];
    f32x4 acc[RB][4];
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // one chunk of G K-steps: the loaded pieces into the wave's stage, back out in the MFMA
    // layout (the same k of each row as a direct load of that layout), RB x 4 MFMAs per
    // K-step in K order. LDS operations of one wave complete in order, so the stage needs
    // no barrier.
    auto stage_chunk = [&](const u32x4 (&ra)[NIA], const u32x4 (&rb)[NIB]) {
#pragma unroll
        for (int i = 0; i < NIA; ++i) *reinterpret_cast<u32x4 *>(sa + stage_at<G>(RPI * i + lr, lc)) = ra[i];
#pragma unroll
        for (int i = 0; i < NIB; ++i) *reinterpret_cast<u32x4 *>(sb + stage_at<G>(RPI * i + lr, lc)) = rb[i];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int h = 0; h < G; ++h) {
            u32x4 av[RB], bv[4];
#pragma unroll
            for (int a = 0; a < RB; ++a)
                av[a] = *reinterpret_cast<const u32x4 *>(sa + stage_at<G>(16 * a + l16, 4 * h + kq));
#pragma unroll
            for (int b = 0; b < 4; ++b)
                bv[b] = *reinterpret_cast<const u32x4 *>(sb + stage_at<G>(16 * b + l16, 4 * h + kq));
#pragma unroll
            for (int a = 0; a < RB; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[a]),
                                                                        __builtin_bit_cast(bf16x8, bv[b]), acc[a][b],
                                                                        0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    if constexpr (NS > 0) {
        // a ring of PD chunks of loads in registers, refilled as each chunk is used
        constexpr int NC = NS / G;                            // chunks per wave
        constexpr int PD = NC < 4 / G ? NC : 4 / G;           // 4 K-steps of loads in flight
        u32x4 ra[PD][NIA], rb[PD][NIB];
#pragma unroll
        for (int s = 0; s < PD; ++s) {
#pragma unroll
            for (int i = 0; i < NIA; ++i) ra[s][i] = *reinterpret_cast<const u32x4 *>(ag[i] + s * G * kKStep);
#pragma unroll
            for (int i = 0; i < NIB; ++i) rb[s][i] = *reinterpret_cast<const u32x4 *>(bg[i] + s * G * kKStep);
        }
        __builtin_amdgcn_sched_barrier(0);                    // keep the ring's loads issued up front
#pragma unroll
        for (int s = 0; s < NC; ++s) {
            stage_chunk(ra[s % PD], rb[s % PD]);
            if (s + PD < NC) {
#pragma unroll
                for (int i = 0; i < NIA; ++i)
                    ra[s % PD][i] = *reinterpret_cast<const u32x4 *>(ag[i] + (s + PD) * G * kKStep);
#pragma unroll
                for (int i = 0; i < NIB; ++i)
                    rb[s % PD][i] = *reinterpret_cast<const u32x4 *>(bg[i] + (s + PD) * G * kKStep);
            }
        }
    } else {
        for (int s = 0; s < nsteps; ++s) {
            u32x4 ra[NIA], rb[NIB];
#pragma unroll
            for (int i = 0; i < NIA; ++i) ra[i] = *reinterpret_cast<const u32x4 *>(ag[i] + s * kKStep);
#pragma unroll
            for (int i = 0; i < NIB; ++i) rb[i] = *reinterpret_cast<const u32x4 *>(bg[i] + s * kKStep);
            stage_chunk(ra, rb);
        }
    }
    // a first step: the root only; a pending merge (done by the tile kernel that follows):
    // every row the request can have
    const int rows = level == 0 ? 1 : R.r[ql].pending() ? rows_bound : W.rec[rp][R.q0 + ql].rows;
    // partial blocks of the four waves, added in a fixed order; wave w finishes the blocks
    // (a, b) with a + b = w mod 4
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) red[wave][a][b][lane] = acc[a][b];
    __syncthreads();
#pragma unroll
    for (int a = 0; a < RB; ++a) {
        const int b = (wave - a) & 3;
        f32x4 v = red[0][a][b][lane];
        v += red[1][a][b][lane];
        v += red[2][a][b][lane];
        v += red[3][a][b][lane];
        // D layout: rows 4 kq + i of row block a, code 16 b + l16 of the block
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = r0 + 16 * a + 4 * kq + i;
            if (row < rows) out[(size_t)(base + row) * 256 + cblk * kGCodes + 16 * b + l16] = v[i];
        }
    }
}

// First steps: each request has one row (the root, in its first slot), so its head is a
// matrix-vector product, 256 dot products over H. The 64-row MFMA tiles would stream the whole
// weight matrix through a few workgroups for one live row; here a request's 256 codes are
// spread over 32 workgroups of 4 waves, 2 codes per wave, so the matrix streams once through
// every CU. All 64 lanes of a wave share a code: lane l sums the products of the 16-byte
// pieces l, l + 64, ... of the hidden row and the weight row (8 elements each, in element
// order), then the 64 lane sums are added by a fixed butterfly, so the logits are
// deterministic (they differ from the MFMA head's only by the order of the fp32 sums).
constexpr int kRootCodesPerWg = 8;
constexpr int kRootBatch = 4;                             // 16-byte pieces of each operand per lane per round

__device__ __forceinline__ float root_dot8(const u32x4 &a, const u32x4 &b, float acc) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        acc = fmaf(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), acc);
        acc = fmaf(__uint_as_float(a[w] & 0xffff0000u), __uint_as_float(b[w] & 0xffff0000u), acc);
    }
    return acc;
}

__global__ __launch_bounds__(256) void k_lmhead_root(StepReqs R, const uint16_t *__restrict__ hidden, int64_t ld,
                                                     int H, const uint16_t *__restrict__ weight,
                                                     float *__restrict__ out) {
    constexpr int G = 256 / kRootCodesPerWg;                  // workgroups per request
    const int ql = (int)blockIdx.x / G, cg = (int)blockIdx.x - ql * G;
    if (ql >= R.n) return;
    const ReqArg ra = R.r[ql];
    if (!ra.step() || ra.sparse_head() || ra.level() != 0) return;
    const int lane = (int)(threadIdx.x & 63u), wave = (int)(threadIdx.x >> 6);
    const int slot = ra.base();
    const int pieces = H >> 3;                                // 16-byte pieces of a row
    const int c0 = cg * kRootCodesPerWg + 2 * wave;           // this wave's codes c0, c0 + 1 (level 0)
    const u32x4 *hp = reinterpret_cast<const u32x4 *>(hidden + (size_t)slot * (size_t)ld);
    const u32x4 *w0 = reinterpret_cast<const u32x4 *>(weight + (size_t)c0 * (size_t)H);
    const u32x4 *w1 = w0 + pieces;
    float a0 = 0.0f, a1 = 0.0f;
    for (int p0 = 0; p0 < pieces; p0 += 64 * kRootBatch) {
        u32x4 hv[kRootBatch], x0[kRootBatch], x1[kRootBatch];
#pragma unroll
        for (int i = 0; i < kRootBatch; ++i) {
            const int p = min(p0 + 64 * i + lane, pieces - 1);  // past the row: read, not summed
            hv[i] = __builtin_nontemporal_load(hp + p);
            x0[i] = w0[p];
            x1[i] = w1[p];
        }
#pragma unroll
        for (int i = 0; i < kRootBatch; ++i)
            if (p0 + 64 * i + lane < pieces) {
                a0 = root_dot8(hv[i], x0[i], a0);
                a1 = root_dot8(hv[i], x1[i], a1);
            }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        a0 += __shfl_xor(a0, o, 64);
        a1 += __shfl_xor(a1, o, 64);
    }
    if (lane == 0) {
        out[(size_t)slot * 256 + c0] = a0;
        out[(size_t)slot * 256 + c0 + 1] = a1;
    }
}

// compute units of the current device (queried once per device)
int cu_count() {
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] <= 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) return 256;
        cache[dev] = c;
    }
    return cache[dev];
}

template <int RB>
void launch_lmhead_rb(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const uint16_t *h, int64_t ld,
                      int H, const uint16_t *wt, float *out, int mt, hipStream_t s) {
    const int tiles = R.n * mt;                               // row tiles over all requests
    const int groups = (tiles + 7) / 8;
    const dim3 grid(8 * groups * 4), block(kGThreads);
    switch (H) {
    case 512: hipLaunchKernelGGL((k_lmhead<4, RB>), grid, block, 0, s, t, w, rp, R, h, ld, H, wt, out, mt); break;
    case 1024: hipLaunchKernelGGL((k_lmhead<8, RB>), grid, block, 0, s, t, w, rp, R, h, ld, H, wt, out, mt); break;
    case 2048: hipLaunchKernelGGL((k_lmhead<16, RB>), grid, block, 0, s, t, w, rp, R, h, ld, H, wt, out, mt); break;
    case 4096: hipLaunchKernelGGL((k_lmhead<32, RB>), grid, block, 0, s, t, w, rp, R, h, ld, H, wt, out, mt); break;
    default: hipLaunchKernelGGL((k_lmhead<0, RB>), grid, block, 0, s, t, w, rp, R, h, ld, H, wt, out, mt); break;
    }
}

}  // namespace

hipError_t launch_lmhead(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *hidden,
                         int64_t ld, int H, const void *weight, float *out, hipStream_t s) {
    if (R.n <= 0) return hipSuccess;
    int rmax = 0;                                             // rows any request of the launch can have
    for (int i = 0; i < R.n; ++i)
        if (R.r[i].step() && !R.r[i].sparse_head()) rmax = std::max(rmax, R.r[i].rmax());
    if (rmax <= 0) return hipSuccess;
    const uint16_t *h = static_cast<const uint16_t *>(hidden), *wt = static_cast<const uint16_t *>(weight);
    bool first = true;                                        // every dense-head request at its first step
    for (int i = 0; i < R.n; ++i)
        if (R.r[i].step() && !R.r[i].sparse_head() && R.r[i].level() != 0) first = false;
    if (first) {
        hipLaunchKernelGGL(k_lmhead_root, dim3(R.n * (256 / kRootCodesPerWg)), dim3(256), 0, s, R, h, ld, H, wt, out);
        return hipGetLastError();
    }
    // the tallest tiles whose 4 code blocks still give every CU a workgroup; else 16 rows
    const int cus = cu_count();
    auto tiles = [&](int rows) { return (rmax + rows - 1) / rows; };
    if (4 * R.n * tiles(64) >= cus) launch_lmhead_rb<4>(t, w, rp, R, h, ld, H, wt, out, tiles(64), s);
    else if (4 * R.n * tiles(32) >= cus) launch_lmhead_rb<2>(t, w, rp, R, h, ld, H, wt, out, tiles(32), s);
    else launch_lmhead_rb<1>(t, w, rp, R, h, ld, H, wt, out, tiles(16), s);
    return hipGetLastError();
}

}  // namespace tcb
