// SID-range lm_head on the gfx950 matrix cores.
//
// flashrec 0.1.0, Features > Decoding ("SID constraint"): the output head is evaluated
// only over the SID token range, i.e. one [V=256][H] matrix per SID level. For every live
// row (slot) of every stepped request, at that request's level l:
//     x[slot][c] = sum_h hidden[slot][h] * W[l][c][h]       (bf16 inputs, fp32 sums)
// The logits go to an fp32 [max_slots][256] workspace that the tile kernel reads next,
// so the masked log-softmax and selection are the same code as for logits from memory.
//
// Tiling. A workgroup of 4 waves computes a 64-row x 64-code block with
// v_mfma_f32_16x16x32_bf16. The block's K range is split across the waves: wave w
// accumulates the whole 64 x 64 block (4 x 4 tiles of 16 x 16, 64 fp32 per lane) over
// its quarter of K with many K-steps of loads in flight (one workgroup per CU leaves each
// wave a whole SIMD and its register file). The loads are row-contiguous (four lanes read
// one row's 64 bytes of a K-step) and each step passes through the wave's own LDS stage
// into the MFMA operand layout (lane = row): loading that layout straight from memory
// touches 16 rows per instruction and runs at about a third of the per-CU load rate
// (measured on gfx950). The four partial blocks are then added through LDS in a
// fixed order (wave 0 + 1 + 2 + 3), so results are deterministic. The four code blocks
// of one row tile are dealt to the same XCD, so the hidden rows they share are read
// from HBM once and then hit that XCD's L2.
//
#include "tcb_internal.h"

namespace tcb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGRows = 64;                 // rows of a block
constexpr int kGCodes = 64;                // codes of a block (4 blocks cover V = 256)
constexpr int kGThreads = 256;             // 4 waves, each over a quarter of K
constexpr int kKStep = 32;                 // K of one MFMA
// a staged row (64 bytes of one K-step) padded to 80 bytes: the 16 rows one MFMA-layout
// read instruction touches start in distinct 16-byte bank groups
constexpr int kStageRow = 80;

// NS = K-steps of 32 per wave (H = 4 * 32 * NS); NS = 0: any H % 128 == 0, one step
// of loads in flight.
template <int NS>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_lmhead(TrieDev T, WaveDev W, int rp, StepReqs R,
                                                      const uint16_t *__restrict__ hidden, int64_t ld, int H,
                                                      const uint16_t *__restrict__ weight,
                                                      float *__restrict__ out) {
    __shared__ f32x4 red[4][4][4][64];                        // [wave][row blk][code blk][lane]
    __shared__ __attribute__((aligned(16))) uint8_t stage[4][2][64 * kStageRow];   // [wave][A, B][row]
    const int MT = W.MT;
    const int xcd = (int)(blockIdx.x & 7u), i8 = (int)(blockIdx.x >> 3);
    const int cblk = i8 & 3;                                  // code block 0..3
    const int gt = (i8 >> 2) * 8 + xcd;                       // row tile over (request, tile)
    const int ql = gt / MT, rt = gt - ql * MT;
    if (ql >= R.n) return;
    const ReqArg ra = R.r[ql];
    if (!ra.step() || ra.sparse_head()) return;
    const int r0 = rt * kGRows;
    if (r0 >= ra.rmax()) return;
    // operand loads are issued for every row the request can have; the live-row count
    // arrives with them and decides which results are stored
    const int rows_bound = ra.rmax(), base = ra.base(), level = ra.level();

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kq = lane >> 4;                // MFMA layout: row l16, k chunk kq
    const int lr = lane >> 2, lc = lane & 3;                  // loads: row lr (+16 i), 16-byte chunk lc
    const int nsteps = NS > 0 ? NS : H / (4 * kKStep);
    const int kw0 = wave * nsteps * kKStep;                   // this wave's first k
    const uint16_t *ag[4], *bg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ar = r0 + 16 * i + lr;                      // rows past the bound read row r0, never stored
        ag[i] = hidden + (size_t)(base + (ar < rows_bound ? ar : r0)) * (size_t)ld + kw0 + 8 * lc;
        bg[i] = weight + ((size_t)level * 256 + (size_t)cblk * kGCodes + 16 * i + lr) * (size_t)H + kw0 + 8 * lc;
    }
    uint8_t *sa = stage[wave][0], *sb = stage[wave][1];
    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // one K-step: the loaded pieces into the wave's stage, back out in the MFMA layout
    // (the same k of each row as a direct load of that layout), 4 x 4 MFMAs. LDS operations
    // of one wave complete in order, so the stage needs no barrier.
    auto stage_step = [&](const u32x4 (&ra)[4], const u32x4 (&rb)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<u32x4 *>(sa + (16 * i + lr) * kStageRow + 16 * lc) = ra[i];
            *reinterpret_cast<u32x4 *>(sb + (16 * i + lr) * kStageRow + 16 * lc) = rb[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        u32x4 av[4], bv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            av[b] = *reinterpret_cast<const u32x4 *>(sa + (16 * b + l16) * kStageRow + 16 * kq);
            bv[b] = *reinterpret_cast<const u32x4 *>(sb + (16 * b + l16) * kStageRow + 16 * kq);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[a]),
                                                                    __builtin_bit_cast(bf16x8, bv[b]), acc[a][b],
                                                                    0, 0, 0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    if constexpr (NS > 0) {
        // a ring of PD K-steps of loads in registers, refilled as each step is used
        constexpr int PD = NS < 4 ? NS : 4;       // deeper rings spill past the 256 VGPRs
        u32x4 ra[PD][4], rb[PD][4];
#pragma unroll
        for (int s = 0; s < PD; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[s][i] = *reinterpret_cast<const u32x4 *>(ag[i] + s * kKStep);
                rb[s][i] = *reinterpret_cast<const u32x4 *>(bg[i] + s * kKStep);
            }
        __builtin_amdgcn_sched_barrier(0);                    // keep the ring's loads issued up front
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            stage_step(ra[s % PD], rb[s % PD]);
            if (s + PD < NS) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ra[s % PD][i] = *reinterpret_cast<const u32x4 *>(ag[i] + (s + PD) * kKStep);
                    rb[s % PD][i] = *reinterpret_cast<const u32x4 *>(bg[i] + (s + PD) * kKStep);
                }
            }
        }
    } else {
        for (int s = 0; s < nsteps; ++s) {
            u32x4 ra[4], rb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[i] = *reinterpret_cast<const u32x4 *>(ag[i] + s * kKStep);
                rb[i] = *reinterpret_cast<const u32x4 *>(bg[i] + s * kKStep);
            }
            stage_step(ra, rb);
        }
    }
    // a first step: the root only; a pending merge (done by the tile kernel that follows):
    // every row the request can have
    const int rows = level == 0 ? 1 : R.r[ql].pending() ? rows_bound : W.rec[rp][R.q0 + ql].rows;
    // partial blocks of the four waves, added in a fixed order; wave w finishes row block w
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) red[wave][a][b][lane] = acc[a][b];
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f32x4 v = red[0][wave][b][lane];
        v += red[1][wave][b][lane];
        v += red[2][wave][b][lane];
        v += red[3][wave][b][lane];
        // D layout: rows 4 kq + i of row block `wave`, code 16 b + l16 of the block
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = r0 + 16 * wave + 4 * kq + i;
            if (row < rows) out[(size_t)(base + row) * 256 + cblk * kGCodes + 16 * b + l16] = v[i];
        }
    }
}

// Children-only lm_head ([FR] Decoding: the dense or CSR-sparse choice, applied to the
// head's flops). One wave per live row: the row's hidden state is read once into registers
// (8 bf16 per lane per chunk of 512), its children are walked in ascending code order, and
// for every 16-byte piece of the logit row (4 codes) that holds a child the 4 dot products
// over H are summed per lane in fp32 and reduced across the wave in a fixed order. Pieces
// holding no child are not written: the tile kernel then reads only the pieces that hold a
// child (the request's gather flag is set with the sparse-head flag).
constexpr int kSpWaves = 4;

__global__ __launch_bounds__(64 * kSpWaves) void k_lmhead_sparse(TrieDev T, WaveDev W, int rp, StepReqs R,
                                                               const uint16_t *__restrict__ hidden, int64_t ld, int H,
                                                               const uint16_t *__restrict__ weight,
                                                               float *__restrict__ out, int quads) {
    const int ql = (int)blockIdx.x / quads, quad = (int)blockIdx.x - ql * quads;
    if (ql >= R.n) return;
    const ReqArg ra = R.r[ql];
    if (!ra.step() || !ra.sparse_head()) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = quad * kSpWaves + wave;
    const int level = ra.level();
    const int rows = level == 0 ? 1 : W.rec[rp][R.q0 + ql].rows;   // a first step: the root only
    if (r >= rows) return;
    const int base = ra.base(), slot = base + r;
    const uint32_t nd = level == 0 ? 0u : (uint32_t)W.node[ra.par()][slot];
    if (nd < T.off[level] || nd >= T.off[level + 1]) return;       // not a node of this depth: the tile kernel flags it
    const uint32_t cb = T.child_begin[nd], ce = T.child_begin[nd + 1];
    const int nch = H / 8;                                         // chunks of 8 bf16
    const u32x4 *hp = reinterpret_cast<const u32x4 *>(hidden + (size_t)slot * (size_t)ld);
    u32x4 hv[8];                                                   // H <= 4096: up to 8 chunks per lane
#pragma unroll
    for (int i = 0; i < 8; ++i) hv[i] = (lane + 64 * i < nch) ? hp[lane + 64 * i] : u32x4{0u, 0u, 0u, 0u};
    const uint16_t *wl = weight + (size_t)level * 256 * (size_t)H;
    int last = -1;
    for (uint32_t k = cb; k < ce; ++k) {
        const int piece = T.child_code[k] >> 2;
        if (piece == last) continue;                               // uniform: every lane walks the same list
        last = piece;
        float d[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 *wp = reinterpret_cast<const u32x4 *>(wl + (size_t)(4 * piece + c) * (size_t)H);
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (lane + 64 * i < nch) {
                    const u32x4 wv = wp[lane + 64 * i];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc = fmaf(__uint_as_float(hv[i][q] << 16), __uint_as_float(wv[q] << 16), acc);
                        acc = fmaf(__uint_as_float(hv[i][q] & 0xffff0000u), __uint_as_float(wv[q] & 0xffff0000u), acc);
                    }
                }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
            d[c] = acc;
        }
        if (lane < 4) out[(size_t)slot * 256 + 4 * piece + lane] = lane == 0 ? d[0] : lane == 1 ? d[1] : lane == 2 ? d[2] : d[3];
    }
}

}  // namespace

hipError_t launch_lmhead_sparse(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *hidden,
                                int64_t ld, int H, const void *weight, float *out, int max_rows, hipStream_t s) {
    if (R.n <= 0 || max_rows <= 0) return hipSuccess;
    if (H > 4096) return hipErrorInvalidValue;
    const int quads = (max_rows + kSpWaves - 1) / kSpWaves;
    hipLaunchKernelGGL(k_lmhead_sparse, dim3(R.n * quads), dim3(64 * kSpWaves), 0, s, t, w, rp, R,
                       static_cast<const uint16_t *>(hidden), ld, H, static_cast<const uint16_t *>(weight), out, quads);
    return hipGetLastError();
}

hipError_t launch_lmhead(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *hidden,
                         int64_t ld, int H, const void *weight, float *out, hipStream_t s) {
    if (R.n <= 0) return hipSuccess;
    const int tiles = R.n * w.MT;                             // row tiles over all requests
    const int groups = (tiles + 7) / 8;
    const dim3 grid(8 * groups * 4), block(kGThreads);
    const uint16_t *h = static_cast<const uint16_t *>(hidden), *wt = static_cast<const uint16_t *>(weight);
    switch (H) {
    case 512: hipLaunchKernelGGL(k_lmhead<4>, grid, block, 0, s, t, w, rp, R, h, ld, H, wt, out); break;
    case 1024: hipLaunchKernelGGL(k_lmhead<8>, grid, block, 0, s, t, w, rp, R, h, ld, H, wt, out); break;
    case 2048: hipLaunchKernelGGL(k_lmhead<16>, grid, block, 0, s, t, w, rp, R, h, ld, H, wt, out); break;
    case 4096: hipLaunchKernelGGL(k_lmhead<32>, grid, block, 0, s, t, w, rp, R, h, ld, H, wt, out); break;
    default: hipLaunchKernelGGL(k_lmhead<0>, grid, block, 0, s, t, w, rp, R, h, ld, H, wt, out); break;
    }
    return hipGetLastError();
}

}  // namespace tcb
