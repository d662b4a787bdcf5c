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
// v_mfma_f32_16x16x32_bf16: wave w owns rows 16w..16w+15 and keeps four 16x16 fp32
// accumulators (codes 0..63 of the block). K is walked in chunks of 64: the block's
// 64 x 64 slice of W is shared through LDS (double-buffered, one barrier per chunk),
// each wave reads its own 16 rows of hidden straight into MFMA operand registers. The
// four code blocks of one row tile are dealt to the same XCD, so the hidden rows they
// share are read from HBM once and then hit that XCD's L2. Each output element is
// accumulated by one wave in a fixed K order: results are deterministic.
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 (64 lanes, l = lane):
//   A (16 x 32):  lane l holds A[l % 16][8 (l / 16) .. 8 (l / 16) + 7]
//   B (32 x 16):  lane l holds B[8 (l / 16) .. 8 (l / 16) + 7][l % 16]
//   D (16 x 16):  lane l holds D[4 (l / 16) + i][l % 16], i = 0..3
// With A = hidden rows and B[k][c] = W[c][k], both operands are 16 contiguous bytes of
// a row-major array.
#include "tcb_internal.h"

namespace tcb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGRows = 64;                 // rows of a block
constexpr int kGCodes = 64;                // codes of a block (4 blocks cover V = 256)
constexpr int kGK = 64;                    // K chunk
constexpr int kGThreads = 256;
constexpr int kBStride = kGK + 8;          // bf16 per code row in LDS (16-byte pad)

__global__ __launch_bounds__(kGThreads) void k_lmhead(TrieDev T, WaveDev W, int rp, int n_req,
                                                      const uint16_t *__restrict__ hidden, int64_t ld, int H,
                                                      const uint16_t *__restrict__ weight,
                                                      float *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][kGCodes * kBStride];
    const int MT = W.MT;
    const int xcd = (int)(blockIdx.x & 7u), i8 = (int)(blockIdx.x >> 3);
    const int cblk = i8 & 3;                                  // code block 0..3
    const int gt = (i8 >> 2) * 8 + xcd;                       // row tile over (request, tile)
    const int q = gt / MT, rt = gt - q * MT;
    if (q >= n_req) return;
    const ReqRec rec = W.rec[rp][q];
    if (rec.status != kReqActive || rec.level >= T.L || rec.rows <= 0) return;
    const int r0 = rt * kGRows;
    if (r0 >= rec.rows) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kq = lane >> 4;
    // A: this lane's hidden row (dead rows read row r0 and are never stored)
    const int ar = r0 + wave * 16 + l16;
    const uint16_t *arow = hidden + (size_t)(rec.base + (ar < rec.rows ? ar : r0)) * (size_t)ld + 8 * kq;
    // B loader: thread t copies 16 k-values of code t / 4 per chunk
    const int bc = tid >> 2, bk = (tid & 3) * 16;
    const uint16_t *brow = weight + ((size_t)rec.level * 256 + (size_t)cblk * kGCodes + bc) * (size_t)H + bk;

    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int nk = H / kGK;
    u32x4 nb0 = *reinterpret_cast<const u32x4 *>(brow);
    u32x4 nb1 = *reinterpret_cast<const u32x4 *>(brow + 8);
    u32x4 na0 = *reinterpret_cast<const u32x4 *>(arow);
    u32x4 na1 = *reinterpret_cast<const u32x4 *>(arow + 32);
    for (int kc = 0; kc < nk; ++kc) {
        uint16_t *sb = sB[kc & 1];
        *reinterpret_cast<u32x4 *>(sb + bc * kBStride + bk) = nb0;
        *reinterpret_cast<u32x4 *>(sb + bc * kBStride + bk + 8) = nb1;
        const u32x4 a0 = na0, a1 = na1;
        __syncthreads();
        if (kc + 1 < nk) {                                    // prefetch the next chunk
            const size_t ko = (size_t)(kc + 1) * kGK;
            nb0 = *reinterpret_cast<const u32x4 *>(brow + ko);
            nb1 = *reinterpret_cast<const u32x4 *>(brow + ko + 8);
            na0 = *reinterpret_cast<const u32x4 *>(arow + ko);
            na1 = *reinterpret_cast<const u32x4 *>(arow + ko + 32);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, ks ? a1 : a0);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 bv = *reinterpret_cast<const u32x4 *>(sb + (16 * c + l16) * kBStride + 32 * ks + 8 * kq);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bv), acc[c], 0, 0, 0);
            }
        }
    }
    // D: rows 4 kq + i of the wave's 16, code 16 c + l16 of the block
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = r0 + wave * 16 + 4 * kq + i;
        if (row < rec.rows) {
            float *o = out + (size_t)(rec.base + row) * 256 + cblk * kGCodes + l16;
#pragma unroll
            for (int c = 0; c < 4; ++c) o[16 * c] = acc[c][i];
        }
    }
}

}  // namespace

hipError_t launch_lmhead(const TrieDev &t, const WaveDev &w, int rp, int n_req, const void *hidden, int64_t ld,
                         int H, const void *weight, float *out, hipStream_t s) {
    if (n_req <= 0) return hipSuccess;
    const int tiles = n_req * w.MT;                           // row tiles over all requests
    const int groups = (tiles + 7) / 8;
    hipLaunchKernelGGL(k_lmhead, dim3(8 * groups * 4), dim3(kGThreads), 0, s, t, w, rp, n_req,
                       static_cast<const uint16_t *>(hidden), ld, H, static_cast<const uint16_t *>(weight), out);
    return hipGetLastError();
}

}  // namespace tcb
