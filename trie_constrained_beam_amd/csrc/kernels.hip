// gfx950 kernels of the step outside the tile kernel (merge, init, finalize, export) and
// the launchers; the tile kernel variants are compiled in tile_f32.hip, tile_bf16.hip,
// tile_f32_sampled.hip and tile_bf16_sampled.hip (device code in beam_device.h).
#include "beam_device.h"

namespace tcb {
namespace {

__global__ __launch_bounds__(kThreads) void k_merge(TrieDev T, WaveDev W, int rp, StepReqs R) {
    __shared__ MergeSmem M;
    __shared__ SelSmem sel;
    __shared__ uint32_t Hs[TCB_MAX_L - 1][kThreads];
    const int ql = blockIdx.x;
    if (ql >= R.n) return;
    trace_mark(W, 0);
    trace_mark(W, 1);
    const ReqArg ra = R.r[ql];
    if (!ra.step()) return;                            // carried over by k_tile
    merge_request(T, W, R.fin, R.q0 + ql, ra, rp, M, sel, Hs, RowsToMemory{W, ra, R.q0 + ql, rp});
}

// ---------------------------------------------------------------------- small kernels
__global__ void k_clear_wave(WaveDev W) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < W.R) {
        const ReqRec r{};
        W.rec[0][i] = r;
        W.rec[1][i] = r;
    }
    if (i == 0) *W.err = 0u;
}

__global__ void k_init(WaveDev W, InitBatch b) {
    const int i = threadIdx.x;
    if (i >= b.n) return;
    ReqRec r{};
    r.base = b.base[i];
    r.width = b.width[i];
    r.rows = 1;
    r.level = 0;
    r.status = kReqActive;
    r.par = 0;
    W.rec[0][b.req[i]] = r;
    W.rec[1][b.req[i]] = r;
    W.node[0][b.base[i]] = 0;          // the root
    W.score[0][b.base[i]] = 0.0f;
    W.phi[0][b.base[i]] = 0.0f;
}

__global__ void k_finalize(TrieDev T, WaveDev W, int rp, FinBatch fb, uint8_t *sids, float *scores,
                           int64_t *items, int32_t *counts) {
    const int i = blockIdx.x;
    if (i >= fb.n) return;
    const int req = fb.req[i], base = fb.base[i], width = fb.width[i], par = fb.par[i];
    const size_t orow = (size_t)fb.out_row[i];
    const int L = T.L;
    const uint32_t leaf0 = T.off[L], leaf1 = T.off[L + 1];
    // the live-row count, and each row's state and last back-pointer for every row the
    // request can have, are loaded at once (rows past the count are dropped)
    const int rows = W.rec[rp][req].rows;
    for (int j = threadIdx.x; j < W.Bmax; j += blockDim.x) {
        const size_t out = orow * (size_t)W.Bmax + (size_t)j;
        uint32_t node = 0u, h = 0u;
        float phi = 0.0f;
        if (j < width) {
            const int slot = base + j;
            node = (uint32_t)W.node[par][slot];
            phi = W.phi[par][slot];
            h = W.hist[(size_t)(L - 1) * W.S + slot];
        }
        if (j < rows) {
            int64_t item = -1;
            if (node >= leaf0 && node < leaf1) item = T.leaf_item[node - leaf0];
            else if (!(W.norm == TCB_NORM_OPEN && (int32_t)node == -1)) atomicOr(W.err, kErrBadNode);
            sids[out * L + (L - 1)] = (uint8_t)(h & 255u);
            uint32_t r = h >> 8;
            for (int lv = L - 2; lv >= 0; --lv) {
                if (r >= (uint32_t)width) {            // corrupt back-pointer: never read past the request
                    atomicOr(W.err, kErrBadNode);
                    break;
                }
                const uint32_t hl = W.hist[(size_t)lv * W.S + base + r];
                sids[out * L + lv] = (uint8_t)(hl & 255u);
                r = hl >> 8;
            }
            scores[out] = phi;                         // summed log-probability
            items[out] = item;
        } else {
            for (int lv = 0; lv < L; ++lv) sids[out * L + lv] = 0;
            scores[out] = -INFINITY;
            items[out] = -1;
        }
    }
    __syncthreads();                                   // every wave has read the record
    if (threadIdx.x == 0) {
        counts[orow] = rows;
        ReqRec fr{};
        fr.base = base;
        fr.width = width;
        fr.rows = rows;
        fr.level = L;
        fr.status = kReqFree;
        fr.par = par;
        W.rec[0][req] = fr;
        W.rec[1][req] = fr;
    }
}

// One workgroup per request id: each request's live rows from its own buffer.
__global__ void k_export(WaveDev W, int rp, int32_t *node, float *score, float *phi, int32_t *rows,
                         int32_t *level) {
    const int q = blockIdx.x;
    const ReqRec r = W.rec[rp][q];
    const bool act = r.status == kReqActive;
    if (threadIdx.x == 0) {
        if (rows) rows[q] = act ? r.rows : 0;
        if (level) level[q] = r.level;
    }
    if (!act) return;
    for (int j = threadIdx.x; j < r.rows && j < r.width; j += blockDim.x) {
        const int slot = r.base + j;
        if (node) node[slot] = W.node[r.par][slot];
        if (score) score[slot] = W.score[r.par][slot];
        if (phi) phi[slot] = W.phi[r.par][slot];
    }
}

}  // namespace

// ---------------------------------------------------------------------- launchers
hipError_t launch_clear_wave(const WaveDev &w, hipStream_t s) {
    hipLaunchKernelGGL(k_clear_wave, dim3((w.R + 255) / 256), dim3(256), 0, s, w);
    return hipGetLastError();
}

hipError_t launch_init(const WaveDev &w, const InitBatch &b, hipStream_t s) {
    hipLaunchKernelGGL(k_init, dim3(1), dim3(InitBatch::kMax), 0, s, w, b);
    return hipGetLastError();
}

int tile_mode(const StepReqs &R, bool fuse) {
    bool first = true;
    for (int i = 0; i < R.n; ++i)
        if (R.r[i].step() && R.r[i].level() != 0) first = false;
    if (first) return kTileFirst;
    if (fuse) return kTileFuse;
    return tile_merges(R) ? kTileMerge : kTilePlain;
}

int tile_grid(const WaveDev &w, const StepReqs &R, bool fuse) {
    if (R.n <= 0) return 0;
    const int mode = tile_mode(R, fuse);
    if (mode == kTileFirst) return 8 * ((R.n + first_xcds(R.n) - 1) / first_xcds(R.n));
    if (mode == kTileMerge) return R.n;
    return 8 * ((R.n + 7) / 8) * w.MT;
}

bool tile_merges(const StepReqs &R) {
    for (int i = 0; i < R.n; ++i)
        if (R.r[i].step() && R.r[i].rmax() > kTileRows) return false;
    return true;
}

hipError_t launch_tile(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *logits,
                       int64_t ld, int dtype, bool sampled, hipStream_t s, bool fuse, bool head) {
    if (R.n <= 0) return hipSuccess;
    // 16-byte row pieces: ld a multiple of 4 (fp32) or 8 (bf16) elements, 16-byte base
    const bool vec = t.V == 256 && (ld % (dtype == TCB_F32 ? 4 : 8)) == 0 && ((uintptr_t)logits % 16) == 0;
    const int merge = tile_mode(R, fuse);
    bool head_rows = false;                        // some request's children's logits come from the tile
    if (head)
        for (int i = 0; i < R.n; ++i)
            if (R.r[i].step() && R.r[i].sparse_head()) head_rows = true;
    if (head_rows) {
        // the host sets the flag only past a request's first step, on fp32 16-byte rows,
        // with children normalisation and without sampling
        if (merge == kTileFirst || dtype != TCB_F32 || sampled || !vec || R.hd.hidden == nullptr)
            return hipErrorInvalidValue;
        return launch_tile_f32_head(t, w, rp, R, logits, ld, vec, merge, s);
    }
    if (dtype == TCB_F32) {
        return sampled ? launch_tile_f32_sampled(t, w, rp, R, logits, ld, vec, merge, s)
                       : launch_tile_f32(t, w, rp, R, logits, ld, vec, merge, s);
    } else {
        return sampled ? launch_tile_bf16_sampled(t, w, rp, R, logits, ld, vec, merge, s)
                       : launch_tile_bf16(t, w, rp, R, logits, ld, vec, merge, s);
    }
}

bool merged_in_tile(const StepReqs &R, bool fuse) {
    const int mode = tile_mode(R, fuse);
    return mode == kTileFirst || mode == kTileMerge;
}

hipError_t launch_merge(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, bool in_tile,
                        hipStream_t s) {
    if (R.n <= 0 || in_tile) return hipSuccess;                   // merged inside the tile kernel
    hipLaunchKernelGGL(k_merge, dim3(R.n), dim3(kThreads), 0, s, t, w, rp, R);
    return hipGetLastError();
}

hipError_t launch_finalize(const TrieDev &t, const WaveDev &w, int rp, const FinBatch &b, uint8_t *sids,
                           float *scores, int64_t *items, int32_t *counts, hipStream_t s) {
    hipLaunchKernelGGL(k_finalize, dim3(b.n), dim3(256), 0, s, t, w, rp, b, sids, scores, items, counts);
    return hipGetLastError();
}

hipError_t launch_export(const WaveDev &w, int rp, int32_t *node, float *score, float *phi, int32_t *rows,
                         int32_t *level, hipStream_t s) {
    hipLaunchKernelGGL(k_export, dim3(w.R), dim3(256), 0, s, w, rp, node, score, phi, rows, level);
    return hipGetLastError();
}



}  // namespace tcb
