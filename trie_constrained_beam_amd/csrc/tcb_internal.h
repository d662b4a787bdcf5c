// Internal layouts shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tcb.h"

namespace tcb {

// --------------------------------------------------------------------- tile shapes
// expand: one workgroup of kTileWaves wave64s handles kTileRows consecutive rows of
// one request; wave w takes rows w, w + kTileWaves, ... of the tile.
constexpr int kTileWaves = 8;
constexpr int kRowsPerWave = 4;
constexpr int kTileRows = kTileWaves * kRowsPerWave;   // 32
constexpr int kExpandThreads = kTileWaves * 64;        // 512
// merge: one workgroup per request
constexpr int kMergeThreads = 1024;
constexpr int kMergeCap = 4096;     // candidates staged in LDS by the merge
constexpr int kSelBins = 1024;      // histogram bins of the exact selection fallback
constexpr int kMaxTilesPerReq = TCB_MAX_WIDTH / kTileRows;
// Request-wide score bins: a candidate of score s falls in bin
// min(kHistBins - 1, floor((s_ref - s) * kHistRes)), s_ref = the request's best row
// score before the step. No candidate beats s_ref (log-probabilities are <= 0), so the
// bins are known to every tile without communication.
constexpr int kHistBins = 512;
constexpr float kHistRes = 32.0f;   // bins per nat: 16 nats of resolution
constexpr int kTileSlack = 512;     // extra tile capacity for the boundary bin

// request status
constexpr int kReqFree = 0;
constexpr int kReqActive = 1;

// sticky device error bits
constexpr uint32_t kErrNonFinite = 1u;
constexpr uint32_t kErrBadNode = 2u;
constexpr uint32_t kErrInternal = 4u;
constexpr uint32_t kInfoMergeSpill = 0x100u;   // merge used its global-memory path

// --------------------------------------------------------------------- device views
struct TrieDev {
    const uint32_t *child_begin;   // [off[L] + 1]
    const uint8_t *child_code;     // [total nodes]
    const int32_t *leaf_item;      // [n leaves]
    const uint32_t *mask;          // [off[mask_depths]][8]
    int32_t L, V, mask_depths, pad;
    uint32_t off[TCB_MAX_L + 2];   // first node id of each depth; off[L+1] = total
};

struct ReqRec {                    // one per request id, 32 bytes
    int32_t base;                  // first slot
    int32_t width;                 // beam width n_i
    int32_t rows;                  // live rows (written by the merge)
    int32_t level;                 // steps taken
    int32_t status;                // kReqFree / kReqActive
    int32_t pad[3];
};

struct WaveDev {
    int32_t *node[2];              // [S] trie node of each slot's row, ping-pong
    float *score[2];               // [S] beam score, ping-pong
    int32_t *parent_slot;          // [S] parent slot at the last step
    uint32_t *hist;                // [L][S] back-pointer (r << 8) | c per level
    ReqRec *rec;                   // [R]
    void *cand;                    // [R][MT][CAPT] 16-byte candidate records kept by each tile
    int32_t *tile_count;           // [R][MT] candidates kept by each tile
    uint16_t *tile_hist;           // [R][MT][kHistBins] score-bin counts of the kept candidates
    uint32_t *err;                 // sticky error / info bits
    int32_t S, R, MT, CAPT, Bmax, norm, validate, pad;
};

// --------------------------------------------------------------------- launchers
struct InitBatch {                 // admitted requests, passed by value
    static constexpr int kMax = 32;
    int32_t n;
    int32_t req[kMax], base[kMax], width[kMax];
};

struct FinBatch {
    static constexpr int kMax = 32;
    int32_t n;
    int32_t req[kMax];
    int32_t out_row[kMax];         // output row of each request in the caller arrays
};

hipError_t launch_clear_wave(const WaveDev &w, hipStream_t s);
hipError_t launch_init(const WaveDev &w, int par, const InitBatch &b, hipStream_t s);
hipError_t launch_expand(const TrieDev &t, const WaveDev &w, int par, int n_req,
                         const void *logits, int64_t ld, int dtype, hipStream_t s);
hipError_t launch_expand_lmhead(const TrieDev &t, const WaveDev &w, int par, int n_req,
                                const void *hidden, int64_t ld, int H, const void *weight,
                                hipStream_t s);
hipError_t launch_merge(const TrieDev &t, const WaveDev &w, int par, int n_req, hipStream_t s);
hipError_t launch_finalize(const TrieDev &t, const WaveDev &w, int par, const FinBatch &b,
                           uint8_t *sids, float *scores, int64_t *items, int32_t *counts,
                           hipStream_t s);
hipError_t launch_export_req(const WaveDev &w, int32_t *rows, int32_t *level, hipStream_t s);

}  // namespace tcb
