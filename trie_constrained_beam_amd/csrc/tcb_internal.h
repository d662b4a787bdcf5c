// Internal layouts shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tcb.h"

namespace tcb {

// --------------------------------------------------------------------- tile shapes
// One beam row is held by 16 lanes (one DPP row of a wave64): lane j of the group
// holds 16 of the row's 256 codes, so a wave holds 4 rows and a workgroup of
// kWaves waves holds a tile of kTileRows consecutive rows of one request.
constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;                 // 1024
constexpr int kRowsPerWave = 4;
constexpr int kTileRows = kWaves * kRowsPerWave;      // 64
constexpr int kMaxTilesPerReq = TCB_MAX_WIDTH / kTileRows;
// Request-wide score bins: a candidate of score s falls in bin
// min(kBins - 1, floor((s_ref - s) * kBinRes)), s_ref = the request's best row score
// before the step. No candidate beats s_ref (log-probabilities are <= 0), so every
// tile of the request bins identically without communicating; a lower bin always
// holds strictly higher scores.
constexpr int kBins = 1024;
constexpr float kBinRes = 32.0f;                      // bins per nat: 32 nats of range
static_assert(kBins == kThreads, "one bin per thread in the scans");
constexpr int kTileCap = 4096;                        // candidates a tile keeps (its region)
constexpr int kMergeCap = 4096;                       // candidates the merge stages in LDS
constexpr int kWinCap = 1024;                         // candidates a tile's window merge stages
static_assert(kTileCap >= TCB_MAX_WIDTH, "a tile's exact path keeps up to n_i candidates");
static_assert(kMergeCap % kThreads == 0, "whole rounds of the workgroup");
static_assert(kMergeCap >= TCB_MAX_WIDTH, "the exact merge path stages up to n_i survivors");
constexpr int kSelBins = 1024;                        // bins of the exact selection

// request status
constexpr int kReqFree = 0;
constexpr int kReqActive = 1;

// sticky device error bits
constexpr uint32_t kErrNonFinite = 1u;
constexpr uint32_t kErrBadNode = 2u;
constexpr uint32_t kErrInternal = 4u;
constexpr uint32_t kInfoMergeSpill = 0x100u;   // a merge used its exact (slow) path
constexpr uint32_t kInfoTileExact = 0x200u;    // a tile used its exact (slow) path

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
    int32_t rows;                  // live rows
    int32_t level;                 // steps taken (== L: finished)
    int32_t status;                // kReqFree / kReqActive
    int32_t par;                   // which node/score buffer holds the live rows
    int32_t pad[2];
};

struct alignas(16) Cand {          // a tile's kept candidate, one 16-byte store / load
    float s;                       // selection key: the beam score (sampled steps: the perturbed key)
    uint32_t f;                    // flat index r * 256 + c within the request
    int32_t n;                     // child node id
    float phi;                     // summed log-probability (equal to s at temperature 0)
};

// A row's child set as the next step reads it with the row (written where the row is made,
// so the step needs no dependent trie load): the 256-bit child mask of the row's node (at
// depths stored with masks), its first child id and the end of its child range.
struct alignas(16) RowInfo {       // 48 bytes: three 16-byte pieces
    uint32_t mask[8];
    uint32_t cb, ce, pad[2];
};

struct WaveDev {
    int32_t *node[2];              // [S] trie node of each slot's row (ping-pong per request)
    float *score[2];               // [S] selection key of the row (ping-pong per request)
    float *phi[2];                 // [S] summed log-probability of the row (= score at T = 0)
    int32_t *parent_slot;          // [S] parent slot at the request's last step
    uint32_t *hist;                // [L][S] back-pointer (r << 8) | c per level
    ReqRec *rec[2];                // [R] request records; a step reads one, writes the other
    // kept candidates of every tile and their cumulative counts by bin, one buffer per step
    // parity (level & 1 of the step that wrote them), so that a step's tiles can merge the
    // previous step's candidates while writing their own
    Cand *cand[2];                 // [R][MT][CAPT]
    uint16_t *tcum[2];             // [R][MT][kBins]
    RowInfo *rinfo;                // [S] child sets of rows made by a first step (ReqArg::rows_info)
    float *lmx;                    // [S][256] logits computed by the SID-range lm_head
    uint32_t *err;                 // sticky error / info bits
    // phase trace of this launch (diagnostics; nullptr: off): kTraceSlots words per
    // workgroup, word 0 = 1 + the XCD it ran on, word i > 0 = the real-time clock when the
    // workgroup passed phase mark i (0 = never)
    uint64_t *trace;
    int32_t S, R, MT, CAPT, Bmax, norm, validate, pad;
};
constexpr int kTraceSlots = TCB_TRACE_SLOTS;

// --------------------------------------------------------------------- step arguments
// What the host knows of every request it steps, passed by value so a kernel's first
// loads need no device-side lookup. Only the live-row count stays on the device.
struct ReqArg {
    int32_t base_flags;            // first slot (< 2^24) | gather << 24 | sparse head << 25 | merge pending << 26
                                   // | rows carry their child sets << 27
    uint32_t bits;                 // width | rmax << 13 | level << 26 | pre << 29 | step << 30 | par << 31
    __host__ __device__ int base() const { return base_flags & 0xFFFFFF; }
    __host__ __device__ bool gather() const { return (base_flags >> 24) & 1; }        // children's sectors only
    __host__ __device__ bool sparse_head() const { return (base_flags >> 25) & 1; }   // lm_head: children's pieces only
    // the request's previous step left its merge to this step's tile kernel
    __host__ __device__ bool pending() const { return (base_flags >> 26) & 1; }
    // the request's rows were made by a first-step kernel, which stored each row's child set
    // in WaveDev::rinfo
    __host__ __device__ bool rows_info() const { return (base_flags >> 27) & 1; }
    __host__ __device__ int width() const { return (int)(bits & 0x1FFFu); }
    __host__ __device__ int rmax() const { return (int)((bits >> 13) & 0x1FFFu); }   // bound on live rows
    __host__ __device__ int level() const { return (int)((bits >> 26) & 0x7u); }
    __host__ __device__ bool prefilter() const { return (bits >> 29) & 1u; }        // sample-bound pruning
    __host__ __device__ bool step() const { return (bits >> 30) & 1u; }
    __host__ __device__ int par() const { return (int)(bits >> 31); }                // node/score buffer
    // the same request as its previous step saw it (one level up, the other buffer)
    __host__ __device__ ReqArg prev_step() const {
        ReqArg p = *this;
        p.bits = (bits & ~((7u << 26) | (1u << 31))) | ((uint32_t)(level() - 1) << 26) | ((uint32_t)(par() ^ 1) << 31);
        return p;
    }
};
static_assert(TCB_MAX_WIDTH < (1 << 13) && TCB_MAX_L <= 8, "ReqArg field widths");
// The tile kernel's prefilter pays off only where rows have many children: it is used
// at depths whose nodes have at least this many children on average (results do not
// depend on it).
constexpr int kPrefilterFanout = 64;
constexpr int kArgReqs = 400;      // requests per launch (the arguments stay under 4 KiB)
// Where a step writes the requests it brings to depth L (row = request id), in the layouts
// of the finalize outputs; sids == nullptr: nowhere (they wait for a finalize call).
struct StepFin {
    uint8_t *sids;                 // [R][Bmax][L]
    float *scores;                 // [R][Bmax]
    int64_t *items;                // [R][Bmax]
    int32_t *counts;               // [R]
};
// The SID-range lm_head's operands, for requests whose argument carries the sparse-head flag:
// the tile kernel computes their rows' logits itself, only for the rows' children.
struct StepHead {
    const uint16_t *hidden;        // bf16 [slots][ld], row = slot
    const uint16_t *weight;        // bf16 [L][256][H]
    int64_t ld;                    // elements between hidden rows (ld % 8 == 0)
    int32_t H;                     // hidden size (H % 128 == 0)
    int32_t pad;
};
struct StepReqs {
    int32_t n;                     // request ids q0 .. q0 + n - 1
    int32_t q0;
    float inv_temp;                // sampled steps: 1 / temperature
    int32_t pad;
    double inv_temp_d;             //                the same in float64
    uint64_t seed;                 //                noise seed
    StepFin fin;
    StepHead hd;                   // lm_head steps: the children-only head's operands
    ReqArg r[kArgReqs];
};
static_assert(sizeof(StepReqs) <= 4096 - 256, "kernel arguments stay under 4 KiB");

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
    int32_t base[kMax], width[kMax], par[kMax];   // host copies of the record's fixed fields
};

// The tile kernel of one logits type and sampling mode (compiled in its own translation
// unit) in one of the modes above; vec: rows read as 16-byte pieces.
#define TCB_TILE_LAUNCHER(name)                                                                              \
    hipError_t name(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *logits, int64_t ld, \
                    bool vec, int mode, hipStream_t s)
TCB_TILE_LAUNCHER(launch_tile_f32);
TCB_TILE_LAUNCHER(launch_tile_bf16);
TCB_TILE_LAUNCHER(launch_tile_f32_sampled);
TCB_TILE_LAUNCHER(launch_tile_bf16_sampled);
// fp32 rows from the dense lm_head, and in-tile children-only logits for the requests with
// the sparse-head flag (children normalisation, 16-byte pieces, no sampling)
TCB_TILE_LAUNCHER(launch_tile_f32_head);

// The kernel launch_tile uses for one launch of R: kTileFirst when every stepped request
// is at its first step (one row each; merged inside the kernel), else kTileFuse when
// pending merges come first, kTileMerge when every request fits one tile (merged inside
// the kernel), kTilePlain otherwise (k_merge or the next step merges).
enum { kTilePlain = 0, kTileMerge = 1, kTileFuse = 2, kTileFirst = 3 };
// How many XCDs take the requests of a first-step launch of n requests (at most 16 per XCD
// of 32 CUs): the requests go to the workgroups b with (b - 1) mod 8 < first_xcds(n). After
// the GPU has been idle (a decode's first launch often follows such a gap) the XCDs start a
// launch's workgroups up to about 4 us apart, XCDs 0 and 1 first, and workgroup b then runs
// on XCD (b - 1) mod 8; behind other work the XCDs start together and the offset differs
// (all measured with the phase trace). Only the time depends on this.
__host__ __device__ inline int first_xcds(int n) {
    const int x = (n + 15) / 16;
    return x < 2 ? 2 : x > 8 ? 8 : x;
}
int tile_mode(const StepReqs &R, bool fuse);
// workgroups of the tile kernel launch_tile would launch for R (phase-trace layout)
int tile_grid(const WaveDev &w, const StepReqs &R, bool fuse);

hipError_t launch_clear_wave(const WaveDev &w, hipStream_t s);
hipError_t launch_init(const WaveDev &w, const InitBatch &b, hipStream_t s);
// A step is the tile kernel followed by the per-request merge kernel; with the SID-range
// lm_head, the lm_head kernel first writes the logits to WaveDev::lmx.
// fuse: some request of R has pending() set; the tile kernel then first does that request's
// previous merge (redundantly in each of its tiles, each keeping its own 64 rows)
// head: an lm_head step (R.hd set); requests with the sparse-head flag then get their
// children's logits computed in the tile kernel, never at their first step
hipError_t launch_tile(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *logits,
                       int64_t ld, int dtype, bool sampled, hipStream_t s, bool fuse = false, bool head = false);
hipError_t launch_lmhead(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, const void *hidden,
                         int64_t ld, int H, const void *weight, float *out, hipStream_t s);
// true when every stepped request of R has at most kTileRows rows: a tile kernel launched
// without a pending merge (fuse false) then merges each request itself
bool tile_merges(const StepReqs &R);
// whether launch_tile(..., fuse) merged the requests of R inside the tile kernel (first-step
// and one-tile launches); a launch that first does pending merges (fuse) leaves this step's
// candidates in memory for k_merge or the next step, whatever the requests' widths
bool merged_in_tile(const StepReqs &R, bool fuse);
// k_merge over the requests of R, unless in_tile (the tile kernel merged them already)
hipError_t launch_merge(const TrieDev &t, const WaveDev &w, int rp, const StepReqs &R, bool in_tile,
                        hipStream_t s);
hipError_t launch_finalize(const TrieDev &t, const WaveDev &w, int rp, const FinBatch &b,
                           uint8_t *sids, float *scores, int64_t *items, int32_t *counts,
                           hipStream_t s);
hipError_t launch_export(const WaveDev &w, int rp, int32_t *node, float *score, float *phi, int32_t *rows,
                         int32_t *level, hipStream_t s);

}  // namespace tcb
