// Layouts shared by the host library and the single-pass scoring kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tcb.h"

namespace tcb {

// Users are scored in groups: the group's token tables sit in LDS together
// (kScoreUG users x L levels x 256 codes x 4 bytes = 128 KiB at L = 4), and one
// v_mfma_f32_32x32x16_bf16 tile holds the group's 32 users x 32 SIDs.
constexpr int kScoreUGNarrow = 32;            // L <= 4
constexpr int kScoreUGWide = 16;              // 5 <= L <= 8
// LDS for the tables: levels padded to 4 (L <= 4) or 8 with zero rows, so every SID
// adds the same number of terms; a row of (depth, code) holds the group's users, padded
// by 4 floats at L <= 4 (a row stride of an odd multiple of 16 bytes spreads the lanes'
// random codes over the LDS banks)
constexpr int kScoreStrideNarrow = kScoreUGNarrow + 4;    // 36 floats, 4 levels
constexpr int kScoreStrideWide = kScoreUGWide;            // 16 floats, 8 levels
constexpr int kScoreTableFloats = kScoreStrideNarrow * (4 * 256 + 1);   // + a row of -inf
static_assert(kScoreStrideWide * (8 * 256 + 1) <= kScoreTableFloats, "wide tables fit the same LDS");
constexpr int kScoreGroup = 16;               // SIDs per group (one DPP row)
constexpr int kScoreBlock = 256;              // SIDs per block (8 MFMA tiles)
constexpr int kScanWaves = 8;
constexpr int kScanThreads = kScanWaves * 64;
constexpr int kScanWGs = 256;                 // one persistent workgroup per CU and user group
constexpr int kSelectThreads = 1024;
constexpr int kRescoreThreads = 256;
constexpr int kRescoreWGs = 16;                // workgroups per user that rescore its picked groups
constexpr int kScoreCand = kScoreGroup * TCB_SCORE_MAX_K;   // candidates of one selection stage

inline int score_ug(int L) { return L <= 4 ? kScoreUGNarrow : kScoreUGWide; }

struct ScoreDev {
    const void *codes;          // [n] leaf codes: u32 (L <= 4) or u64, byte d = code at depth d
    const int32_t *leaf_item;   // [n] lowest catalog row of each SID
    const float *table_in;      // [U][L][V] caller table
    float *table;               // [groups][L][256][UG] normalised, user-minor (written by the scan)
    const uint16_t *user_vec;   // [U][D] bf16, or null
    const uint16_t *emb;        // [n][D] bf16 in leaf order, or null
    float *gmax;                // [groups][ceil(n / 256)][UG][16] best score of each 16-SID group
    float *bmax;                // [groups][UG][ceil(n / 256)] best score of each 256-SID block
    float *lse_part;            // [groups][kScanWGs][UG][2] (max, sum of exp) per scan workgroup
    int32_t *pick;              // [U][TCB_SCORE_MAX_K] group ids chosen for rescoring, ascending
    int32_t *npick;             // [U] their number
    float *cand;                // [U][kScoreCand] rescored scores of the picked groups' SIDs
    int32_t *out_leaf;          // [U][K]
    int32_t *out_item;          // [U][K] or null
    float *out_score;           // [U][K]
    float *out_lse;             // [U] or null
    int64_t n;                  // valid SIDs (leaves)
    int32_t L, V, U, D, K, kind, groups, ug;
    float w;
};

struct ScoreLayout {
    size_t table = 0, gmax = 0, bmax = 0, lse = 0, pick = 0, npick = 0, cand = 0, total = 0;
};
ScoreLayout score_layout(int L, int64_t n, int max_users);

// ev: null, or 3 events recorded before the scan kernel, before the selection kernels and after
hipError_t launch_score(const ScoreDev &a, hipStream_t s, const hipEvent_t *ev);

// The static scratch of tcb_score_catalog_static on the current device: its address (taken
// once per device) and size.
constexpr size_t kStaticScoreScratch = TCB_SCORE_STATIC_SCRATCH;
static_assert(TCB_SCORE_STATIC_SCRATCH == (64u << 20), "header and library agree");
constexpr int kMaxScratchDevices = 64;
hipError_t static_score_scratch(void **ptr, size_t *bytes);

}  // namespace tcb
