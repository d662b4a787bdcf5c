// Host-side object layouts of libtcb.
#pragma once

#include <string>
#include <utility>
#include <array>
#include <vector>

#include "tcb_internal.h"

struct tcb_trie {
    int32_t L = 0, V = 0, mask_depths = 0;
    int64_t n_items = 0, n_distinct = 0;
    std::vector<int64_t> nodes_per_depth;  // [L+1]
    std::vector<int64_t> off;              // [L+2]
    std::vector<uint32_t> child_begin;     // [off[L] + 1]
    std::vector<uint8_t> child_code;       // [total nodes]
    std::vector<int32_t> leaf_item;        // [n_distinct]
    std::vector<uint32_t> mask;            // [off[mask_depths] * 8]
    std::vector<uint8_t> image;            // device image, uploaded as one copy
    size_t o_child_begin = 0, o_child_code = 0, o_leaf = 0, o_mask = 0, image_bytes = 0;
    void *d_image = nullptr;               // caller-owned, set by tcb_trie_upload
    std::vector<uint8_t> codes;            // leaf codes for single-pass scoring (built on demand)
    void *d_codes = nullptr;               // caller-owned, set by tcb_trie_upload_codes
};

struct tcb_beams {
    struct Req {
        bool used = false;
        bool pending = false;              // its last step's merge is deferred to its next step
        bool rinfo = false;                // its rows carry their child sets (made by a first step)
        int32_t base = 0, width = 0, level = 0;
    };
    tcb::TrieDev tdev{};
    tcb::WaveDev w{};
    int32_t L = 0, V = 0;
    uint32_t prefilter_levels = 0;         // bit d: the tile kernel prefilters rows at depth d
    uint32_t gather_levels[3] = {0, 0, 0}; // bit d: fp32 / bf16 rows at depth d read children's sectors only
    int32_t read_mode = TCB_READ_AUTO;
    uint32_t sparse_head_levels = 0;       // bit d: the lm_head computes only children's pieces at depth d
    int64_t depth_nodes[TCB_MAX_L + 1] = {};   // trie nodes per depth: a bound on any request's rows
    int rp = 0;                            // which request-record buffer is current
    int64_t steps = 0;
    std::vector<Req> reqs;
    std::vector<std::pair<int32_t, int32_t>> free_ranges;  // (start, length), sorted
    // admitted requests whose initial device state (record, root row) is not written yet:
    // their first step does not read it, so it is written only if something else would
    // read it first (export, finalize); (request id, slot base, width)
    std::vector<std::array<int32_t, 3>> pending_init;
    // finalize staging inside the workspace
    uint8_t *d_fin_sids = nullptr;
    float *d_fin_scores = nullptr;
    int64_t *d_fin_items = nullptr;
    int32_t *d_fin_counts = nullptr;
    // where a step writes the requests it finishes (tcb_beams_set_finish_outputs); none if null
    tcb::StepFin fin{};
    // a step's merge deferred into the next step's tile kernel: its launch arguments and
    // request-record buffer, launched as k_merge instead if something else reads state first
    bool merge_pending = false;
    int deferred_rp = 0;
    std::vector<tcb::StepReqs> deferred;
    // optional kernel timing: 4 events per step (before the lm_head, before the tile kernel,
    // before the merge, after the merge)
    std::vector<hipEvent_t> events;
    int32_t timing_cap = 0, timing_used = 0, timing_repeat = 1;
    // optional phase trace (tcb_beams_set_trace): launches append kTraceSlots words per
    // workgroup to trace_buf while they fit; trace_log holds (kind, level, grid, offset)
    uint64_t *trace_buf = nullptr;
    int64_t trace_cap = 0, trace_used = 0;
    std::vector<int32_t> trace_log;
    ~tcb_beams() {
        for (auto e : events) (void)hipEventDestroy(e);
    }
};

namespace tcb_host {
tcb_status set_error(tcb_status code, const std::string &msg);
}

tcb_status tcb_trie_build_impl(const uint8_t *sids, int64_t n_items, int32_t L, int32_t V,
                               int32_t mask_depths, tcb_trie **out);
