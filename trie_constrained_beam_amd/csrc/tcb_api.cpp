// libtcb host ABI: argument validation, workspace carving, slot and request-id
// allocation, and kernel launches on the caller's stream.
//
// Scheduling follows flashrec 0.1.0, Features > Decoding ("Scheduling"): requests are
// admitted between steps under a beam-row slot budget, and the rows of every admitted
// request share each step. Requests never compete for survivors.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "tcb_host.h"

namespace tcb_host {
thread_local std::string g_last_error;

tcb_status set_error(tcb_status code, const std::string &msg) {
    g_last_error = msg;
    return code;
}
}  // namespace tcb_host

using tcb_host::set_error;

namespace {

tcb_status hip_fail(hipError_t e, const char *what) {
    return set_error(TCB_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
    int32_t MT = 0, CAPT = 0;
    size_t node[2]{}, score[2]{}, phi[2]{}, parent_slot = 0, hist = 0, rec[2]{}, rinfo = 0;
    size_t cand = 0, tcum = 0, lmx = 0, err = 0;
    size_t fin_sids = 0, fin_scores = 0, fin_items = 0, fin_counts = 0, total = 0;
};

Layout make_layout(int L, int S, int R, int Bmax) {
    Layout l;
    l.MT = (Bmax + tcb::kTileRows - 1) / tcb::kTileRows;
    l.CAPT = tcb::kTileCap;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    const size_t s = (size_t)S, r = (size_t)R;
    l.node[0] = take(s * 4);
    l.node[1] = take(s * 4);
    l.score[0] = take(s * 4);
    l.score[1] = take(s * 4);
    l.phi[0] = take(s * 4);
    l.phi[1] = take(s * 4);
    l.parent_slot = take(s * 4);
    l.hist = take((size_t)L * s * 4);
    l.rinfo = take(s * sizeof(tcb::RowInfo));
    l.rec[0] = take(r * sizeof(tcb::ReqRec));
    l.rec[1] = take(r * sizeof(tcb::ReqRec));
    const size_t ncand = r * (size_t)l.MT * (size_t)l.CAPT;
    l.cand = take(2 * ncand * sizeof(tcb::Cand));
    l.tcum = take(2 * r * (size_t)l.MT * tcb::kBins * 2);
    l.lmx = take(s * 256 * 4);
    l.err = take(256);
    l.fin_sids = take(r * (size_t)Bmax * (size_t)L);
    l.fin_scores = take(r * (size_t)Bmax * 4);
    l.fin_items = take(r * (size_t)Bmax * 8);
    l.fin_counts = take(r * 4);
    l.total = o;
    return l;
}

int n_req_hw(const tcb_beams *b) {
    int n = 0;
    for (int i = 0; i < (int)b->reqs.size(); ++i)
        if (b->reqs[(size_t)i].used) n = i + 1;
    return n;
}

bool take_slots(std::vector<std::pair<int32_t, int32_t>> &fr, int32_t width, int32_t *base) {
    for (size_t i = 0; i < fr.size(); ++i) {
        if (fr[i].second >= width) {
            *base = fr[i].first;
            fr[i].first += width;
            fr[i].second -= width;
            if (fr[i].second == 0) fr.erase(fr.begin() + (long)i);
            return true;
        }
    }
    return false;
}

void give_slots(std::vector<std::pair<int32_t, int32_t>> &fr, int32_t base, int32_t width) {
    auto it = std::lower_bound(fr.begin(), fr.end(), std::make_pair(base, 0));
    it = fr.insert(it, {base, width});
    size_t i = (size_t)(it - fr.begin());
    if (i + 1 < fr.size() && fr[i].first + fr[i].second == fr[i + 1].first) {
        fr[i].second += fr[i + 1].second;
        fr.erase(fr.begin() + (long)i + 1);
    }
    if (i > 0 && fr[i - 1].first + fr[i - 1].second == fr[i].first) {
        fr[i - 1].second += fr[i].second;
        fr.erase(fr.begin() + (long)i);
    }
}

tcb_status read_err(tcb_beams *b, hipStream_t s, uint32_t *err) {
    hipError_t e = hipMemcpyAsync(err, b->w.err, 4, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "read error flags");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    return TCB_OK;
}

tcb_status err_status(uint32_t err) {
    if (err & tcb::kErrNonFinite) return set_error(TCB_E_NONFINITE, "a non-finite logit was read");
    if (err & tcb::kErrBadNode) return set_error(TCB_E_DEVICE, "a row held a node outside its depth");
    if (err & tcb::kErrInternal) return set_error(TCB_E_DEVICE, "internal invariant violated on device");
    return TCB_OK;
}

tcb_status check_finalize_args(tcb_beams *b, int32_t n, const int32_t *req_ids) {
    if (!b || !req_ids || n <= 0) return set_error(TCB_E_ARG, "finalize: bad arguments");
    if (n > b->w.R) return set_error(TCB_E_ARG, "finalize: n exceeds max_requests");
    std::vector<char> seen(b->reqs.size(), 0);
    for (int i = 0; i < n; ++i) {
        const int r = req_ids[i];
        if (r < 0 || r >= (int)b->reqs.size() || !b->reqs[(size_t)r].used)
            return set_error(TCB_E_ARG, "finalize: unknown request id " + std::to_string(r));
        if (seen[(size_t)r]) return set_error(TCB_E_ARG, "finalize: request id repeated");
        seen[(size_t)r] = 1;
        if (b->reqs[(size_t)r].level < b->L)
            return set_error(TCB_E_STATE, "finalize: request " + std::to_string(r) + " is at level " +
                                              std::to_string(b->reqs[(size_t)r].level) + " < L");
    }
    return TCB_OK;
}

// Writes the initial device state of requests admitted since the last step: needed only
// before something other than a step reads request state (a step starts a fresh request
// from its known initial state without reading it).
tcb_status flush_init(tcb_beams *b, hipStream_t s) {
    const auto &p = b->pending_init;
    for (size_t i0 = 0; i0 < p.size(); i0 += tcb::InitBatch::kMax) {
        tcb::InitBatch ib{};
        ib.n = (int32_t)std::min(p.size() - i0, (size_t)tcb::InitBatch::kMax);
        for (int j = 0; j < ib.n; ++j) {
            ib.req[j] = p[i0 + (size_t)j][0];
            ib.base[j] = p[i0 + (size_t)j][1];
            ib.width[j] = p[i0 + (size_t)j][2];
        }
        hipError_t e = tcb::launch_init(b->w, ib, s);
        if (e != hipSuccess) return hip_fail(e, "beam_init launch");
    }
    b->pending_init.clear();
    return TCB_OK;
}

// Highest level among the requests a launch steps (the phase trace's label).
int32_t launch_level(const tcb::StepReqs &R) {
    int32_t lv = 0;
    for (int i = 0; i < R.n; ++i)
        if (R.r[i].step()) lv = std::max(lv, (int32_t)R.r[i].level());
    return lv;
}

// The wave's device view for one launch: with a phase trace armed and room left, the
// launch gets its own region of the trace buffer and an entry in the trace log.
tcb::WaveDev traced(tcb_beams *b, int32_t kind, int32_t level, int32_t grid) {
    tcb::WaveDev w = b->w;
    w.trace = nullptr;
    const int64_t words = (int64_t)grid * tcb::kTraceSlots;
    if (b->trace_buf && grid > 0 && b->trace_used + words <= b->trace_cap) {
        w.trace = b->trace_buf + b->trace_used;
        b->trace_log.insert(b->trace_log.end(), {kind, level, grid, (int32_t)b->trace_used});
        b->trace_used += words;
    }
    return w;
}

// Launches a merge left for the next step's tile kernel as k_merge (before anything other
// than a step reads request state).
tcb_status flush_merge(tcb_beams *b, hipStream_t s) {
    if (!b->merge_pending) return TCB_OK;
    for (const auto &R : b->deferred) {
        // a deferred step merged nothing inside its tile kernel
        const tcb::WaveDev w = traced(b, TCB_TRACE_MERGE, launch_level(R), R.n);
        hipError_t e = tcb::launch_merge(b->tdev, w, b->deferred_rp, R, false, s);
        if (e != hipSuccess) return hip_fail(e, "merge launch");
    }
    for (auto &q : b->reqs) q.pending = false;
    b->merge_pending = false;
    return TCB_OK;
}

tcb_status run_finalize(tcb_beams *b, int32_t n, const int32_t *req_ids, uint8_t *sids,
                        float *scores, int64_t *items, int32_t *counts, hipStream_t s) {
    tcb_status st = flush_merge(b, s);
    if (st) return st;
    st = flush_init(b, s);
    if (st) return st;
    for (int i0 = 0; i0 < n; i0 += tcb::FinBatch::kMax) {
        tcb::FinBatch fb{};
        fb.n = std::min(n - i0, tcb::FinBatch::kMax);
        for (int j = 0; j < fb.n; ++j) {
            const auto &rq = b->reqs[(size_t)req_ids[i0 + j]];
            fb.req[j] = req_ids[i0 + j];
            fb.out_row[j] = i0 + j;
            fb.base[j] = rq.base;
            fb.width[j] = rq.width;
            fb.par[j] = rq.level & 1;      // a step at level t reads buffer t & 1 and writes the other
        }
        hipError_t e = tcb::launch_finalize(b->tdev, b->w, b->rp, fb, sids, scores, items, counts, s);
        if (e != hipSuccess) return hip_fail(e, "finalize launch");
    }
    return TCB_OK;
}

void release(tcb_beams *b, int32_t n, const int32_t *req_ids) {
    for (int i = 0; i < n; ++i) {
        auto &q = b->reqs[(size_t)req_ids[i]];
        give_slots(b->free_ranges, q.base, q.width);
        q = tcb_beams::Req{};
    }
}

}  // namespace

extern "C" {

const char *tcb_last_error(void) { return tcb_host::g_last_error.c_str(); }

const char *tcb_version(void) { return "tcb 0.1.0 gfx950"; }

// --------------------------------------------------------------------------- trie
tcb_status tcb_build_trie(const uint8_t *sids, int64_t n_items, int32_t L, int32_t V,
                          int32_t mask_depths, tcb_trie **out) {
    if (n_items >= (int64_t)0x7FFFFFFF) return set_error(TCB_E_ARG, "build_trie: n_items >= 2^31");
    return tcb_trie_build_impl(sids, n_items, L, V, mask_depths, out);
}

tcb_status tcb_trie_info(const tcb_trie *t, tcb_trie_info_t *out) {
    if (!t || !out) return set_error(TCB_E_ARG, "trie_info: null pointer");
    std::memset(out, 0, sizeof(*out));
    out->L = t->L;
    out->V = t->V;
    out->mask_depths = t->mask_depths;
    out->n_items = t->n_items;
    out->n_distinct = t->n_distinct;
    for (int d = 0; d <= t->L; ++d) out->nodes_per_depth[d] = t->nodes_per_depth[(size_t)d];
    for (int d = 0; d <= t->L + 1; ++d) out->node_offset[d] = t->off[(size_t)d];
    out->device_bytes = t->image_bytes;
    return TCB_OK;
}

tcb_status tcb_trie_host_arrays(const tcb_trie *t, const uint32_t **child_begin,
                                const uint8_t **child_code, const int32_t **leaf_item) {
    if (!t) return set_error(TCB_E_ARG, "trie_host_arrays: null trie");
    if (child_begin) *child_begin = t->child_begin.data();
    if (child_code) *child_code = t->child_code.data();
    if (leaf_item) *leaf_item = t->leaf_item.data();
    return TCB_OK;
}

tcb_status tcb_trie_upload(tcb_trie *t, void *d_buf, size_t bytes, void *stream) {
    if (!t || !d_buf) return set_error(TCB_E_ARG, "trie_upload: null pointer");
    if (bytes < t->image_bytes) return set_error(TCB_E_WORKSPACE, "trie_upload: buffer too small");
    if (((uintptr_t)d_buf & 255) != 0) return set_error(TCB_E_WORKSPACE, "trie_upload: buffer not 256-byte aligned");
    hipError_t e = hipMemcpyAsync(d_buf, t->image.data(), t->image_bytes, hipMemcpyHostToDevice,
                                  (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "trie_upload copy");
    t->d_image = d_buf;
    return TCB_OK;
}

void tcb_trie_destroy(tcb_trie *t) { delete t; }

// --------------------------------------------------------------------------- wave
tcb_status tcb_beams_workspace_bytes(const tcb_trie *t, int32_t max_slots, int32_t max_requests,
                                     int32_t max_width, size_t *bytes) {
    if (!t || !bytes) return set_error(TCB_E_ARG, "workspace_bytes: null pointer");
    if (max_slots <= 0 || max_requests <= 0 || max_width <= 0 || max_width > TCB_MAX_WIDTH)
        return set_error(TCB_E_ARG, "workspace_bytes: sizes out of range");
    if (max_slots >= (1 << 24)) return set_error(TCB_E_ARG, "workspace_bytes: max_slots >= 2^24");
    *bytes = make_layout(t->L, max_slots, max_requests, max_width).total;
    return TCB_OK;
}

tcb_status tcb_beams_create(const tcb_trie *t, int32_t max_slots, int32_t max_requests,
                            int32_t max_width, int32_t norm, void *d_ws, size_t ws_bytes,
                            void *stream, tcb_beams **out) {
    if (!t || !d_ws || !out) return set_error(TCB_E_ARG, "beams_create: null pointer");
    if (!t->d_image) return set_error(TCB_E_STATE, "beams_create: trie not uploaded");
    if (norm != TCB_NORM_CHILDREN && norm != TCB_NORM_LEVEL && norm != TCB_NORM_OPEN)
        return set_error(TCB_E_ARG, "beams_create: bad norm");
    size_t need = 0;
    tcb_status st = tcb_beams_workspace_bytes(t, max_slots, max_requests, max_width, &need);
    if (st) return st;
    if (ws_bytes < need) return set_error(TCB_E_WORKSPACE, "beams_create: workspace too small");
    if (((uintptr_t)d_ws & 255) != 0) return set_error(TCB_E_WORKSPACE, "beams_create: workspace not 256-byte aligned");
    *out = nullptr;
    tcb_beams *b = new (std::nothrow) tcb_beams();
    if (!b) return set_error(TCB_E_ARG, "beams_create: out of host memory");
    b->L = t->L;
    b->V = t->V;
    for (int d = 0; d < t->L; ++d)
        if (t->nodes_per_depth[(size_t)d + 1] >= (int64_t)tcb::kPrefilterFanout * t->nodes_per_depth[(size_t)d])
            b->prefilter_levels |= 1u << d;
    for (int d = 0; d <= t->L; ++d) b->depth_nodes[d] = t->nodes_per_depth[(size_t)d];
    // gather at depths where a row's children touch under half of its 64-byte sectors
    // (16 of them for fp32 rows, 8 for bf16), by the depth's mean fanout
    for (int d = 0; d < t->L; ++d) {
        const double fan = (double)t->nodes_per_depth[(size_t)d + 1] / (double)t->nodes_per_depth[(size_t)d];
        for (int k = 0; k < 2; ++k) {
            const double sectors = k == 0 ? 16.0 : 8.0;
            if (1.0 - std::pow(1.0 - 1.0 / sectors, fan) < 0.5) b->gather_levels[k] |= 1u << d;
        }
        // children-only lm_head (in the tile kernel) where rows have at most two children on
        // average: each child costs the tile one dot product over H on the vector ALUs and a
        // weight row read from L2, so it pays only where the dense head's 256 codes per row
        // are almost all masked off
        if (fan <= 2.0) b->sparse_head_levels |= 1u << d;
    }
    const uint8_t *img = (const uint8_t *)t->d_image;
    b->tdev.child_begin = (const uint32_t *)(img + t->o_child_begin);
    b->tdev.child_code = img + t->o_child_code;
    b->tdev.leaf_item = (const int32_t *)(img + t->o_leaf);
    b->tdev.mask = (const uint32_t *)(img + t->o_mask);
    b->tdev.L = t->L;
    b->tdev.V = t->V;
    b->tdev.mask_depths = t->mask_depths;
    for (int d = 0; d <= t->L + 1; ++d) b->tdev.off[d] = (uint32_t)t->off[(size_t)d];

    const Layout l = make_layout(t->L, max_slots, max_requests, max_width);
    uint8_t *ws = (uint8_t *)d_ws;
    auto &w = b->w;
    for (int p = 0; p < 2; ++p) {
        w.node[p] = (int32_t *)(ws + l.node[p]);
        w.score[p] = (float *)(ws + l.score[p]);
        w.phi[p] = (float *)(ws + l.phi[p]);
    }
    w.parent_slot = (int32_t *)(ws + l.parent_slot);
    w.hist = (uint32_t *)(ws + l.hist);
    w.rinfo = (tcb::RowInfo *)(ws + l.rinfo);
    w.rec[0] = (tcb::ReqRec *)(ws + l.rec[0]);
    w.rec[1] = (tcb::ReqRec *)(ws + l.rec[1]);
    {
        const size_t ncand = (size_t)max_requests * (size_t)l.MT * (size_t)l.CAPT;
        const size_t ntc = (size_t)max_requests * (size_t)l.MT * tcb::kBins;
        w.cand[0] = (tcb::Cand *)(ws + l.cand);
        w.cand[1] = w.cand[0] + ncand;
        w.tcum[0] = (uint16_t *)(ws + l.tcum);
        w.tcum[1] = w.tcum[0] + ntc;
    }
    w.lmx = (float *)(ws + l.lmx);
    w.err = (uint32_t *)(ws + l.err);
    w.S = max_slots;
    w.R = max_requests;
    w.MT = l.MT;
    w.CAPT = l.CAPT;
    w.Bmax = max_width;
    w.norm = norm;
    w.validate = 0;
    b->d_fin_sids = ws + l.fin_sids;
    b->d_fin_scores = (float *)(ws + l.fin_scores);
    b->d_fin_items = (int64_t *)(ws + l.fin_items);
    b->d_fin_counts = (int32_t *)(ws + l.fin_counts);
    b->reqs.assign((size_t)max_requests, tcb_beams::Req{});
    b->free_ranges.push_back({0, max_slots});
    hipError_t e = tcb::launch_clear_wave(w, (hipStream_t)stream);
    if (e != hipSuccess) {
        delete b;
        return hip_fail(e, "beams_create clear");
    }
    *out = b;
    return TCB_OK;
}

tcb_status tcb_beam_init(tcb_beams *b, int32_t n, const int32_t *widths, int32_t *out_req_ids,
                         int32_t *out_slot_base, void *stream) {
    if (!b || !widths || n <= 0) return set_error(TCB_E_ARG, "beam_init: bad arguments");
    for (int i = 0; i < n; ++i)
        if (widths[i] < 1 || widths[i] > b->w.Bmax)
            return set_error(TCB_E_ARG, "beam_init: width " + std::to_string(widths[i]) +
                                            " outside 1..max_width");
    // all-or-nothing: plan on copies, commit only if everything fits
    auto fr = b->free_ranges;
    std::vector<int32_t> ids, bases;
    int next = 0;
    for (int i = 0; i < n; ++i) {
        while (next < (int)b->reqs.size() && b->reqs[(size_t)next].used) ++next;
        if (next >= (int)b->reqs.size())
            return set_error(TCB_E_BUDGET, "beam_init: no free request id");
        int32_t base = 0;
        if (!take_slots(fr, widths[i], &base))
            return set_error(TCB_E_BUDGET, "beam_init: slot budget exhausted");
        ids.push_back(next);
        bases.push_back(base);
        ++next;
    }
    (void)stream;                          // the initial state is written lazily (flush_init)
    for (int i = 0; i < n; ++i) b->pending_init.push_back({ids[(size_t)i], bases[(size_t)i], widths[i]});
    b->free_ranges = fr;
    for (int i = 0; i < n; ++i) {
        auto &q = b->reqs[(size_t)ids[(size_t)i]];
        q.used = true;
        q.base = bases[(size_t)i];
        q.width = widths[i];
        q.level = 0;
        if (out_req_ids) out_req_ids[i] = ids[(size_t)i];
        if (out_slot_base) out_slot_base[i] = bases[(size_t)i];
    }
    return TCB_OK;
}

static tcb_status step_common(tcb_beams *b) {
    for (const auto &q : b->reqs)
        if (q.used && q.level < b->L) return TCB_OK;
    return set_error(TCB_E_STATE, "beam_step: no admitted request is unfinished");
}

static void step_done(tcb_beams *b) {
    b->pending_init.clear();               // every admitted request took its first step
    b->rp ^= 1;
    b->steps++;
    for (auto &q : b->reqs)
        if (q.used && q.level < b->L) {
            q.level++;
            if (q.level == b->L && b->fin.sids) {   // written out by the step itself: released
                give_slots(b->free_ranges, q.base, q.width);
                q = tcb_beams::Req{};
            }
        }
}

}  // extern "C"

// Launch the optional lm_head kernel through `head` (which may launch nothing), the tile
// kernel through `tile`, then the merge kernel. With timing on, HIP events bracket the
// three launches separately.
// The per-request kernel arguments of one step, in launches of up to tcb::kArgReqs ids.
static void step_args(const tcb_beams *b, std::vector<tcb::StepReqs> &out, int dt_index, bool head) {
    const int nr = n_req_hw(b);
    out.clear();
    for (int q0 = 0; q0 < nr; q0 += tcb::kArgReqs) {
        out.emplace_back();
        tcb::StepReqs &R = out.back();
        R.q0 = q0;
        R.n = std::min(nr - q0, tcb::kArgReqs);
        R.fin = b->fin;
        for (int i = 0; i < R.n; ++i) {
            const auto &rq = b->reqs[(size_t)(q0 + i)];
            const bool step = rq.used && rq.level < b->L;
            const uint32_t width = step ? (uint32_t)rq.width : 0u;
            // rows at level t are distinct depth-t prefixes (catalog prefixes unless the wave
            // is unconstrained), at most the beam width
            const bool open = b->w.norm == TCB_NORM_OPEN;
            const int64_t prefixes = rq.level == 0 ? 1 : open ? (int64_t)width : b->depth_nodes[rq.level < b->L ? rq.level : 0];
            const uint32_t rmax = (uint32_t)std::min<int64_t>(width, prefixes);
            const uint32_t level = step ? (uint32_t)rq.level : 0u;
            // a first step has one row, at most V <= 256 candidates: nothing to prefilter
            const uint32_t pre = level == 0 ? 0u : open ? 1u : (b->prefilter_levels >> level) & 1u;
            // gather only the logit sectors that hold a child where rows have few children
            const bool by_level = b->read_mode == TCB_READ_GATHER || (b->read_mode == TCB_READ_AUTO &&
                                                                      (b->gather_levels[dt_index] >> level & 1u));
            // a pending merge comes first in the tile kernel: rows are then read whole, issued
            // before the merge, as their pieces would wait for the merged rows' nodes
            const bool pend = step && rq.pending;
            const bool gather = !open && b->w.norm == TCB_NORM_CHILDREN && step && dt_index < 2 && by_level && !pend;
            // an lm_head step past the first computes only the children's logits where rows
            // have few children, in the tile kernel (no head launch for the request)
            const bool sparse = head && !open && b->w.norm == TCB_NORM_CHILDREN && step && level > 0 &&
                                (b->read_mode == TCB_READ_GATHER ||
                                 (b->read_mode == TCB_READ_AUTO && (b->sparse_head_levels >> level & 1u)));
            const bool rinfo = step && rq.rinfo;
            R.r[i].base_flags = rq.base | (gather ? 1 << 24 : 0) | (sparse ? 1 << 25 : 0) | (pend ? 1 << 26 : 0) |
                                (rinfo ? 1 << 27 : 0);
            R.r[i].bits = width | rmax << 13 | level << 26 | pre << 29 | (step ? 1u : 0u) << 30 | (level & 1u) << 31;
        }
    }
}

// Which per-level gather mask applies to a step: 0 (fp32 rows) or 1 (bf16 rows) when the
// tile kernel reads the rows with 16-byte vector loads, else 2 (never gather).
static int gather_index(const void *logits, int64_t ld, int32_t dtype, int V) {
    const bool vec = V == 256 && (ld % (dtype == TCB_F32 ? 4 : 8)) == 0 && ((uintptr_t)logits % 16) == 0;
    return vec ? (dtype == TCB_F32 ? 0 : 1) : 2;
}

// fuse_ok: this step's kernels can take a pending merge (its tile kernel does it first; no
// kernel before it needs the merged rows); otherwise the pending merge is launched first. A
// step may leave its own merge to the next step.
template <class HeadLaunch, class TileLaunch>
static tcb_status run_step(tcb_beams *b, hipStream_t s, HeadLaunch head, TileLaunch tile, int dt_index,
                           double temperature = 0.0, uint64_t seed = 0, bool sparse_head = false,
                           bool fuse_ok = true) {
    static thread_local std::vector<tcb::StepReqs> args;
    const bool can_defer = true;
    if (!fuse_ok) {
        const tcb_status st = flush_merge(b, s);
        if (st) return st;
    }
    const bool fuse = b->merge_pending;                // this step's tile kernel does those merges
    step_args(b, args, dt_index, sparse_head);
    for (auto &R : args) {
        R.inv_temp_d = temperature > 0.0 ? 1.0 / temperature : 0.0;
        R.inv_temp = (float)R.inv_temp_d;
        R.seed = seed;
    }
    const bool timed = b->timing_used < b->timing_cap;
    hipEvent_t *ev = timed ? &b->events[(size_t)b->timing_used * 4] : nullptr;
    // with timing on, each kernel runs timing_repeat times back to back between its events:
    // within a step every kernel rewrites the same outputs from unchanged inputs
    const int rep = timed ? b->timing_repeat : 1;
    hipError_t e = timed ? hipEventRecord(ev[0], s) : hipSuccess;
    for (int i = 0; i < rep && e == hipSuccess; ++i)
        for (size_t c = 0; c < args.size() && e == hipSuccess; ++c) e = head(args[c]);
    if (e != hipSuccess) return hip_fail(e, "lm_head kernel launch");
    if (timed) e = hipEventRecord(ev[1], s);
    for (int i = 0; i < rep && e == hipSuccess; ++i)
        for (size_t c = 0; c < args.size() && e == hipSuccess; ++c)
            e = tile(traced(b, TCB_TRACE_TILE, launch_level(args[c]), tcb::tile_grid(b->w, args[c], fuse)), args[c],
                     fuse);
    if (e != hipSuccess) return hip_fail(e, "tile kernel launch");
    if (fuse) {
        for (auto &q : b->reqs) q.pending = false;
        b->merge_pending = false;
    }
    // rows made by a first-step kernel carry their child sets into the next step
    for (const auto &R : args) {
        const bool first = tcb::tile_mode(R, fuse) == tcb::kTileFirst;
        for (int i = 0; i < R.n; ++i)
            if (R.r[i].step()) b->reqs[(size_t)(R.q0 + i)].rinfo = first;
    }
    // defer this step's merge to the next step's tile kernel unless a request finishes now
    // or the tile kernel merged every request itself
    bool defer = can_defer;
    for (const auto &q : b->reqs)
        if (q.used && q.level < b->L && q.level + 1 >= b->L) defer = false;
    for (const auto &R : args)
        if (tcb::merged_in_tile(R, fuse)) defer = false;
    if (timed) e = hipEventRecord(ev[2], s);
    if (defer) {
        b->deferred = args;
        b->deferred_rp = b->rp;
        for (auto &q : b->reqs)
            if (q.used && q.level < b->L) q.pending = true;
        b->merge_pending = true;
    } else {
        for (int i = 0; i < rep && e == hipSuccess; ++i)
            for (size_t c = 0; c < args.size() && e == hipSuccess; ++c)
                e = tcb::launch_merge(b->tdev,
                                      tcb::merged_in_tile(args[c], fuse)
                                          ? b->w
                                          : traced(b, TCB_TRACE_MERGE, launch_level(args[c]), args[c].n),
                                      b->rp, args[c], tcb::merged_in_tile(args[c], fuse), s);
    }
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    if (timed) {
        e = hipEventRecord(ev[3], s);
        if (e != hipSuccess) return hip_fail(e, "event record");
        b->timing_used++;
    }
    step_done(b);
    return TCB_OK;
}

extern "C" {

tcb_status tcb_beam_step(tcb_beams *b, const void *d_logits, int64_t ld, int32_t dtype, void *stream) {
    if (!b || !d_logits) return set_error(TCB_E_ARG, "beam_step: null pointer");
    if (dtype != TCB_F32 && dtype != TCB_BF16) return set_error(TCB_E_ARG, "beam_step: bad dtype");
    if (ld < b->V) return set_error(TCB_E_ARG, "beam_step: ld < V");
    tcb_status st = step_common(b);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    return run_step(
        b, s, [](const tcb::StepReqs &) { return hipSuccess; },
        [&](const tcb::WaveDev &w, const tcb::StepReqs &R, bool fuse) {
            return tcb::launch_tile(b->tdev, w, b->rp, R, d_logits, ld, dtype, false, s, fuse);
        },
        gather_index(d_logits, ld, dtype, b->V));
}

tcb_status tcb_beam_step_sampled(tcb_beams *b, const void *d_logits, int64_t ld, int32_t dtype, float temperature,
                                 uint64_t seed, void *stream) {
    if (!b || !d_logits) return set_error(TCB_E_ARG, "beam_step_sampled: null pointer");
    if (dtype != TCB_F32 && dtype != TCB_BF16) return set_error(TCB_E_ARG, "beam_step_sampled: bad dtype");
    if (ld < b->V) return set_error(TCB_E_ARG, "beam_step_sampled: ld < V");
    if (!(temperature > 0.0f) || !std::isfinite(temperature) || !std::isfinite(1.0f / temperature))
        return set_error(TCB_E_ARG, "beam_step_sampled: temperature must be finite and > 0");
    tcb_status st = step_common(b);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    return run_step(
        b, s, [](const tcb::StepReqs &) { return hipSuccess; },
        [&](const tcb::WaveDev &w, const tcb::StepReqs &R, bool fuse) {
            return tcb::launch_tile(b->tdev, w, b->rp, R, d_logits, ld, dtype, true, s, fuse);
        },
        gather_index(d_logits, ld, dtype, b->V), (double)temperature, seed);
}

tcb_status tcb_beam_step_lmhead(tcb_beams *b, const void *d_hidden, int64_t ld_hidden, int32_t H,
                                const void *d_weight, void *stream) {
    if (!b || !d_hidden || !d_weight) return set_error(TCB_E_ARG, "beam_step_lmhead: null pointer");
    if (H <= 0 || H % 128 != 0) return set_error(TCB_E_ARG, "beam_step_lmhead: H must be a positive multiple of 128");
    if (ld_hidden < H) return set_error(TCB_E_ARG, "beam_step_lmhead: ld_hidden < H");
    if (((uintptr_t)d_hidden & 15) || ((uintptr_t)d_weight & 15) || (ld_hidden % 8))
        return set_error(TCB_E_ARG, "beam_step_lmhead: hidden/weight must be 16-byte aligned, ld % 8 == 0");
    if (b->V != 256) return set_error(TCB_E_ARG, "beam_step_lmhead: needs a trie with V = 256");
    tcb_status st = step_common(b);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    // the dense head (its own launch) writes the logits of the requests without the
    // sparse-head flag; the tile kernel computes the children's logits of the others itself,
    // after any pending merge it does first, so no merge has to be launched ahead of the step
    const tcb::StepHead hd{static_cast<const uint16_t *>(d_hidden), static_cast<const uint16_t *>(d_weight), ld_hidden,
                           H, 0};
    return run_step(
        b, s,
        [&](const tcb::StepReqs &R) {
            bool dense = false;
            for (int i = 0; i < R.n; ++i)
                if (R.r[i].step() && !R.r[i].sparse_head()) dense = true;
            return dense ? tcb::launch_lmhead(b->tdev, b->w, b->rp, R, d_hidden, ld_hidden, H, d_weight, b->w.lmx, s)
                         : hipSuccess;
        },
        [&](const tcb::WaveDev &w, const tcb::StepReqs &R, bool fuse) {
            static thread_local tcb::StepReqs Rh;
            Rh = R;
            Rh.hd = hd;
            return tcb::launch_tile(b->tdev, w, b->rp, Rh, b->w.lmx, 256, TCB_F32, false, s, fuse, true);
        },
        2, 0.0, 0, true, true);
}

tcb_status tcb_beam_export(tcb_beams *b, int32_t *d_node, float *d_score, float *d_phi, int32_t *d_parent_slot,
                           uint32_t *d_hist, int32_t *d_rows, int32_t *d_level, void *stream) {
    if (!b) return set_error(TCB_E_ARG, "beam_export: null wave");
    hipStream_t s = (hipStream_t)stream;
    tcb_status st = flush_merge(b, s);
    if (st) return st;
    st = flush_init(b, s);
    if (st) return st;
    const size_t S = (size_t)b->w.S;
    hipError_t e = hipSuccess;
    if (d_parent_slot && e == hipSuccess)
        e = hipMemcpyAsync(d_parent_slot, b->w.parent_slot, S * 4, hipMemcpyDeviceToDevice, s);
    if (d_hist && e == hipSuccess)
        e = hipMemcpyAsync(d_hist, b->w.hist, (size_t)b->L * S * 4, hipMemcpyDeviceToDevice, s);
    if ((d_node || d_score || d_phi || d_rows || d_level) && e == hipSuccess)
        e = tcb::launch_export(b->w, b->rp, d_node, d_score, d_phi, d_rows, d_level, s);
    if (e != hipSuccess) return hip_fail(e, "beam_export");
    return TCB_OK;
}

tcb_status tcb_beams_set_finish_outputs(tcb_beams *b, uint8_t *d_sids, float *d_scores, int64_t *d_items,
                                        int32_t *d_counts) {
    if (!b) return set_error(TCB_E_ARG, "set_finish_outputs: null wave");
    const int given = (d_sids != nullptr) + (d_scores != nullptr) + (d_items != nullptr) + (d_counts != nullptr);
    if (given != 0 && given != 4) return set_error(TCB_E_ARG, "set_finish_outputs: give all four buffers or none");
    b->fin = tcb::StepFin{d_sids, d_scores, d_items, d_counts};
    return TCB_OK;
}

tcb_status tcb_beams_status(const tcb_beams *b, tcb_beams_status_t *out) {
    if (!b || !out) return set_error(TCB_E_ARG, "beams_status: null pointer");
    std::memset(out, 0, sizeof(*out));
    out->steps = b->steps;
    for (const auto &q : b->reqs) {
        if (!q.used) {
            out->free_requests++;
            continue;
        }
        if (q.level < b->L) out->active++;
        else out->finished++;
    }
    for (const auto &r : b->free_ranges) out->free_slots += r.second;
    return TCB_OK;
}

tcb_status tcb_request_level(const tcb_beams *b, int32_t req_id, int32_t *level) {
    if (!b || !level) return set_error(TCB_E_ARG, "request_level: null pointer");
    if (req_id < 0 || req_id >= (int)b->reqs.size() || !b->reqs[(size_t)req_id].used)
        return set_error(TCB_E_ARG, "request_level: unknown request id");
    *level = b->reqs[(size_t)req_id].level;
    return TCB_OK;
}

tcb_status tcb_beams_set_read_mode(tcb_beams *b, int32_t mode) {
    if (!b || mode < TCB_READ_AUTO || mode > TCB_READ_GATHER) return set_error(TCB_E_ARG, "set_read_mode: bad arguments");
    b->read_mode = mode;
    return TCB_OK;
}

tcb_status tcb_beams_set_validate(tcb_beams *b, int32_t on) {
    if (!b) return set_error(TCB_E_ARG, "set_validate: null wave");
    b->w.validate = on ? 1 : 0;
    return TCB_OK;
}

tcb_status tcb_beam_check(tcb_beams *b, void *stream) {
    if (!b) return set_error(TCB_E_ARG, "beam_check: null wave");
    uint32_t err = 0;
    tcb_status st = read_err(b, (hipStream_t)stream, &err);
    if (st) return st;
    return err_status(err);
}

tcb_status tcb_beam_finalize(tcb_beams *b, int32_t n, const int32_t *req_ids, uint8_t *h_sids,
                             float *h_scores, int64_t *h_items, int32_t *h_counts, void *stream) {
    tcb_status st = check_finalize_args(b, n, req_ids);
    if (st) return st;
    if (!h_sids || !h_scores || !h_items || !h_counts)
        return set_error(TCB_E_ARG, "finalize: null output pointer");
    hipStream_t s = (hipStream_t)stream;
    st = run_finalize(b, n, req_ids, b->d_fin_sids, b->d_fin_scores, b->d_fin_items, b->d_fin_counts, s);
    if (st) return st;
    const size_t rowsz = (size_t)b->w.Bmax;
    hipError_t e = hipMemcpyAsync(h_sids, b->d_fin_sids, (size_t)n * rowsz * (size_t)b->L, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h_scores, b->d_fin_scores, (size_t)n * rowsz * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h_items, b->d_fin_items, (size_t)n * rowsz * 8, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h_counts, b->d_fin_counts, (size_t)n * 4, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "finalize copy");
    uint32_t err = 0;
    st = read_err(b, s, &err);
    if (st) return st;
    release(b, n, req_ids);
    return err_status(err);
}

tcb_status tcb_beam_finalize_device(tcb_beams *b, int32_t n, const int32_t *req_ids, uint8_t *d_sids,
                                    float *d_scores, int64_t *d_items, int32_t *d_counts, void *stream) {
    tcb_status st = check_finalize_args(b, n, req_ids);
    if (st) return st;
    if (!d_sids || !d_scores || !d_items || !d_counts)
        return set_error(TCB_E_ARG, "finalize_device: null output pointer");
    st = run_finalize(b, n, req_ids, d_sids, d_scores, d_items, d_counts, (hipStream_t)stream);
    if (st) return st;
    release(b, n, req_ids);
    return TCB_OK;
}

tcb_status tcb_beams_enable_timing(tcb_beams *b, int32_t capacity, int32_t repeat) {
    if (!b || capacity < 0 || repeat < 1 || repeat > 1000) return set_error(TCB_E_ARG, "enable_timing: bad arguments");
    for (auto e : b->events) (void)hipEventDestroy(e);
    b->events.clear();
    b->timing_cap = 0;
    b->timing_used = 0;
    b->timing_repeat = repeat;
    for (int32_t i = 0; i < capacity * 4; ++i) {
        hipEvent_t e;
        hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) {
            for (auto x : b->events) (void)hipEventDestroy(x);
            b->events.clear();
            return hip_fail(r, "enable_timing: hipEventCreate");
        }
        b->events.push_back(e);
    }
    b->timing_cap = capacity;
    return TCB_OK;
}

tcb_status tcb_beams_timing(tcb_beams *b, double *head_ms, double *tile_ms, double *merge_ms, int32_t *steps) {
    if (!b || !head_ms || !tile_ms || !merge_ms || !steps) return set_error(TCB_E_ARG, "timing: null pointer");
    if (b->timing_cap == 0) return set_error(TCB_E_STATE, "timing: not enabled");
    double th = 0.0, ta = 0.0, tb = 0.0;
    for (int32_t i = 0; i < b->timing_used; ++i) {
        hipEvent_t *ev = &b->events[(size_t)i * 4];
        hipError_t r = hipEventSynchronize(ev[3]);
        float h = 0.f, a = 0.f, c = 0.f;
        if (r == hipSuccess) r = hipEventElapsedTime(&h, ev[0], ev[1]);
        if (r == hipSuccess) r = hipEventElapsedTime(&a, ev[1], ev[2]);
        if (r == hipSuccess) r = hipEventElapsedTime(&c, ev[2], ev[3]);
        if (r != hipSuccess) return hip_fail(r, "timing: elapsed time");
        th += h / b->timing_repeat;
        ta += a / b->timing_repeat;
        tb += c / b->timing_repeat;
    }
    *head_ms = th;
    *tile_ms = ta;
    *merge_ms = tb;
    *steps = b->timing_used;
    return TCB_OK;
}

tcb_status tcb_beams_set_trace(tcb_beams *b, uint64_t *d_buf, int64_t capacity_words) {
    if (!b || capacity_words < 0 || (capacity_words > 0 && !d_buf)) return set_error(TCB_E_ARG, "set_trace: bad arguments");
    b->trace_buf = capacity_words > 0 ? d_buf : nullptr;
    b->trace_cap = capacity_words;
    b->trace_used = 0;
    b->trace_log.clear();
    return TCB_OK;
}

tcb_status tcb_beams_trace_log(const tcb_beams *b, int32_t *out, int32_t max_launches, int32_t *n) {
    if (!b || !n || max_launches < 0 || (max_launches > 0 && !out)) return set_error(TCB_E_ARG, "trace_log: bad arguments");
    const int32_t have = (int32_t)(b->trace_log.size() / 4);
    *n = have;
    if (max_launches > 0 && have > 0)
        std::memcpy(out, b->trace_log.data(), sizeof(int32_t) * 4 * (size_t)std::min(have, max_launches));
    return TCB_OK;
}

void tcb_beams_destroy(tcb_beams *b) { delete b; }

}  // extern "C"
