// Host side of single-pass scoring of every valid SID (SPRINT summary, method and
// inference paragraphs): argument checks, the leaf-code table, workspace layout and
// launches. All arithmetic runs in score.hip.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "score_internal.h"
#include "tcb_host.h"

using tcb_host::set_error;

namespace {

tcb_status hip_fail(hipError_t e, const char *what) {
    return set_error(TCB_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Leaf codes, built from the CSR arrays top-down: the prefix of a child is its
// parent's prefix with the child's code appended at byte d.
tcb_status build_codes(tcb_trie *t) {
    if (!t->codes.empty()) return TCB_OK;
    const int L = t->L;
    const size_t width = L <= 4 ? 4 : 8;
    std::vector<uint64_t> pref;
    try {
        pref.assign((size_t)t->off[L + 1], 0);
        t->codes.assign((size_t)t->n_distinct * width, 0);
    } catch (const std::bad_alloc &) {
        return set_error(TCB_E_ARG, "trie codes: out of host memory");
    }
    for (int d = 0; d < L; ++d)
        for (int64_t nd = t->off[d]; nd < t->off[d + 1]; ++nd)
            for (uint32_t c = t->child_begin[(size_t)nd]; c < t->child_begin[(size_t)nd + 1]; ++c)
                pref[c] = pref[(size_t)nd] | ((uint64_t)t->child_code[c] << (8 * d));
    for (int64_t i = 0; i < t->n_distinct; ++i) {
        const uint64_t v = pref[(size_t)(t->off[L] + i)];
        std::memcpy(t->codes.data() + (size_t)i * width, &v, width);   // little-endian: byte d = depth d
    }
    return TCB_OK;
}

// Diagnostic kernel timing of tcb_score_catalog calls (process-wide).
struct ScoreTiming {
    std::mutex mu;
    std::vector<hipEvent_t> ev;
    int cap = 0, used = 0;
    void release() {
        for (auto e : ev) (void)hipEventDestroy(e);
        ev.clear();
        cap = used = 0;
    }
};
ScoreTiming g_timing;

}  // namespace

extern "C" {

tcb_status tcb_trie_codes_bytes(const tcb_trie *t, size_t *bytes) {
    if (!t || !bytes) return set_error(TCB_E_ARG, "trie_codes_bytes: null pointer");
    *bytes = (size_t)t->n_distinct * (t->L <= 4 ? 4 : 8);
    return TCB_OK;
}

tcb_status tcb_trie_upload_codes(tcb_trie *t, void *d_buf, size_t bytes, void *stream) {
    if (!t || !d_buf) return set_error(TCB_E_ARG, "trie_upload_codes: null pointer");
    if (((uintptr_t)d_buf & 255) != 0) return set_error(TCB_E_WORKSPACE, "trie_upload_codes: buffer not 256-byte aligned");
    size_t need = 0;
    tcb_trie_codes_bytes(t, &need);
    if (bytes < need) return set_error(TCB_E_WORKSPACE, "trie_upload_codes: buffer too small");
    const tcb_status st = build_codes(t);
    if (st != TCB_OK) return st;
    const hipError_t e = hipMemcpyAsync(d_buf, t->codes.data(), need, hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "trie_upload_codes copy");
    t->d_codes = d_buf;
    return TCB_OK;
}

tcb_status tcb_score_workspace_bytes(const tcb_trie *t, int32_t max_users, size_t *bytes) {
    if (!t || !bytes) return set_error(TCB_E_ARG, "score_workspace_bytes: null pointer");
    if (max_users <= 0) return set_error(TCB_E_ARG, "score_workspace_bytes: max_users must be > 0");
    *bytes = tcb::score_layout(t->L, t->n_distinct, max_users).total;
    return TCB_OK;
}

tcb_status tcb_score_catalog(const tcb_trie *t, int32_t n_users, const float *d_table,
                             int32_t table_kind, const void *d_user_vec, const void *d_sid_emb,
                             int32_t dim, float sid_weight, int32_t k, int32_t *d_leaf,
                             int32_t *d_item, float *d_score, float *d_lse, void *d_ws,
                             size_t ws_bytes, void *stream) {
    if (!t || !d_table || !d_leaf || !d_score || !d_ws) return set_error(TCB_E_ARG, "score_catalog: null pointer");
    if (!t->d_image) return set_error(TCB_E_STATE, "score_catalog: trie not uploaded");
    if (!t->d_codes) return set_error(TCB_E_STATE, "score_catalog: leaf codes not uploaded");
    if (n_users <= 0) return set_error(TCB_E_ARG, "score_catalog: n_users must be > 0");
    if (k < 1 || k > TCB_SCORE_MAX_K) return set_error(TCB_E_ARG, "score_catalog: k must be in 1..512");
    if (table_kind != TCB_TABLE_LOGPROB && table_kind != TCB_TABLE_LOGITS)
        return set_error(TCB_E_ARG, "score_catalog: bad table_kind");
    if (t->n_distinct > TCB_SCORE_MAX_SIDS) return set_error(TCB_E_ARG, "score_catalog: more than 2^25 SIDs");
    const bool sid_term = d_user_vec || d_sid_emb;
    if (sid_term) {
        if (!d_user_vec || !d_sid_emb)
            return set_error(TCB_E_ARG, "score_catalog: user vectors and SID embeddings go together");
        if (dim != 32 && dim != 64 && dim != 128 && dim != 256)
            return set_error(TCB_E_ARG, "score_catalog: dim must be 32, 64, 128 or 256");
        if ((((uintptr_t)d_user_vec | (uintptr_t)d_sid_emb) & 15) != 0)
            return set_error(TCB_E_ARG, "score_catalog: user vectors / embeddings not 16-byte aligned");
        if (!std::isfinite(sid_weight)) return set_error(TCB_E_ARG, "score_catalog: sid_weight not finite");
    }
    if (((uintptr_t)d_ws & 255) != 0) return set_error(TCB_E_WORKSPACE, "score_catalog: workspace not 256-byte aligned");
    const tcb::ScoreLayout lay = tcb::score_layout(t->L, t->n_distinct, n_users);
    if (ws_bytes < lay.total) return set_error(TCB_E_WORKSPACE, "score_catalog: workspace too small");

    tcb::ScoreDev a{};
    uint8_t *ws = static_cast<uint8_t *>(d_ws);
    a.codes = t->d_codes;
    a.leaf_item = reinterpret_cast<const int32_t *>(static_cast<const uint8_t *>(t->d_image) + t->o_leaf);
    a.table_in = d_table;
    a.table = reinterpret_cast<float *>(ws + lay.table);
    a.user_vec = sid_term ? static_cast<const uint16_t *>(d_user_vec) : nullptr;
    a.emb = sid_term ? static_cast<const uint16_t *>(d_sid_emb) : nullptr;
    a.gmax = reinterpret_cast<float *>(ws + lay.gmax);
    a.bmax = reinterpret_cast<float *>(ws + lay.bmax);
    a.lse_part = reinterpret_cast<float *>(ws + lay.lse);
    a.pick = reinterpret_cast<int32_t *>(ws + lay.pick);
    a.npick = reinterpret_cast<int32_t *>(ws + lay.npick);
    a.cand = reinterpret_cast<float *>(ws + lay.cand);
    a.out_leaf = d_leaf;
    a.out_item = d_item;
    a.out_score = d_score;
    a.out_lse = d_lse;
    a.n = t->n_distinct;
    a.L = t->L;
    a.V = t->V;
    a.U = n_users;
    a.D = sid_term ? dim : 0;
    a.K = k;
    a.kind = table_kind;
    a.ug = tcb::score_ug(t->L);
    a.groups = (n_users + a.ug - 1) / a.ug;
    a.w = sid_term ? sid_weight : 0.0f;
    const hipEvent_t *ev = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_timing.mu);
        if (g_timing.used < g_timing.cap) ev = g_timing.ev.data() + 3 * (g_timing.used++);
    }
    const hipError_t e = tcb::launch_score(a, (hipStream_t)stream, ev);
    if (e != hipSuccess) return hip_fail(e, "score_catalog launch");
    return TCB_OK;
}

tcb_status tcb_score_catalog_static(const tcb_trie *t, int32_t n_users, const float *d_table,
                                    int32_t table_kind, const void *d_user_vec, const void *d_sid_emb,
                                    int32_t dim, float sid_weight, int32_t k, int32_t *d_leaf,
                                    int32_t *d_item, float *d_score, float *d_lse, void *stream) {
    if (!t) return set_error(TCB_E_ARG, "score_catalog_static: null trie");
    if (n_users <= 0) return set_error(TCB_E_ARG, "score_catalog_static: n_users must be > 0");
    const size_t need = tcb::score_layout(t->L, t->n_distinct, n_users).total;
    if (need > tcb::kStaticScoreScratch)
        return set_error(TCB_E_WORKSPACE, "score_catalog_static: " + std::to_string(n_users) + " users x " +
                                              std::to_string(t->n_distinct) + " SIDs need " + std::to_string(need) +
                                              " bytes of scratch; the static scratch holds " +
                                              std::to_string(tcb::kStaticScoreScratch));
    void *ws = nullptr;
    size_t cap = 0;
    const hipError_t e = tcb::static_score_scratch(&ws, &cap);
    if (e != hipSuccess) return hip_fail(e, "score_catalog_static: scratch address");
    return tcb_score_catalog(t, n_users, d_table, table_kind, d_user_vec, d_sid_emb, dim, sid_weight, k, d_leaf,
                             d_item, d_score, d_lse, ws, cap, stream);
}

tcb_status tcb_score_enable_timing(int32_t capacity) {
    if (capacity < 0 || capacity > 100000) return set_error(TCB_E_ARG, "score_enable_timing: capacity out of range");
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.release();
    if (capacity == 0) return TCB_OK;
    g_timing.ev.resize((size_t)capacity * 3);
    for (auto &e : g_timing.ev) {
        const hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) {
            e = nullptr;
            g_timing.ev.erase(std::remove(g_timing.ev.begin(), g_timing.ev.end(), nullptr), g_timing.ev.end());
            g_timing.release();
            return hip_fail(r, "score_enable_timing event");
        }
    }
    g_timing.cap = capacity;
    return TCB_OK;
}

tcb_status tcb_score_timing(double *scan_ms, double *select_ms, int32_t *calls) {
    if (!scan_ms || !select_ms || !calls) return set_error(TCB_E_ARG, "score_timing: null pointer");
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.cap == 0) return set_error(TCB_E_STATE, "score_timing: timing not enabled");
    double acc[2] = {0.0, 0.0};
    for (int c = 0; c < g_timing.used; ++c) {
        const hipEvent_t *e = g_timing.ev.data() + 3 * c;
        hipError_t r = hipEventSynchronize(e[2]);
        if (r != hipSuccess) return hip_fail(r, "score_timing sync");
        for (int k = 0; k < 2; ++k) {
            float ms = 0.0f;
            r = hipEventElapsedTime(&ms, e[k], e[k + 1]);
            if (r != hipSuccess) return hip_fail(r, "score_timing elapsed");
            acc[k] += ms;
        }
    }
    *scan_ms = acc[0];
    *select_ms = acc[1];
    *calls = g_timing.used;
    return TCB_OK;
}

}  // extern "C"
