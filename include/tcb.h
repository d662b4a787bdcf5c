/*
 * tcb.h -- catalog-constrained wide-beam expansion on MI355X (gfx950).
 *
 * C ABI of libtcb.so. The operation is one step of generative-recommendation
 * decoding over semantic IDs (SIDs): every live beam row's logits over its level's
 * code range are masked to the children of the row's node in a prefix trie of
 * valid catalog SIDs, log-softmaxed and added to the beam score; each request then
 * keeps its best n (beam width) (row, child) candidates, ranked best-first, and the
 * survivors are re-indexed by parent row and trie node.
 *
 * Sources (web pages; cited by title and section):
 *   [FR]  flashrec 0.1.0 (PyPI project page): Features > Decoding ("SID
 *         constraint": dense or CSR-sparse trie, illegal SIDs never candidates,
 *         lm_head only over the SID token range; "Scheduling": requests admitted
 *         into decode waves between steps under a beam-row slot budget),
 *         Features > Serving ("API": deterministic top-k at temperature 0, Gumbel
 *         top-k without replacement above it), Quickstart (beam width n, ranked
 *         choices with a sequence score, --batch-slots).
 *   [OLA] OneLA summary: section 2.1 (candidates globally selected across the
 *         beam), sections 2.4 / 3.3 (children keep an index to their parent;
 *         records are append-only and never moved).
 *   [SP]  SPRINT summary, method paragraph (one pass gives an L x M table of
 *         per-position token distributions and a user vector; scoring a valid SID
 *         is a table lookup plus one matrix product) and inference paragraph (valid
 *         SIDs of a prefix trie scored by their token log-probability sum plus a
 *         SID-level similarity, then top-K; the softmax runs over the valid SIDs).
 *
 * Conventions
 *   - Every call returns tcb_status: TCB_OK (0) or a negative error code. On error
 *     tcb_last_error() returns a thread-local message. Argument errors are found on
 *     the host before any device work, so they leave every object unchanged.
 *   - Device pointers ("d_") are HIP device addresses owned by the caller; they
 *     must stay valid until the work enqueued on the stream has completed. The
 *     library never allocates device memory. Host pointers ("h_" or plain) are
 *     read or written before the call returns unless stated otherwise.
 *   - "stream" is a hipStream_t passed as void* (NULL = the default stream).
 *   - A tcb_trie is immutable after tcb_trie_upload and may be shared by several
 *     tcb_beams. A tcb_beams object is used from one host thread and one stream.
 *   - Only tcb_beam_check and tcb_beam_finalize synchronise the stream.
 *   - A step may leave its per-request merge (the ranking of the candidates into the
 *     new rows) to the next step's kernels; tcb_beam_export, the finalize calls and a
 *     step that needs the merged rows first launch it themselves. Results do not
 *     depend on where the merge runs; a wave's steps therefore go to one stream.
 */
#ifndef TCB_H
#define TCB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tcb_status;

enum {
    TCB_OK = 0,
    TCB_E_ARG = -1,        /* null pointer, bad size, bad enum value             */
    TCB_E_RANGE = -2,      /* a SID code >= V, L or V out of range               */
    TCB_E_BUDGET = -3,     /* beam widths exceed the free slots or request ids   */
    TCB_E_STATE = -4,      /* call not valid in the current state                */
    TCB_E_WORKSPACE = -5,  /* device buffer too small or misaligned              */
    TCB_E_HIP = -6,        /* a HIP runtime call failed                          */
    TCB_E_NONFINITE = -7,  /* a non-finite logit was seen (validation on)        */
    TCB_E_DEVICE = -8      /* the device found corrupt state; destroy the wave   */
};

enum { TCB_F32 = 0, TCB_BF16 = 1 };                 /* logits element type           */
enum { TCB_NORM_CHILDREN = 0, TCB_NORM_LEVEL = 1, TCB_NORM_OPEN = 2 }; /* normaliser / constraint */

#define TCB_MAX_L 8
#define TCB_MAX_V 256
#define TCB_MAX_WIDTH 4096
#define TCB_MASK_AUTO (-1)          /* mask_depths: choose from the trie's size        */
#define TCB_MASK_AUTO_BYTES (1ll << 30) /* ... masks on the leading depths up to this  */

typedef struct tcb_trie tcb_trie;
typedef struct tcb_beams tcb_beams;

const char *tcb_last_error(void);
const char *tcb_version(void);

/* ------------------------------------------------------------------------ trie */

/* Build the prefix trie of a SID catalog on the host ([FR] Decoding, "SID
 * constraint"; [SP] inference).
 *   sids        host [n_items][L] uint8, row i = SID of catalog item i
 *   n_items     > 0
 *   L           SID depth, 1..TCB_MAX_L
 *   V           codes per level, 2..256; every code must be < V
 *   mask_depths depths 0..mask_depths-1 also get a 256-bit child mask per node
 *               ("dense" trie); deeper nodes use only the CSR child list. 0..L, or
 *               TCB_MASK_AUTO: every leading depth whose masks, counted together with
 *               the shallower depths' (32 bytes per node), fit in TCB_MASK_AUTO_BYTES;
 *               normally all of them (tcb_trie_info reports the choice).
 *               Results do not depend on this choice; only speed does.
 * Duplicated SIDs collapse onto one leaf whose item is the lowest catalog row.
 * Nodes are numbered depth-major and lexicographically: the root is 0, depth d
 * holds ids [off_d, off_{d+1}) in ascending prefix order, so the children of a node
 * are a contiguous id range in ascending code order.
 * Errors: TCB_E_ARG (null, n_items <= 0, mask_depths out of range),
 *         TCB_E_RANGE (L or V out of range, a code >= V). */
tcb_status tcb_build_trie(const uint8_t *sids, int64_t n_items, int32_t L, int32_t V,
                          int32_t mask_depths, tcb_trie **out);

typedef struct {
    int32_t L, V, mask_depths;
    int64_t n_items;                       /* catalog rows given                      */
    int64_t n_distinct;                    /* distinct SIDs = leaves                  */
    int64_t nodes_per_depth[TCB_MAX_L + 1];
    int64_t node_offset[TCB_MAX_L + 2];    /* off_d; node_offset[L+1] = total nodes   */
    size_t device_bytes;                   /* size of the device image                */
} tcb_trie_info_t;

tcb_status tcb_trie_info(const tcb_trie *t, tcb_trie_info_t *out);

/* Host views of the CSR arrays (valid until tcb_trie_destroy), for inspection:
 *   child_begin [node_offset[L] + 1]  children of internal node n are node ids
 *                                      child_begin[n] .. child_begin[n+1]-1
 *   child_code  [total nodes]         code on the edge into node k (0 for the root)
 *   leaf_item   [n_distinct]          catalog row of leaf node_offset[L] + j       */
tcb_status tcb_trie_host_arrays(const tcb_trie *t, const uint32_t **child_begin,
                                const uint8_t **child_code, const int32_t **leaf_item);

/* Copy the trie image into caller-owned device memory of at least
 * tcb_trie_info().device_bytes bytes (256-byte aligned). Asynchronous on stream;
 * the host image stays owned by the trie. A later upload replaces the previous one
 * for every wave created afterwards. Errors: TCB_E_ARG, TCB_E_WORKSPACE, TCB_E_HIP. */
tcb_status tcb_trie_upload(tcb_trie *t, void *d_buf, size_t bytes, void *stream);

void tcb_trie_destroy(tcb_trie *t);

/* ------------------------------------------------------------------------ wave */

/* Device workspace needed by a wave (tcb_beams) with at most max_slots beam rows
 * in flight, max_requests requests in flight and beams at most max_width wide. */
tcb_status tcb_beams_workspace_bytes(const tcb_trie *t, int32_t max_slots,
                                     int32_t max_requests, int32_t max_width, size_t *bytes);

/* Create a decode wave over an uploaded trie ([FR] Decoding, "Scheduling": rows of
 * different requests share a step under a beam-row slot budget).
 *   norm   TCB_NORM_CHILDREN (log-softmax over the node's children),
 *          TCB_NORM_LEVEL (over all V codes of the level, then masked), or
 *          TCB_NORM_OPEN: no SID constraint, as an open-vocabulary engine decodes
 *          ([FR] Evaluation compares the share of illegal beams with and without
 *          the constraint): every code is a candidate, normalised over all V
 *          codes; a row whose prefix has left the catalog has node -1, and such
 *          beams are finalised with item -1
 *   d_ws   caller-owned device workspace of ws_bytes >= tcb_beams_workspace_bytes,
 *          256-byte aligned; the wave initialises it on `stream`.
 * Errors: TCB_E_ARG, TCB_E_STATE (trie not uploaded), TCB_E_WORKSPACE, TCB_E_HIP. */
tcb_status tcb_beams_create(const tcb_trie *t, int32_t max_slots, int32_t max_requests,
                            int32_t max_width, int32_t norm, void *d_ws, size_t ws_bytes,
                            void *stream, tcb_beams **out);

/* Admit n requests at the root (one row, score 0) before the next step ([FR]
 * Decoding, "Scheduling": requests join decode waves between steps while their beam
 * rows fit the slot budget, and then share every step with the requests already in
 * flight. The pages give no start state; the plainest reading, taken here, is one
 * row at the root, the empty prefix, with score 0).
 *   widths         host [n], beam width n_i of each request, 1..max_width
 *   out_req_ids    host [n] (may be NULL): request id of each admitted request
 *   out_slot_base  host [n] (may be NULL): request i owns slots
 *                  [base_i, base_i + n_i); its live rows are the first rows_i of
 *                  them, best first. Logits / hidden rows are indexed by slot.
 * All or nothing: if the requests do not all fit in the free slots / ids the call
 * returns TCB_E_BUDGET and admits none. Nothing is launched: a request's first step
 * starts from this known state without reading it, and the device copy of the state is
 * written on the stream of an export or finalize that would read it first (`stream`
 * is unused). */
tcb_status tcb_beam_init(tcb_beams *b, int32_t n, const int32_t *widths,
                         int32_t *out_req_ids, int32_t *out_slot_base, void *stream);

/* One constrained beam step for every admitted, unfinished request ([FR] Decoding;
 * [OLA] 2.1; [SP] inference).
 *   d_logits  device [max_slots][ld] of dtype TCB_F32 or TCB_BF16; row `slot` holds
 *             the V logits of that slot's row at its request's current level. Rows
 *             of a request's slot range beyond its live rows may be read and are
 *             ignored. ld >= V (elements).
 * Per request: candidates (r, c) for every live row r and child code c of its node,
 * scored s_r + logp(c); the best min(n_i, #candidates) by (score desc, r*V+c asc)
 * become the new rows in rank order, with parent slot base_i + r and a
 * back-pointer (r, c) appended for this level. Requests never compete.
 * Errors: TCB_E_ARG, TCB_E_STATE (no unfinished request), TCB_E_HIP. */
tcb_status tcb_beam_step(tcb_beams *b, const void *d_logits, int64_t ld, int32_t dtype,
                         void *stream);

/* The step above temperature 0: a Gumbel top-k without replacement over SIDs ([FR]
 * Serving, "API": deterministic top-k at temperature 0, Gumbel top-k without
 * replacement above it). Same arguments as tcb_beam_step plus
 *   temperature  finite and > 0: each row's children are scored by the masked
 *                log-softmax of x / temperature; a beam's log-probability phi is the
 *                sum of those terms (reported as its score by tcb_beam_finalize)
 *   seed         the noise seed of this step
 * Every beam carries phi and a perturbed key G (root: 0, 0). Child c of row r draws
 * g = phi_r + logp(c) + Gumbel(0, 1), the uniform coming from SplitMix64 keyed by
 * (seed, request id, level, r, c); its key is g conditioned on the maximum over r's
 * children being G_r (stochastic beam search), and the request keeps its best
 * min(n_i, #candidates) children by (key desc, r*V+c asc). Over a whole decode the
 * beams are then a sample of distinct SIDs without replacement from the tempered SID
 * distribution. Errors as tcb_beam_step; TCB_E_ARG for a bad temperature. */
tcb_status tcb_beam_step_sampled(tcb_beams *b, const void *d_logits, int64_t ld, int32_t dtype,
                                 float temperature, uint64_t seed, void *stream);

/* Same step with the logits computed on chip by the SID-range lm_head ([FR]
 * Decoding: lm_head only over the SID token range):
 *   x[slot][c] = sum_h hidden[slot][h] * W[level][c][h], fp32 accumulate, no bias.
 *   d_hidden  device bf16 [max_slots][ld_hidden], ld_hidden >= H, ld_hidden % 8 == 0,
 *             H % 128 == 0, 16-byte aligned; row `slot` is that slot's hidden state
 *   d_weight  device bf16 [L][256][H] contiguous (one [256][H] matrix per level),
 *             16-byte aligned; the trie must have V = 256
 * Where rows have many children the dense head (MFMA, its own launch) writes all 256
 * logits of each row to an fp32 [max_slots][256] part of the workspace and the step
 * kernel reads them; where they have about one (tcb_beams_set_read_mode), the step kernel
 * computes only the children's logits itself and keeps them on chip. The masked
 * log-softmax and selection are those of tcb_beam_step.
 * Errors as tcb_beam_step; TCB_E_ARG for the shape and alignment conditions above. */
tcb_status tcb_beam_step_lmhead(tcb_beams *b, const void *d_hidden, int64_t ld_hidden,
                                int32_t H, const void *d_weight, void *stream);

/* Copy the current wave state into caller device buffers (any may be NULL):
 *   d_node, d_score       [max_slots]  node id and selection key of each slot's row
 *   d_phi                 [max_slots]  summed log-probability of each slot's row (equal
 *                                      to the key unless a step was sampled)
 *   d_parent_slot         [max_slots]  slot of each row's parent at the last step
 *   d_hist                [L][max_slots] back-pointer of level t: (r << 8) | c
 *   d_rows, d_level       [max_requests] live rows and levels per request id
 * Rows beyond a request's live count hold stale values. Asynchronous. With every
 * buffer NULL nothing is copied: the call only launches a merge the last step left to
 * the next step, so that the state is current (a caller whose next logits depend on
 * this step's survivors reads them between steps, and the merge then runs on its own). */
tcb_status tcb_beam_export(tcb_beams *b, int32_t *d_node, float *d_score, float *d_phi,
                           int32_t *d_parent_slot, uint32_t *d_hist, int32_t *d_rows,
                           int32_t *d_level, void *stream);

/* Host-side status (no device access): steps taken, requests admitted and
 * finished, free slots. */
typedef struct {
    int64_t steps;
    int32_t active;          /* admitted and not yet at depth L */
    int32_t finished;        /* at depth L, awaiting finalize   */
    int32_t free_slots;
    int32_t free_requests;
} tcb_beams_status_t;
tcb_status tcb_beams_status(const tcb_beams *b, tcb_beams_status_t *out);

/* Level of a request (host-side; levels advance by one per step). */
tcb_status tcb_request_level(const tcb_beams *b, int32_t req_id, int32_t *level);

/* Turn on non-finite checks of every logit read (sticky TCB_E_NONFINITE). With sector
 * gathering (below) only the logits of a row's children are read and checked. */
tcb_status tcb_beams_set_validate(tcb_beams *b, int32_t on);

/* How tcb_beam_step / tcb_beam_step_sampled read a row's logits ([FR] Decoding: a
 * dense or CSR-sparse trie; the sparse reading applied to the logits traffic):
 *   TCB_READ_AUTO    whole rows at depths with many children per row; where a row's
 *                    children touch under half of its 64-byte sectors on average, only
 *                    the 16-byte pieces holding a child (default)
 *   TCB_READ_DENSE   always whole rows
 *   TCB_READ_GATHER  always only the pieces holding a child
 * Results are bitwise the same in every mode; only traffic and latency differ. Sector
 * gathering applies to the children normaliser with 16-byte aligned rows (otherwise
 * rows are read whole).
 * For tcb_beam_step_lmhead the same modes choose the head: DENSE computes every row's
 * 256 logits (MFMA, its own launch); GATHER computes, inside the step kernel and after
 * the rows' nodes are known, only the logits of each row's children (one dot product
 * over H per child), so no logits are written or read; AUTO does so at depths whose
 * nodes have at most two children on average. A request's first step always uses the
 * dense head. The two heads sum in different orders, so their logits agree to fp32
 * rounding rather than bitwise. Errors: TCB_E_ARG. */
enum { TCB_READ_AUTO = 0, TCB_READ_DENSE = 1, TCB_READ_GATHER = 2 };
tcb_status tcb_beams_set_read_mode(tcb_beams *b, int32_t mode);

/* Synchronise `stream` and report a sticky device error, if any. */
tcb_status tcb_beam_check(tcb_beams *b, void *stream);

/* Finished requests' beams, ranked best-first with their scores ([FR] Quickstart:
 * ranked choices with a sequence score), then release their slots and ids.
 *   req_ids    host [n], requests at depth L
 *   h_sids     host [n][max_width][L] uint8   codes, walked back from the
 *                                             per-level back-pointers
 *   h_scores   host [n][max_width] float      summed log-probabilities
 *   h_items    host [n][max_width] int64      catalog row of the SID
 *   h_counts   host [n] int32                 number of beams of each request
 * Entries past a request's count are zero / -inf / -1. Synchronises `stream`.
 * Errors: TCB_E_ARG, TCB_E_STATE (a request not finished), TCB_E_NONFINITE,
 *         TCB_E_DEVICE, TCB_E_HIP. */
tcb_status tcb_beam_finalize(tcb_beams *b, int32_t n, const int32_t *req_ids,
                             uint8_t *h_sids, float *h_scores, int64_t *h_items,
                             int32_t *h_counts, void *stream);

/* As tcb_beam_finalize, but writes caller device buffers of the same layouts and
 * does not synchronise; the ids and slots are reusable by the next tcb_beam_init
 * (stream order keeps the gather ahead of any reuse). */
tcb_status tcb_beam_finalize_device(tcb_beams *b, int32_t n, const int32_t *req_ids,
                                    uint8_t *d_sids, float *d_scores, int64_t *d_items,
                                    int32_t *d_counts, void *stream);

/* Finish requests inside the step that completes them ([FR] Quickstart: ranked choices
 * with a sequence score; Features > Decoding, "CUDA graphs": the whole expansion step is
 * one graph replay, and "Scheduling": slots are reused by requests admitted between steps).
 * Once set, every step (of any kind) that brings a request to depth L also writes that
 * request's beams into row `req_id` of these caller device buffers, with the content
 * and layout tcb_beam_finalize gives a row:
 *   d_sids     [max_requests][max_width][L] uint8
 *   d_scores   [max_requests][max_width] float
 *   d_items    [max_requests][max_width] int64
 *   d_counts   [max_requests] int32
 * and releases the request's id and slots at once (tcb_beam_finalize then no longer
 * knows the id). The writes are made by the step's own kernels on its stream: a row is
 * complete when the step's work on that stream is, and is overwritten when its id,
 * re-admitted, finishes again. Requests already at depth L are not affected. The
 * buffers must stay allocated while set; all four NULL turns the mode off.
 * Errors: TCB_E_ARG (a null wave, or some but not all buffers NULL). */
tcb_status tcb_beams_set_finish_outputs(tcb_beams *b, uint8_t *d_sids, float *d_scores,
                                        int64_t *d_items, int32_t *d_counts);

/* Diagnostics: record HIP events on `stream` around the kernels of each of the next
 * `capacity` steps (the lm_head kernel of tcb_beam_step_lmhead, the tile kernel, then the
 * per-request merge kernel); 0 stops recording and releases the events. While recording,
 * each kernel is launched `repeat` times (1..1000) back to back between its events; within
 * a step every kernel rewrites the same outputs from unchanged inputs, so results do not
 * change, and the reported durations are per launch. The events are created here (no
 * device memory). */
tcb_status tcb_beams_enable_timing(tcb_beams *b, int32_t capacity, int32_t repeat);

/* Synchronise the recorded events and report, over the steps recorded since
 * tcb_beams_enable_timing, the summed per-launch lm_head (0 for tcb_beam_step), tile-kernel
 * and merge-kernel durations (ms) and the number of steps.
 * Errors: TCB_E_STATE (timing not enabled), TCB_E_HIP. */
tcb_status tcb_beams_timing(tcb_beams *b, double *head_ms, double *tile_ms, double *merge_ms,
                            int32_t *steps);

/* Phase trace (diagnostics). Arms a trace of the kernels this wave launches from now
 * on: each tile or merge launch that still fits appends, per workgroup, TCB_TRACE_SLOTS
 * 64-bit words to d_buf (caller-owned device memory of capacity_words words): word 0 =
 * 1 + the XCD the workgroup ran on, word i > 0 = the 100 MHz real-time clock when the
 * workgroup passed phase mark i (0 if it never did). Tile marks: 1 start, 2 the previous
 * step's merge done (steps that merge it first), 14 logits and child bits in registers,
 * 15 keys computed (the first wave), 3 every wave's rows loaded and log-softmaxed, 4
 * prefilter bound, 5 candidates binned, 6 staged for an in-tile merge, 7 done; merge
 * marks (also a tile's merge of the previous step): 1 start, 8 counts read, 11 window
 * bins found, 12 staging offsets, 13 thread 0's candidate staged, 9 candidates staged,
 * 10 done; in k_merge's finishing merge 11 marks the ranks written (after 9). capacity_words = 0 turns
 * tracing off. Launches captured into a HIP graph keep the buffer they were captured
 * with. Errors: TCB_E_ARG. */
#define TCB_TRACE_SLOTS 16
enum { TCB_TRACE_TILE = 1, TCB_TRACE_MERGE = 2 };
tcb_status tcb_beams_set_trace(tcb_beams *b, uint64_t *d_buf, int64_t capacity_words);

/* The traced launches since tcb_beams_set_trace: 4 int32 per launch (kind TCB_TRACE_*,
 * the highest level it stepped, workgroups, word offset of its region in d_buf), at most
 * max_launches of them written to out; *n = how many were traced. Errors: TCB_E_ARG. */
tcb_status tcb_beams_trace_log(const tcb_beams *b, int32_t *out, int32_t max_launches, int32_t *n);

void tcb_beams_destroy(tcb_beams *b);

/* ------------------------------------------------------------------------------
 * Single-pass scoring of every valid SID ([SP] method and inference paragraphs)
 *
 *   score(u, s) = sum_d T_u[d][c_d(s)] + w * <v_u, e_s>
 *   lse(u)      = log sum over valid s of exp(score(u, s))      (P(s|u) = exp(score - lse))
 *
 * over the trie's leaves s (distinct SIDs, leaf j = the j-th smallest SID). T_u is user
 * u's L x V table of per-position token log-probabilities (or raw per-position logits,
 * normalised here by a log-softmax over the V codes of each position); v_u (the user
 * vector) and e_s (one SID-level embedding row per leaf) are bf16, accumulated in
 * fp32. Users never interact. The K best SIDs per user are returned ranked by
 * (score desc, leaf asc).
 * ------------------------------------------------------------------------------ */
#define TCB_SCORE_MAX_K 512
#define TCB_SCORE_MAX_SIDS (1 << 25)
enum { TCB_TABLE_LOGPROB = 0, TCB_TABLE_LOGITS = 1 };

/* Device copy of every leaf's codes, needed by tcb_score_catalog: 4 bytes per leaf for
 * L <= 4, 8 bytes otherwise (byte d = the code at depth d). tcb_trie_upload_codes
 * copies it asynchronously into caller memory (256-byte aligned) of at least
 * *bytes; the host copy stays owned by the trie. Errors: TCB_E_ARG, TCB_E_WORKSPACE,
 * TCB_E_HIP. */
tcb_status tcb_trie_codes_bytes(const tcb_trie *t, size_t *bytes);
tcb_status tcb_trie_upload_codes(tcb_trie *t, void *d_buf, size_t bytes, void *stream);

/* Workspace for tcb_score_catalog calls of up to max_users users on this trie: the
 * normalised tables, the best score of every 16-SID group and 256-SID block per user,
 * and log-normaliser partials (about 4.3 bytes per user and leaf). */
tcb_status tcb_score_workspace_bytes(const tcb_trie *t, int32_t max_users, size_t *bytes);

/* Score every valid SID for n_users users and keep each user's best k.
 *   d_table     float [n_users][L][V]: per-position log-probabilities
 *               (TCB_TABLE_LOGPROB) or raw logits (TCB_TABLE_LOGITS)
 *   d_user_vec  bf16 bits [n_users][dim] and d_sid_emb bf16 bits [n_distinct][dim] in
 *               leaf order, both 16-byte aligned, or both NULL (no SID-level term);
 *               dim in {32, 64, 128, 256}
 *   sid_weight  w, a finite scalar
 *   k           1..TCB_SCORE_MAX_K
 *   outputs     d_leaf int32 [n_users][k] leaf ids (node id - node_offset[L]),
 *               d_score float [n_users][k], d_item int32 [n_users][k] (catalog row,
 *               may be NULL), d_lse float [n_users] (may be NULL: the log-normaliser
 *               is then not computed); rows past n_distinct get leaf -1, item -1 and
 *               score -inf
 * Inputs must be finite; at most TCB_SCORE_MAX_SIDS valid SIDs. Needs tcb_trie_upload
 * and tcb_trie_upload_codes first and a
 * workspace of tcb_score_workspace_bytes(t, n_users) (256-byte aligned). Asynchronous
 * on stream; no device memory is allocated. Errors: TCB_E_ARG, TCB_E_STATE (trie or
 * codes not uploaded), TCB_E_WORKSPACE, TCB_E_HIP. */
tcb_status tcb_score_catalog(const tcb_trie *t, int32_t n_users, const float *d_table,
                             int32_t table_kind, const void *d_user_vec, const void *d_sid_emb,
                             int32_t dim, float sid_weight, int32_t k, int32_t *d_leaf,
                             int32_t *d_item, float *d_score, float *d_lse, void *d_ws,
                             size_t ws_bytes, void *stream);

/* tcb_score_catalog for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same arguments and
 * results without the workspace. The scratch is a static array of TCB_SCORE_STATIC_SCRATCH
 * bytes per GPU, held until the process ends; calls on one GPU share it, so calls that
 * overlap on one GPU (concurrent streams or threads) race. A call needing more scratch
 * than that (tcb_score_workspace_bytes) returns TCB_E_WORKSPACE and launches nothing. No
 * allocation happens. Errors as tcb_score_catalog. */
#define TCB_SCORE_STATIC_SCRATCH (64u << 20)
tcb_status tcb_score_catalog_static(const tcb_trie *t, int32_t n_users, const float *d_table,
                                    int32_t table_kind, const void *d_user_vec, const void *d_sid_emb,
                                    int32_t dim, float sid_weight, int32_t k, int32_t *d_leaf,
                                    int32_t *d_item, float *d_score, float *d_lse, void *stream);

/* Diagnostics: record HIP events around the two kernels (scan, selection) of each of
 * the next `capacity` tcb_score_catalog calls in this process (0..100000; 0 stops
 * recording and releases the events). */
tcb_status tcb_score_enable_timing(int32_t capacity);

/* Synchronise the recorded events and report the summed durations (ms) of the scan and
 * selection kernels over the calls recorded since tcb_score_enable_timing, and their
 * number. Errors: TCB_E_STATE (timing not enabled), TCB_E_HIP. */
tcb_status tcb_score_timing(double *scan_ms, double *select_ms, int32_t *calls);

#ifdef __cplusplus
}
#endif
#endif /* TCB_H */
