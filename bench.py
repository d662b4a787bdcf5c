#!/usr/bin/env python3
"""Throughput of the catalog-constrained wide-beam decode on one MI355X.

One bench step = one full decode of the workload's batch on the GPU: admit every
request at the root, run L constrained beam steps (masked log-softmax, per-request
top-n, parent-gather / trie-advance); the last step also writes each request's ranked
beams into device buffers (the wave's finish outputs), so a decode is L steps and no
separate finalize pass.
The default workload is 32 requests x beam 512, L = 4, a catalog of 4M Zipf(1.1) SIDs
and bf16 logits N(0, 3^2). Inputs (trie image, per-step logits) are resident in HBM
before the timed region; consecutive decodes rotate through a pool of input copies
larger than the 256 MB Infinity Cache, so every decode streams its logits from HBM.
Decodes are replayed from captured HIP graphs, each holding ``--graph-decodes`` decodes of
consecutive input copies (a graph launch costs about 4 us on the GPU before its first kernel,
so it is paid once per group; ``--graph 0``: eager launches, one library call per step). The
line also gives ``ms_per_step_eager``: the same decodes launched eagerly, timed right after.

Also measured in the same run:
  * the other workloads as legs of their own ("legs"): 1 request x beam 50 (L = 3, 20k
    SIDs), 64 requests x beam 128 (L = 4, 1M Zipf SIDs, fp32), and the mixed decode wave
    (256 requests of widths 50..512 admitted FIFO under 32,768 slots, L = 5, 8M SIDs; a
    step there is one run of the whole workload), each with its tile kernel's roofline and
    the oracle timed beside it;
  * a 1 GiB device-to-device copy, the measured bandwidth beside the 8 TB/s spec;
  * per-kernel durations with HIP events on the launch stream (an eager pass);
  * the SID-range lm_head leg: 8 requests x beam 512, hidden 2048, its MFMA kernel
    against the bf16 dense peak;
  * the single-pass scoring leg: every SID of the same 4M catalog scored for 32 users
    (per-position logits plus a 64-dim SID-level term), top 512 kept per user; its scan
    kernel against the HBM peak;
  * the CPU oracle on a bounded sample of each workload, on every core (up to 16
    processes) and on one core, with the CPU's model name (a baseline, not a target); for
    the lm_head workload its fp64 product is timed apart from the steps.

Prints one JSON line on stdout. Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import multiprocessing as mp
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "constrained beam-rows×steps/sec and achieved HBM GB/s at B=512, 1 MI355X"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 matrix peak, published
STATE_BYTES = 8                 # node id + score read per live row
TRIE_BYTES = 8                  # child range (or first child + mask word) per live row
MERGE_WRITE_BYTES = 18          # node, score, parent slot, back-pointer (+ code) per survivor
KERNEL_SOURCES = ["trie_constrained_beam_amd/csrc/" + f for f in (
    "beam_device.h", "kernels.hip", "tile_bf16.hip", "tile_f32.hip", "tcb_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_tile_b512x32_l4_4m_zipf_bf16_traffic.txt")
SCORE_SOURCES = ["trie_constrained_beam_amd/csrc/score.hip", "trie_constrained_beam_amd/csrc/score_internal.h"]
SCORE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_score_scan_score_u32_k512_l4_4m_zipf_d64_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(path=TRAFFIC_FILE, sources=KERNEL_SOURCES):
    """HBM bytes per launch of a kernel from its committed counter profile, if that was
    taken on the current kernel source (else None)."""
    try:
        fields = dict(line.split(":", 1) for line in open(path) if ":" in line)
    except OSError:
        return None
    if fields.get("kernel_source_sha", "").strip() != kernel_source_sha(sources):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- CPU oracle
_CPU = {}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _oracle_request(i):
    """One request of the workload decoded by the oracle (its logits drawn here, untimed
    apart from the decode); returns (beam-rows x steps, seconds)."""
    import oracle
    from trie_constrained_beam_amd import synth
    wl, w = _CPU["wl"], _CPU["widths"][i]
    xs = [synth.logits_rowkeyed(wl.seed, t, i, w, wl.sigma, bf16=wl.bf16) for t in range(wl.L)]
    t0 = time.perf_counter()
    res = oracle.decode(_CPU["otrie"], w,
                        lambda t, pref: oracle.widen_logits(xs[t][:len(pref)], "bf16" if wl.bf16 else "f32"))
    el = time.perf_counter() - t0
    return sum(int(h["cand_parent"].max()) + 1 for h in res["history"]), el


def _oracle_lmhead_request(i):
    """One request of the lm_head workload: per step the fp64 product of its live rows'
    hidden states and the level's weights, then the step; returns (rows x steps, GEMM
    seconds, step seconds)."""
    import numpy as np
    import oracle
    wl, w, base = _CPU["wl"], _CPU["widths"][i], _CPU["bases"][i]
    hid, wts = _CPU["hidden"], _CPU["weights"]
    otrie = _CPU["otrie"]
    prefixes = np.zeros(1, dtype=np.uint64)
    scores = np.zeros(1)
    rows, t_gemm, t_step = 0, 0.0, 0.0
    for t in range(wl.L):
        r = prefixes.size
        rows += r
        t0 = time.perf_counter()
        x64 = oracle.lmhead_logits(hid[t][base:base + r], wts[t])
        t1 = time.perf_counter()
        h = oracle.expand_request(otrie, t, prefixes, scores, x64, w)
        t2 = time.perf_counter()
        t_gemm += t1 - t0
        t_step += t2 - t1
        prefixes, scores = h["prefix"], h["score"]
    return rows, t_gemm, t_step


def cpu_baseline(wl, cat, seconds, workers=None, lmhead=None):
    """The oracle decoding requests of this workload (one request per task, round robin)
    until ``seconds`` have passed, in ``workers`` processes (default: every core, at most
    16) or in this process (workers = 1); rows x steps per second of wall time. lmhead:
    (hidden [L] arrays, weights [L]) for the lm_head workload, whose fp64 GEMM is timed
    separately from the steps."""
    import oracle
    widths = list(wl.widths)
    _CPU.update(wl=wl, widths=widths, otrie=oracle.OracleTrie(cat),
                bases=[sum(widths[:i]) for i in range(len(widths))])
    if lmhead is not None:
        _CPU.update(hidden=lmhead[0], weights=lmhead[1])
    fn = _oracle_lmhead_request if lmhead is not None else _oracle_request
    cores = host_cores()
    workers = workers or max(1, min(16, cores))
    workers = min(workers, len(widths)) if lmhead is None else min(workers, len(widths))
    done_rows, n_req, gemm_s, step_s = 0, 0, 0.0, 0.0
    t0 = time.perf_counter()
    if workers == 1:
        while time.perf_counter() - t0 < seconds:
            out = fn(n_req % len(widths))
            done_rows += out[0]
            if lmhead is not None:
                gemm_s += out[1]
                step_s += out[2]
            n_req += 1
    else:
        ctx = mp.get_context("fork")             # before any GPU use in this process
        with ctx.Pool(workers) as pool:
            while time.perf_counter() - t0 < seconds:
                batch = [(n_req + k) % len(widths) for k in range(workers)]
                for out in pool.map(fn, batch):
                    done_rows += out[0]
                    if lmhead is not None:
                        gemm_s += out[1]
                        step_s += out[2]
                n_req += len(batch)
    el = time.perf_counter() - t0
    res = {"value": done_rows / el, "unit": "beam-rows x steps/s", "cores": workers, "kind": "oracle",
           "cpu": cpu_model(),
           "sample": f"{n_req} request decodes of this workload ({done_rows} beam-rows x steps) in "
                     f"{el:.1f} s, {workers} worker process{'es' if workers > 1 else ''} (one request each, "
                     f"numpy float64) on {host_cores()} cores available"}
    if lmhead is not None:
        res["gemm_seconds"] = gemm_s
        res["step_seconds"] = step_s
        res["sample"] += f"; of the requests' CPU time {gemm_s:.1f} s in the fp64 lm_head product, {step_s:.1f} s in the steps"
    return res


def cpu_baselines(wl, cat, seconds, lmhead=None, row_bytes=None):
    """The oracle on every core (up to 16 processes) and on one core; with row_bytes (the
    GPU roofline's algorithmic bytes per row-step) also its effective GB/s on those bytes."""
    many = cpu_baseline(wl, cat, seconds, None, lmhead)
    one = cpu_baseline(wl, cat, max(2.0, seconds / 3), 1, lmhead)
    many["one_core"] = {k: one[k] for k in ("value", "cores", "sample")}
    if row_bytes:
        many["effective_GBps"] = many["value"] * row_bytes / 1e9
        many["one_core"]["effective_GBps"] = one["value"] * row_bytes / 1e9
    return many


def row_bytes(wl):
    """Algorithmic bytes per row-step of a workload's step kernels (the roofline's figure)."""
    return 256 * (2 if wl.bf16 else 4) + STATE_BYTES + TRIE_BYTES


def child_sector_bytes(trie, nodes_by_step, dsize):
    """The child-sector lower bound of a decode: for every live row of every step, 64 bytes
    for each 64-byte sector of its logit row that holds a child of its node."""
    import numpy as np
    cb, cc, _ = trie.host_arrays()
    per = 64 // dsize                                  # codes per sector
    total = 0
    for nodes in nodes_by_step:
        nodes = np.asarray(nodes, dtype=np.int64)
        st, en = cb[nodes].astype(np.int64), cb[nodes + 1].astype(np.int64)
        cnt = en - st
        if cnt.sum() == 0:
            continue
        row = np.repeat(np.arange(nodes.size), cnt)
        first = np.repeat(st - np.concatenate(([0], np.cumsum(cnt)[:-1])), cnt)
        sec = cc[first + np.arange(cnt.sum())].astype(np.int64) // per
        new = np.ones(sec.size, dtype=bool)                 # codes ascend within a row
        new[1:] = (sec[1:] != sec[:-1]) | (row[1:] != row[:-1])
        total += 64 * int(new.sum())
    return total


# ----------------------------------------------------------------------------- GPU legs
def make_pool(tensors_fn, per_decode_bytes, pool_gib, multiple=1):
    """Copies of one decode's inputs filling at least ``pool_gib`` GiB, their count a multiple of
    ``multiple`` (the decodes per captured graph), so that graphs of that many decodes divide it."""
    n = max(1, math.ceil(pool_gib * 2 ** 30 / per_decode_bytes))
    n = -(-n // max(1, multiple)) * max(1, multiple)
    first = tensors_fn()
    return [first] + [[x.clone() for x in first] for _ in range(n - 1)]


def capture(decode, n):
    import torch
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                decode(c)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return graphs


def capture_groups(decode, n, group):
    """Graphs of ``group`` decodes each: graph i runs decode(i * group + j), j < group, for
    the n input copies (n a multiple of group)."""
    return capture(lambda i: [decode(i * group + j) for j in range(group)], n // group)


def decode_groups(steps, want, pool):
    """Decodes per graph: the largest divisor of both ``steps`` and the pool size that is at
    most ``want``, so that exactly ``steps`` decodes are timed and every copy is used."""
    return max(g for g in range(1, max(1, want) + 1) if steps % g == 0 and pool % g == 0)


def timed(run, steps, warmup):
    import torch
    for d in range(warmup):
        run(d)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for d in range(steps):
        run(d)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def verify_replay(trie, widths, xs, fin, ids, dev, step=None, read_mode="auto"):
    """The last timed decode's outputs (every pool copy holds the same inputs) against a
    decode of the same inputs with an export after every step, which runs each step's merge
    in the merge kernel and finalizes separately: bitwise equal, or the bench fails.
    step(beams, x): one step on input x (default: beams.step(x)); read_mode: the head or
    read mode of the timed decode."""
    import numpy as np
    import torch
    from trie_constrained_beam_amd import Beams
    torch.cuda.synchronize()
    idx = np.asarray(ids)
    got = {k: v.cpu().numpy()[idx] for k, v in fin.items()}
    ref_beams = Beams(trie, sum(widths), len(widths), max(widths), device=dev)
    ref_beams.set_read_mode(read_mode)
    rid, _ = ref_beams.init(widths)
    for x in xs:
        if step is None:
            ref_beams.step(x)
        else:
            step(ref_beams, x)
        ref_beams.export()
    ref = ref_beams.finalize(rid)
    ref_beams.check()
    for k in ("counts", "sids", "scores", "items"):
        if not np.array_equal(got[k], ref[k]):
            raise SystemExit(f"bench: the timed decode's {k} differ from the step-by-step decode")
    log(f"[bench] timed decode outputs equal a step-by-step decode of the same inputs (bitwise)")


def merge_steps(trie, widths, L, deferred=True):
    """Steps of a decode that launch the merge kernel: a step whose requests all have at
    most 64 possible rows (one tile; depth-t prefixes of the catalog, at most the beam
    width) is merged inside the tile kernel; with back-to-back plain steps (deferred) every
    other step's merge runs inside the next step's tile kernel, so only the last step's
    merge is launched."""
    npd = trie.nodes_per_depth
    wide = [max(min(w, 1 if t == 0 else npd[t]) for w in widths) > 64 for t in range(L)]
    return int(wide[L - 1]) if deferred else sum(wide)


def one_wave_leg(args, wl, cat, dev):
    """A one-wave workload (every request admitted at once): its decode captured per input
    copy and replayed, verified against a step-by-step decode, and its kernels timed."""
    import numpy as np
    import torch
    from trie_constrained_beam_amd import Beams, Trie, synth
    trie = Trie(cat, device=dev)
    widths = list(wl.widths)
    S, R, B, V, L = sum(widths), len(widths), max(widths), trie.V, trie.L
    beams = Beams(trie, S, R, B, device=dev)
    ids, bases = beams.init(widths)
    host = []
    for t in range(L):
        h = np.zeros((S, V), dtype=np.uint16 if wl.bf16 else np.float32)
        for i, (w, b) in enumerate(zip(widths, bases)):
            h[b:b + w] = synth.logits_rowkeyed(wl.seed, t, i, w, wl.sigma, bf16=wl.bf16)
        host.append(h)

    def upload():
        if wl.bf16:
            return [torch.from_numpy(h.view(np.int16)).to(dev).view(torch.bfloat16) for h in host]
        return [torch.from_numpy(h).to(dev) for h in host]
    per_decode = sum(h.nbytes for h in host)
    pool = make_pool(upload, per_decode, args.pool_gib, args.graph_decodes)
    fin = beams.set_finish_outputs(True)   # the last step writes each request's beams (row = id)
    log(f"[bench] pool {len(pool)} x {per_decode / 2**20:.1f} MiB of logits")
    rows_per_step, nodes_by_step = [], []
    idx = torch.as_tensor(ids, device=dev).long()
    for t in range(L):
        ex = beams.export()
        rows = ex["rows"][idx].cpu().numpy()
        node = ex["node"].cpu().numpy()
        rows_per_step.append(int(rows.sum()))
        nodes_by_step.append(np.concatenate([node[b:b + int(k)] for b, k in zip(bases, rows)]))
        beams.step(pool[0][t])
    torch.cuda.synchronize()
    rows_x_steps = sum(rows_per_step)
    sector_bytes = child_sector_bytes(trie, nodes_by_step, 2 if wl.bf16 else 4)
    log(f"[bench] live rows per step {rows_per_step} -> {rows_x_steps} rows x steps per decode; "
        f"child-sector bound {sector_bytes / rows_x_steps:.1f} B per row-step")

    def decode(c):
        rid, _ = beams.init(widths)
        for t in range(L):
            beams.step(pool[c][t])
    group = decode_groups(args.steps, args.graph_decodes, len(pool)) if args.graph else 1
    graphs = capture_groups(decode, len(pool), group) if args.graph else None

    def run(d):
        if graphs is not None:
            graphs[d % len(graphs)].replay()
        else:
            decode(d % len(pool))
    elapsed = timed(run, args.steps // group, -(-args.warmup // group))
    # the same decodes launched eagerly (one library call per step, no graph), for comparison
    n_eager = max(1, args.steps // 5)
    elapsed_eager = timed(lambda d: decode(d % len(pool)), n_eager, 5) / n_eager
    verify_replay(trie, widths, pool[0], fin, ids, dev)
    # the same decodes with the state brought up to date after every step but the last (each
    # merge then runs as its own kernel, as for a caller whose next logits depend on the
    # survivors), replayed from graphs of the same size; the outputs are verified again
    def decode_unfused(c):
        rid, _ = beams.init(widths)
        for t in range(L):
            beams.step(pool[c][t])
            if t + 1 < L:
                beams.flush()
    if max(widths) > 64:                     # beams of at most 64 rows merge in their tile kernel
        graphs_u = capture_groups(decode_unfused, len(pool), group) if args.graph else None
        n_unfused = max(group, args.steps // 5 // group * group)

        def run_u(d):
            if graphs_u is not None:
                graphs_u[d % len(graphs_u)].replay()
            else:
                decode_unfused(d % len(pool))
        elapsed_unfused = timed(run_u, n_unfused // group, 2) / n_unfused
        verify_replay(trie, widths, pool[0], fin, ids, dev)
        del graphs_u
    else:
        elapsed_unfused = elapsed / args.steps
    # per-kernel durations: the same decodes again, eagerly, with events on the launch stream
    # around 10 back-to-back launches of each kernel (dispatch latency amortised)
    n_ev = min(args.steps, 100)
    beams.enable_timing(n_ev * L, 10)
    for d in range(n_ev):
        decode(d % len(pool))
    _, tile_ms, merge_ms, n_timed = beams.timing()
    # cold: one launch per step, each decode on another input copy (logits from HBM)
    beams.enable_timing(n_ev * L, 1)
    for d in range(n_ev):
        decode((d + 1) % len(pool))
    _, tile_ms_c, _, n_timed_c = beams.timing()
    beams.enable_timing(0)
    n_merge = n_timed // L * merge_steps(trie, widths, L)    # merge launches among the timed steps
    return {"elapsed": elapsed, "rows_x_steps": rows_x_steps, "rows_per_step": rows_per_step,
            "graph_decodes": group if args.graph else 0, "eager_ms_per_decode": elapsed_eager * 1e3,
            "unfused_ms_per_decode": elapsed_unfused * 1e3,
            "tile_us": tile_ms * 1e3 / n_timed, "tile_us_cold": tile_ms_c * 1e3 / n_timed_c,
            "merge_us": merge_ms * 1e3 / n_merge if n_merge else None,
            "pool": len(pool), "sector_bytes": sector_bytes,
            "dsize": 2 if wl.bf16 else 4, "V": V, "L": L, "R": R, "B": B}


TRACE_ORDER = [1, 8, 11, 12, 13, 9, 10, 2, 14, 15, 3, 4, 5, 6, 7]
MERGE_TRACE_ORDER = [1, 8, 9, 11, 10]                # k_merge (11: ranks written, finishing merge)
TRACE_NAMES = {1: "start", 8: "counts", 11: "window", 12: "offsets", 13: "cand", 9: "staged", 10: "merged",
               14: "logits", 15: "keys",
               2: "prev-merge", 3: "softmax", 4: "prefilter", 5: "binned", 6: "in-tile-staged", 7: "done"}


def phase_trace(args, wl, cat, dev):
    """Phase marks of every workgroup of one decode of the workload, the last of a captured
    graph of ``--graph-decodes`` decodes (the timed route; ``--graph 0``: launched eagerly), run
    ``args.phase_trace`` times, each time right behind ``args.trace_behind`` untraced decodes of
    other input copies run back to back (0: after an idle GPU). Prints, per launch, the start skew
    across workgroups, the span from the first start to the last mark, and the median
    per-workgroup time between consecutive marks (100 MHz clock)."""
    import numpy as np
    import torch
    from trie_constrained_beam_amd import Beams, Trie, synth
    trie = Trie(cat, device=dev)
    widths = list(wl.widths)
    S, R, B, V, L = sum(widths), len(widths), max(widths), trie.V, trie.L
    beams = Beams(trie, S, R, B, device=dev)
    host = []
    for t in range(L):
        h = np.zeros((S, V), dtype=np.uint16 if wl.bf16 else np.float32)
        for i, w in enumerate(widths):
            base = sum(widths[:i])
            h[base:base + w] = synth.logits_rowkeyed(wl.seed, t, i, w, wl.sigma, bf16=wl.bf16)
        host.append(torch.from_numpy(h.view(np.int16) if wl.bf16 else h).to(dev))
    xs = [x.view(torch.bfloat16) if wl.bf16 else x for x in host]
    beams.set_finish_outputs(True)
    nb = args.trace_behind
    pool = [xs] + [[x.clone() for x in xs] for _ in range(nb)]

    def decode(c):
        beams.init(widths)
        for t in range(L):
            beams.step(pool[c][t])
    for d in range(3):
        decode(d % len(pool))
    torch.cuda.synchronize()
    group = max(1, args.graph_decodes) if args.graph else 1
    if args.graph:
        others = [o.replay for o in capture(lambda c: decode(c + 1), nb)] if nb else []
        beams.set_trace(64 * 2 ** 20 // 8)
        # a graph of `group` decodes, as the timed loop captures them; the last one is read
        run_traced = capture(lambda _: [decode(j % len(pool)) for j in range(group)], 1)[0].replay
    else:                                             # eager launches, one call per step
        beams.set_trace(64 * 2 ** 20 // 8)

        def other(c):
            beams.pause_trace(True)
            decode(c + 1)
        others = [lambda c=c: other(c) for c in range(nb)]

        def run_traced():
            beams.pause_trace(False)
            decode(0)
    reps = []
    for _ in range(args.phase_trace):
        for o in others:
            o()
        run_traced()
        torch.cuda.synchronize()
        tr = beams.trace()
        reps.append(tr[len(tr) - len(tr) // group:])     # the last decode's launches
        torch.cuda.synchronize()
    beams.set_trace(0)
    how = (f"replays of a graph of {group} decodes (the last one traced)" if args.graph else "eager decodes")
    lines = [f"# workload {wl.name}: {args.phase_trace} {how}, each behind {nb} other decodes run back to "
             f"back; times in us (median over runs; per-workgroup phases: median over workgroups)"]
    # timeline: each launch's first start and last mark, from the decode's first start
    tl = []
    for rep in reps:
        t0 = min(int(r[2][r[2][:, 0] > 0, 1].min()) for r in rep)
        row = []
        for r in rep:
            rec = r[2][r[2][:, 0] > 0]
            row.append(((rec[:, 1].min() - t0) / 100.0, (rec[:, 1:].max() - t0) / 100.0))
        tl.append(row)
    tl = np.median(np.asarray(tl), axis=0)
    lines.append("# timeline (first start .. last mark): " +
                 ", ".join(f"{a:.2f}..{b:.2f}" for a, b in tl) + f"; decode span {tl[-1][1]:.2f}")
    for li, (kind, level, _) in enumerate(reps[0]):
        recs = [r[li][2] for r in reps]
        name = {1: "tile", 2: "merge"}.get(kind, str(kind))
        skew, span, phases, xst = [], [], {}, []
        for rec in recs:
            ran = rec[:, 0] > 0
            rec = rec[ran]
            st = rec[:, 1]
            skew.append((st.max() - st.min()) / 100.0)
            xst.append([(st[rec[:, 0] == x + 1].min() - st.min()) / 100.0 if (rec[:, 0] == x + 1).any() else 0.0
                        for x in range(8)])
            last = rec[:, 2:].max(axis=1)
            span.append((np.maximum(last, st).max() - st.min()) / 100.0)
            order = MERGE_TRACE_ORDER if kind == 2 else TRACE_ORDER
            names = {**TRACE_NAMES, **({11: "ranked"} if kind == 2 else {})}
            marks = [m for m in order if (rec[:, m] > 0).any()]
            for a, b in zip(marks, marks[1:]):
                both = (rec[:, a] > 0) & (rec[:, b] > 0)
                if both.any():
                    phases.setdefault(f"{names[a]}->{names[b]}", []).append(
                        float(np.median(rec[both, b] - rec[both, a])) / 100.0)
        xcd = np.bincount(recs[0][recs[0][:, 0] > 0, 0] - 1, minlength=8)
        bx = [int(recs[0][b, 0]) - 1 for b in range(min(8, recs[0].shape[0]))]   # XCD of workgroups 0..7
        ph = ", ".join(f"{k} {np.median(v):.2f}" for k, v in phases.items())
        lines.append(f"{name:5s} level {level} workgroups {recs[0].shape[0]:4d} (ran {int((recs[0][:, 0] > 0).sum())}, "
                     f"per XCD {xcd.tolist()}, workgroups 0..7 on XCDs {bx}): start skew {np.median(skew):.2f} (first start per XCD "
                     f"{np.round(np.median(np.asarray(xst), axis=0), 2).tolist()}), span {np.median(span):.2f}; {ph}")
    print("\n".join(lines), flush=True)


def leg_summary(m, steps):
    """Throughput and the tile kernel's roofline of a measured leg."""
    value = m["rows_x_steps"] * steps / m["elapsed"]
    unit_bytes = m["V"] * m["dsize"] + STATE_BYTES + TRIE_BYTES          # per row-step, tile kernel
    launches = m.get("launches", m["L"])
    bytes_per_launch = m["rows_x_steps"] * unit_bytes / launches
    achieved = bytes_per_launch / (m["tile_us"] * 1e-6) / 1e9
    return value, unit_bytes, bytes_per_launch, achieved


def mixed_leg(args, wl, cat, dev):
    """The mixed decode wave: requests admitted FIFO under the slot budget between steps,
    finished requests released by the step that completes them, so the whole run of the
    workload (every request decoded) is one captured graph per input copy."""
    import numpy as np
    import torch
    from trie_constrained_beam_amd import Beams, Trie, synth
    trie = Trie(cat, device=dev)
    widths = list(wl.widths)
    L, S, V = wl.L, wl.slot_budget, trie.V
    beams = Beams(trie, S, len(widths), max(widths), device=dev)
    beams.set_finish_outputs(True)
    # the FIFO schedule does not depend on the logits: record it once with zero logits
    zero = torch.zeros((S, V), dtype=torch.float32, device=dev)
    sched = []                       # per step: (widths admitted before it, live (index, base, level))
    head, live = 0, []
    while head < len(widths) or live:
        st = beams.status()
        free, free_ids, take = st["free_slots"], st["free_requests"], []
        while head + len(take) < len(widths) and widths[head + len(take)] <= free and free_ids > 0:
            free -= widths[head + len(take)]
            free_ids -= 1
            take.append(head + len(take))
        admitted = []
        while take:
            try:
                rids, bases = beams.init([widths[i] for i in take])
                admitted = [(i, int(b)) for i, b in zip(take, bases)]
                break
            except Exception:                     # fragmented slots: admit fewer this time
                take.pop()
        head += len(admitted)
        live += [[i, b, 0] for i, b in admitted]
        sched.append(([widths[i] for i, _ in admitted], [tuple(e) for e in live]))
        beams.step(zero)
        for e in live:
            e[2] += 1
        live = [e for e in live if e[2] < L]
    torch.cuda.synchronize()
    host = []
    for _, lv in sched:
        h = np.zeros((S, V), dtype=np.float32)
        for i, b, level in lv:
            h[b:b + widths[i]] = synth.logits_rowkeyed(wl.seed, level, i, widths[i], wl.sigma)
        host.append(h)
    per_run = sum(h.nbytes for h in host)
    pool = make_pool(lambda: [torch.from_numpy(h).to(dev) for h in host], per_run, args.pool_gib)
    log(f"[bench] mixed wave: {len(widths)} requests in {len(sched)} steps; pool {len(pool)} x "
        f"{per_run / 2**20:.0f} MiB of logits")

    def run_once(c):
        for s_i, (admit, _) in enumerate(sched):
            if admit:
                beams.init(admit)
            beams.step(pool[c][s_i])

    # rows x steps of one run: the live rows of every step, exported along an eager run
    rows = []
    id_of = {}
    head2 = 0
    for s_i, (admit, lv) in enumerate(sched):
        if admit:
            rids, _ = beams.init(admit)
            for k, rid in enumerate(rids):
                id_of[head2 + k] = int(rid)
            head2 += len(admit)
        ex = beams.export()["rows"].cpu().numpy()
        rows.append(int(sum(ex[id_of[i]] for i, _, _ in lv)))
        beams.step(pool[0][s_i])
    torch.cuda.synchronize()
    rows_x_steps = sum(rows)
    graphs = capture(run_once, len(pool)) if args.graph else None

    def run(d):
        if graphs is not None:
            graphs[d % len(pool)].replay()
        else:
            run_once(d % len(pool))
    steps = max(5, args.steps // 4)
    elapsed = timed(run, steps, max(2, args.warmup // 4))
    n_ev = min(steps, 20)
    beams.enable_timing(n_ev * len(sched), 10)
    for d in range(n_ev):
        run_once(d % len(pool))
    _, tile_ms, merge_ms, n_timed = beams.timing()
    beams.enable_timing(0)
    return {"elapsed": elapsed, "steps": steps, "rows_x_steps": rows_x_steps, "rows_per_step": rows,
            "tile_us": tile_ms * 1e3 / n_timed, "merge_ms_per_run": merge_ms / max(1, n_timed // len(sched)),
            "pool": len(pool), "dsize": 4, "V": V, "L": L, "launches": len(sched), "R": len(widths),
            "B": max(widths)}


def copy_peak(dev, gib=1.0):
    """A device-to-device copy of ``gib`` GiB: read + write bytes per second (GB/s)."""
    import torch
    n = int(gib * 2 ** 30)
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    reps = 20
    t0 = time.perf_counter()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    return 2.0 * n * reps / el / 1e9


def lmhead_leg(args, dev, read_mode="dense"):
    """The fused lm_head workload. read_mode "dense": the MFMA head at every level (its
    roofline); "auto": the library's per-level choice (the children-only head only where
    rows touch at most one 4-code piece on average)."""
    import numpy as np
    import torch
    from trie_constrained_beam_amd import Beams, Trie, synth
    wl = synth.WORKLOADS["lmhead_b512x8_l4_1m_h2048"]
    cat = wl.catalog()
    trie = Trie(cat, device=dev)
    widths = list(wl.widths)
    S, R, B, L, H = sum(widths), len(widths), max(widths), wl.L, wl.hidden
    beams = Beams(trie, S, R, B, device=dev)
    beams.set_read_mode(read_mode)
    weights = np.stack([synth.lmhead_weight(wl.seed, lv, 256, H) for lv in range(L)])
    w_dev = torch.from_numpy(weights.view(np.int16)).to(dev).view(torch.bfloat16)
    host = [synth.hidden_states(wl.seed, t, S, H) for t in range(L)]
    per_decode = sum(h.nbytes for h in host)
    pool = make_pool(lambda: [torch.from_numpy(h.view(np.int16)).to(dev).view(torch.bfloat16) for h in host],
                     per_decode, args.pool_gib, args.graph_decodes)
    fin = beams.set_finish_outputs(True)   # the last step writes each request's beams (row = id)
    ids, _ = beams.init(widths)
    rows_per_step = []
    idx = torch.as_tensor(ids, device=dev).long()
    for t in range(L):
        rows_per_step.append(int(beams.export()["rows"][idx].sum().item()))
        beams.step_lmhead(pool[0][t], w_dev)
    torch.cuda.synchronize()

    def decode(c):
        rid, _ = beams.init(widths)
        for t in range(L):
            beams.step_lmhead(pool[c][t], w_dev)
    steps = max(10, args.steps // 5)
    group = decode_groups(steps, args.graph_decodes, len(pool)) if args.graph else 1
    graphs = capture_groups(decode, len(pool), group) if args.graph else None

    def run(d):
        if graphs is not None:
            graphs[d % len(graphs)].replay()
        else:
            decode(d % len(pool))
    elapsed = timed(run, steps // group, -(-max(2, args.warmup // 5) // group))
    verify_replay(trie, widths, pool[0], fin, ids, dev,
                  step=lambda b, x: b.step_lmhead(x, w_dev), read_mode=read_mode)
    n_ev = min(steps, 50)
    beams.enable_timing(n_ev * L, 10)
    for d in range(n_ev):
        decode(d % len(pool))
    head_ms, tile_ms, merge_ms, n_timed = beams.timing()
    # cold: one launch per step, each decode on another copy of the hidden states (from HBM)
    beams.enable_timing(n_ev * L, 1)
    for d in range(n_ev):
        decode((d + 1) % len(pool))
    head_ms_c, _, _, n_timed_c = beams.timing()
    beams.enable_timing(0)
    n_merge = n_timed // L * merge_steps(trie, widths, L)
    rows_x_steps = sum(rows_per_step)
    head_s = head_ms / 1e3 / n_timed                       # average head launch(es) per step
    head_s_c = head_ms_c / 1e3 / n_timed_c
    res = {"workload": wl.name, "read_mode": read_mode, "rows_per_step": rows_per_step,
           "value": rows_x_steps * steps / elapsed, "unit": "beam-rows x steps/s",
           "ms_per_step": elapsed * 1e3 / steps, "steps": steps, "graph_decodes": group if args.graph else 0,
           "head_avg_us": head_s * 1e6,
           "head_avg_us_cold": head_s_c * 1e6,
           "tile_avg_us": tile_ms * 1e3 / n_timed, "merge_avg_us": merge_ms * 1e3 / n_merge if n_merge else None}
    if read_mode == "dense":
        flop_per_decode = 2.0 * rows_x_steps * 256 * H
        achieved = flop_per_decode / L / head_s / 1e12
        res["roofline"] = {"bound": "mfma", "kernel": "k_lmhead", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None,
                           "flop_per_launch": flop_per_decode / L, "avg_launch_us": head_s * 1e6,
                           "timing": "warm: 10 back-to-back launches on the same hidden states",
                           "avg_launch_us_cold": head_s_c * 1e6,
                           "achieved_cold": flop_per_decode / L / head_s_c / 1e12}
        log(f"[bench] lm_head leg: rows per step {rows_per_step}; lm_head avg {head_s * 1e6:.2f} us "
            f"({achieved:.0f} TFLOP/s), tile {res['tile_avg_us']:.2f} us"
            + (f", merge {res['merge_avg_us']:.2f} us" if res["merge_avg_us"] is not None else ""))
    else:
        log(f"[bench] lm_head leg ({read_mode}): {elapsed * 1e3 / steps:.3f} ms per decode, head avg "
            f"{head_s * 1e6:.2f} us per step")
    return res


def _score_inputs(wl, trie, dev):
    import numpy as np
    import torch
    from trie_constrained_beam_amd import synth
    table = torch.from_numpy(synth.score_logits(wl.seed, wl.users, trie.L, wl.sigma)).to(dev)
    uvec_h = synth.user_vectors(wl.seed, wl.users, wl.dim)
    emb_h = synth.sid_embeddings(wl.seed, trie.n_distinct, wl.dim)
    uvec = torch.from_numpy(uvec_h.view(np.int16)).to(dev).view(torch.bfloat16)
    emb = torch.from_numpy(emb_h.view(np.int16)).to(dev).view(torch.bfloat16)
    return table, uvec, emb, uvec_h, emb_h


def score_cpu_baseline(wl, cat, seconds):
    """The oracle scoring every SID for users of this workload, one after another, until
    ``seconds`` have passed; user-SID scores per second."""
    import numpy as np
    import oracle
    from trie_constrained_beam_amd import synth
    otrie = oracle.OracleTrie(cat)
    tab = synth.score_logits(wl.seed, wl.users, otrie.L, wl.sigma)
    u64 = oracle.widen_logits(synth.user_vectors(wl.seed, wl.users, wl.dim), "bf16")
    e64 = oracle.widen_logits(synth.sid_embeddings(wl.seed, otrie.n_distinct, wl.dim), "bf16")
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        u = done % wl.users
        oracle.score_catalog(otrie, tab[u].astype(np.float64), wl.k, oracle.TABLE_LOGITS, u64[u], e64, 1.0)
        done += 1
    el = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    return {"value": done * otrie.n_distinct / el, "unit": "user-SID scores/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} users x {otrie.n_distinct} SIDs scored and ranked in {el:.1f} s (numpy float64, "
                      f"one process; its BLAS product may use up to {threads} threads)"}


def score_leg(args, cat, dev):
    import ctypes as C
    import torch
    from trie_constrained_beam_amd import Trie, score_catalog, score_workspace_bytes, synth
    from trie_constrained_beam_amd import _lib
    wl = synth.SCORE_WORKLOADS["score_u32_k512_l4_4m_zipf_d64"]
    trie = Trie(cat, device=dev).upload_codes(dev)
    n = trie.n_distinct
    table, uvec, emb, _, _ = _score_inputs(wl, trie, dev)
    ws = torch.empty(score_workspace_bytes(trie, wl.users), dtype=torch.uint8, device=dev)

    def run(_):
        score_catalog(trie, table, wl.k, "logits", uvec, emb, 1.0, want_lse=True, workspace=ws)
    steps = max(10, args.steps // 20)
    elapsed = timed(run, steps, max(2, args.warmup // 5))
    n_ev = min(steps, 50)
    lib = _lib.lib()
    _lib.check(lib.tcb_score_enable_timing(n_ev))
    for d in range(n_ev):
        run(d)
    s_ms, x_ms, calls = C.c_double(), C.c_double(), C.c_int32()
    _lib.check(lib.tcb_score_timing(C.byref(s_ms), C.byref(x_ms), C.byref(calls)))
    _lib.check(lib.tcb_score_enable_timing(0))
    k = max(1, calls.value)
    scan_us, sel_us = s_ms.value * 1e3 / k, x_ms.value * 1e3 / k
    code_bytes = 4 if trie.L <= 4 else 8
    unit_bytes = code_bytes + 2 * wl.dim                     # per SID and group of 32 users
    groups = -(-wl.users // 32)
    bytes_per_launch = float(n) * unit_bytes * groups
    achieved = bytes_per_launch / (scan_us * 1e-6) / 1e9
    traffic = recorded_traffic(SCORE_TRAFFIC_FILE, SCORE_SOURCES)
    value = wl.users * n * steps / elapsed
    log(f"[bench] scoring leg: {wl.users} users x {n} SIDs, top {wl.k}: {elapsed * 1e3 / steps:.3f} ms per call; "
        f"scan {scan_us:.1f} us ({achieved:.0f} GB/s), select {sel_us:.1f} us")
    return {"workload": wl.name, "value": value, "unit": "user-SID scores/s", "steps": steps,
            "ms_per_step": elapsed * 1e3 / steps, "users": wl.users, "sids": n, "dim": wl.dim, "k": wl.k,
            "roofline": {"bound": "hbm", "kernel": "k_score_scan", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                         "traffic": None if traffic is None else traffic / (scan_us * 1e-6) / 1e9,
                         "traffic_bytes_per_launch": traffic,
                         "bytes_per_sid": unit_bytes, "bytes_per_launch": bytes_per_launch,
                         "avg_launch_us": scan_us},
            "select_avg_us": sel_us,
            "kernel_source_sha": kernel_source_sha(SCORE_SOURCES)}


ONE_WAVE_LEGS = ["b50x1_l3_20k_f32", "b128x64_l4_1m_zipf_f32"]
MIXED_LEG = "mixed256_l5_8m_f32"


def roofline_extra(m, bytes_per_launch):
    """The step kernels timed cold (one launch per step, inputs from another copy each
    decode) and the decode's child-sector lower bound, beside the warm roofline."""
    out = {"timing": "warm: 10 back-to-back launches of each step's kernel on the same inputs"}
    if m.get("tile_us_cold"):
        out["avg_launch_us_cold"] = m["tile_us_cold"]
        out["achieved_cold"] = bytes_per_launch / (m["tile_us_cold"] * 1e-6) / 1e9
    if m.get("sector_bytes"):
        out["child_sector_bytes_per_row_step"] = m["sector_bytes"] / m["rows_x_steps"]
    return out


def leg_record(wl, m, steps, cat, cpu):
    """The JSON record of a measured one-wave or mixed leg."""
    value, unit_bytes, bpl, achieved = leg_summary(m, steps)
    rec = {"workload": wl.name, "value": value, "unit": "beam-rows x steps/s", "steps": steps,
           "ms_per_step": m["elapsed"] * 1e3 / steps, "requests": m["R"], "beam_width": m["B"], "L": m["L"],
           "ms_per_step_unfused": m.get("unfused_ms_per_decode"),
           "catalog": int(cat.shape[0]), "rows_per_step": m["rows_per_step"], "rows_x_steps_per_decode":
           m["rows_x_steps"], "input_pool_copies": m["pool"], "decodes_per_graph": m.get("graph_decodes"),
           "roofline": {"bound": "hbm", "kernel": "k_tile", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                        "bytes_per_row_step": unit_bytes, "bytes_per_launch": bpl, "avg_launch_us": m["tile_us"],
                        **roofline_extra(m, bpl)},
           "cpu_baseline": cpu}
    if m.get("merge_us") is not None:
        rec["merge_avg_us"] = m["merge_us"]
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000, help="timed decodes")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b512x32_l4_4m_zipf_bf16")
    ap.add_argument("--pool-gib", type=float, default=1.0, help="size of each rotated input pool")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle baseline budget (0: skip)")
    ap.add_argument("--graph", type=int, default=1, help="replay the decodes from captured HIP graphs")
    ap.add_argument("--graph-decodes", type=int, default=8,
                    help="decodes (of consecutive input copies) per captured graph, at most")
    ap.add_argument("--lmhead", type=int, default=1, help="also run the SID-range lm_head leg")
    ap.add_argument("--score", type=int, default=1, help="also run the single-pass scoring leg")
    ap.add_argument("--legs", type=int, default=1, help="also run the other workloads' legs")
    ap.add_argument("--phase-trace", type=int, default=0,
                    help="only print the phase trace of one decode replayed this many times (diagnostics)")
    ap.add_argument("--trace-behind", type=int, default=16,
                    help="phase trace: untraced decodes (other input copies) replayed before each traced one")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): requests "
              "are independent, so the path shards by request with no per-step communication; "
              "run one process per GPU instead.", file=sys.stderr)
        sys.exit(2)

    from trie_constrained_beam_amd import synth
    wl = synth.WORKLOADS[args.workload]
    if wl.slot_budget or wl.hidden:
        raise SystemExit(f"workload {wl.name} is a parity case, not a bench line")
    t0 = time.perf_counter()
    cat = wl.catalog()
    log(f"[bench] catalog {cat.shape} in {time.perf_counter() - t0:.1f}s")
    if args.phase_trace:
        import torch
        torch.cuda.set_device(0)
        phase_trace(args, wl, cat, torch.device("cuda:0"))
        return
    legs = [synth.WORKLOADS[n] for n in ONE_WAVE_LEGS + [MIXED_LEG] if args.legs and n != wl.name]
    cats = {w.name: w.catalog() for w in legs}
    lm_wl = synth.WORKLOADS["lmhead_b512x8_l4_1m_h2048"]
    lm_cat = lm_wl.catalog() if args.lmhead else None
    # the CPU oracle first: its worker processes are forked before this process touches the GPU
    cpu = score_cpu = None
    leg_cpu, lm_cpu = {}, None
    if args.cpu_seconds > 0:
        cpu = cpu_baselines(wl, cat, args.cpu_seconds, row_bytes=row_bytes(wl))
        log(f"[bench] oracle {cpu['value']:.0f} rows x steps/s ({cpu['cores']} processes), "
            f"{cpu['one_core']['value']:.0f} on one core; {cpu['cpu']}")
        for w in legs:
            leg_cpu[w.name] = cpu_baselines(w, cats[w.name], max(3.0, args.cpu_seconds / 3), row_bytes=row_bytes(w))
            log(f"[bench] oracle {w.name}: {leg_cpu[w.name]['value']:.0f} rows x steps/s")
        if args.lmhead:
            import numpy as np
            S = sum(lm_wl.widths)
            hid = [synth.hidden_states(lm_wl.seed, t, S, lm_wl.hidden) for t in range(lm_wl.L)]
            wts = [synth.lmhead_weight(lm_wl.seed, lv, 256, lm_wl.hidden) for lv in range(lm_wl.L)]
            lm_cpu = cpu_baselines(lm_wl, lm_cat, max(3.0, args.cpu_seconds / 3), lmhead=(hid, wts))
            log(f"[bench] oracle lm_head workload: {lm_cpu['value']:.0f} rows x steps/s")
        if args.score:
            swl = synth.SCORE_WORKLOADS["score_u32_k512_l4_4m_zipf_d64"]
            score_cpu = score_cpu_baseline(swl, cat if swl.catalog_of == wl.name else swl.catalog(),
                                           max(3.0, args.cpu_seconds / 3))
            log(f"[bench] oracle scoring {score_cpu['value']:.3g} user-SID scores/s")

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copy_gbps = copy_peak(dev)
    log(f"[bench] 1 GiB device-to-device copy: {copy_gbps:.0f} GB/s (read + write)")
    m = one_wave_leg(args, wl, cat, dev)
    value, unit_bytes, bytes_per_launch, achieved = leg_summary(m, args.steps)
    traffic = recorded_traffic()
    log(f"[bench] {args.steps} decodes ({m['graph_decodes']} per graph) in {m['elapsed'] * 1e3:.1f} ms; "
        f"tile kernel avg {m['tile_us']:.2f} us "
        f"({achieved:.0f} GB/s)" + (f", merge kernel avg {m['merge_us']:.2f} us" if m["merge_us"] is not None else ""))
    leg_out = {}
    for w in legs:
        if w.slot_budget:
            lm_ = mixed_leg(args, w, cats[w.name], dev)
            st = lm_["steps"]
        else:
            a2 = argparse.Namespace(**vars(args))
            a2.steps = args.steps * (50 if w.name == "b50x1_l3_20k_f32" else 1)
            lm_ = one_wave_leg(a2, w, cats[w.name], dev)
            st = a2.steps
        leg_out[w.name] = leg_record(w, lm_, st, cats[w.name], leg_cpu.get(w.name))
        r = leg_out[w.name]
        log(f"[bench] leg {w.name}: {r['value']:.4g} rows x steps/s, {r['ms_per_step'] * 1e3:.1f} us per decode; "
            f"tile avg {r['roofline']['avg_launch_us']:.2f} us ({r['roofline']['achieved']:.0f} GB/s)")
    lm = None
    if args.lmhead:
        lm = lmhead_leg(args, dev, "dense")
        lm["auto"] = lmhead_leg(args, dev, "auto")
        lm["cpu_baseline"] = lm_cpu
    sc = None
    if args.score:
        swl = synth.SCORE_WORKLOADS["score_u32_k512_l4_4m_zipf_d64"]
        sc = score_leg(args, cat if swl.catalog_of == wl.name else swl.catalog(), dev)
        sc["cpu_baseline"] = score_cpu

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "beam-rows x steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["elapsed"] * 1e3 / args.steps,
        "ms_per_step_eager": m["eager_ms_per_decode"],
        "ms_per_step_unfused": m["unfused_ms_per_decode"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "requests": m["R"], "beam_width": m["B"], "L": m["L"],
                   "catalog": int(cat.shape[0]), "catalog_levels": "zipf(1.1) at every level",
                   "logits": ("bf16" if wl.bf16 else "f32") + f" N(0,{wl.sigma:g}^2), upcast to f32",
                   "rows_x_steps_per_decode": m["rows_x_steps"], "rows_per_step": m["rows_per_step"],
                   "graph": bool(args.graph), "decodes_per_graph": m["graph_decodes"],
                   "input_pool_copies": m["pool"]},
        "roofline": {"bound": "hbm", "kernel": "k_tile", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None if traffic is None else traffic / (m["tile_us"] * 1e-6) / 1e9,
                     "traffic_bytes_per_launch": traffic, "bytes_per_row_step": unit_bytes, "bytes_per_launch": bytes_per_launch,
                     "avg_launch_us": m["tile_us"], "measured_copy_GBps": copy_gbps,
                     **roofline_extra(m, bytes_per_launch)},
        "hbm_GBps_wall": m["rows_x_steps"] * (unit_bytes + MERGE_WRITE_BYTES) * args.steps / m["elapsed"] / 1e9,
        "merge_avg_us": m["merge_us"],
        "legs": leg_out,
        "lmhead": lm,
        "score": sc,
        "cpu_baseline": cpu,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
