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
Each decode is replayed as a captured HIP graph (``--graph 0``: eager launches).

Also measured in the same run:
  * per-kernel durations with HIP events on the launch stream (an eager pass);
  * the SID-range lm_head leg: 8 requests x beam 512, hidden 2048, its MFMA kernel
    against the bf16 dense peak;
  * the single-pass scoring leg: every SID of the same 4M catalog scored for 32 users
    (per-position logits plus a 64-dim SID-level term), top 512 kept per user; its scan
    kernel against the HBM peak;
  * the CPU oracle on a bounded sample of the same workload (a baseline, not a target).

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
KERNEL_SOURCES = ["trie_constrained_beam_amd/csrc/kernels.hip", "trie_constrained_beam_amd/csrc/tcb_internal.h"]
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


def _oracle_request(i):
    import oracle
    wl, widths, xs = _CPU["wl"], _CPU["widths"], _CPU["xs"][i]
    res = oracle.decode(_CPU["otrie"], widths[i],
                        lambda t, pref: oracle.widen_logits(xs[t][:len(pref)], "bf16" if wl.bf16 else "f32"))
    return sum(int(h["cand_parent"].max()) + 1 for h in res["history"])


def cpu_baseline(wl, cat, seconds):
    """The oracle decoding requests of this workload in a process pool (one request per
    task) until ``seconds`` have passed; rows x steps per second of wall time."""
    import oracle
    from trie_constrained_beam_amd import synth
    widths = list(wl.widths)
    _CPU.update(wl=wl, widths=widths, otrie=oracle.OracleTrie(cat),
                xs=[[synth.logits_rowkeyed(wl.seed, t, i, w, wl.sigma, bf16=wl.bf16) for t in range(wl.L)]
                    for i, w in enumerate(widths)])
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    workers = max(1, min(16, cores, len(widths)))
    ctx = mp.get_context("fork")                 # before any GPU use in this process
    done_rows, n_req = 0, 0
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        while time.perf_counter() - t0 < seconds:
            batch = [(n_req + k) % len(widths) for k in range(workers)]
            done_rows += sum(pool.map(_oracle_request, batch))
            n_req += len(batch)
    el = time.perf_counter() - t0
    return {"value": done_rows / el, "unit": "beam-rows x steps/s", "cores": workers, "kind": "oracle",
            "sample": f"{n_req} request decodes of this workload ({done_rows} beam-rows x steps) in "
                      f"{el:.1f} s, {workers} worker processes (one request each, numpy float64) on "
                      f"{platform.machine()} with {cores} cores available"}


# ----------------------------------------------------------------------------- GPU legs
def make_pool(tensors_fn, per_decode_bytes, pool_gib):
    n = max(1, math.ceil(pool_gib * 2 ** 30 / per_decode_bytes))
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


def merge_steps(trie, widths, L, deferred=True):
    """Steps of a decode that launch the merge kernel: a step whose requests all have at
    most 64 possible rows (one tile; depth-t prefixes of the catalog, at most the beam
    width) is merged inside the tile kernel; with back-to-back plain steps (deferred) every
    other step's merge runs inside the next step's tile kernel, so only the last step's
    merge is launched."""
    npd = trie.nodes_per_depth
    wide = [max(min(w, 1 if t == 0 else npd[t]) for w in widths) > 64 for t in range(L)]
    return int(wide[L - 1]) if deferred else sum(wide)


def main_leg(args, wl, cat, dev):
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
    pool = make_pool(upload, per_decode, args.pool_gib)
    beams.set_finish_outputs(True)       # the last step writes each request's beams (row = id)
    log(f"[bench] pool {len(pool)} x {per_decode / 2**20:.1f} MiB of logits")
    rows_per_step = []
    idx = torch.as_tensor(ids, device=dev).long()
    for t in range(L):
        rows_per_step.append(int(beams.export()["rows"][idx].sum().item()))
        beams.step(pool[0][t])
    torch.cuda.synchronize()
    rows_x_steps = sum(rows_per_step)
    log(f"[bench] live rows per step {rows_per_step} -> {rows_x_steps} rows x steps per decode")

    def decode(c):
        rid, _ = beams.init(widths)
        for t in range(L):
            beams.step(pool[c][t])
    graphs = capture(decode, len(pool)) if args.graph else None

    def run(d):
        if graphs is not None:
            graphs[d % len(pool)].replay()
        else:
            decode(d % len(pool))
    elapsed = timed(run, args.steps, args.warmup)
    # per-kernel durations: the same decodes again, eagerly, with events on the launch stream
    # around 10 back-to-back launches of each kernel (dispatch latency amortised)
    n_ev = min(args.steps, 100)
    beams.enable_timing(n_ev * L, 10)
    for d in range(n_ev):
        decode(d % len(pool))
    _, tile_ms, merge_ms, n_timed = beams.timing()
    beams.enable_timing(0)
    n_merge = n_timed // L * merge_steps(trie, widths, L)    # merge launches among the timed steps
    return {"elapsed": elapsed, "rows_x_steps": rows_x_steps, "rows_per_step": rows_per_step,
            "tile_us": tile_ms * 1e3 / n_timed, "merge_us": merge_ms * 1e3 / max(1, n_merge), "pool": len(pool),
            "dsize": 2 if wl.bf16 else 4, "V": V, "L": L, "R": R, "B": B}


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
                     per_decode, args.pool_gib)
    beams.set_finish_outputs(True)       # the last step writes each request's beams (row = id)
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
    graphs = capture(decode, len(pool)) if args.graph else None

    def run(d):
        if graphs is not None:
            graphs[d % len(pool)].replay()
        else:
            decode(d % len(pool))
    steps = max(10, args.steps // 5)
    elapsed = timed(run, steps, max(2, args.warmup // 5))
    n_ev = min(steps, 50)
    beams.enable_timing(n_ev * L, 10)
    for d in range(n_ev):
        decode(d % len(pool))
    head_ms, tile_ms, merge_ms, n_timed = beams.timing()
    beams.enable_timing(0)
    n_merge = n_timed // L * merge_steps(trie, widths, L)
    rows_x_steps = sum(rows_per_step)
    head_s = head_ms / 1e3 / n_timed                       # average head launch(es) per step
    res = {"workload": wl.name, "read_mode": read_mode, "rows_per_step": rows_per_step,
           "value": rows_x_steps * steps / elapsed, "unit": "beam-rows x steps/s",
           "ms_per_step": elapsed * 1e3 / steps, "steps": steps, "head_avg_us": head_s * 1e6,
           "tile_avg_us": tile_ms * 1e3 / n_timed, "merge_avg_us": merge_ms * 1e3 / max(1, n_merge)}
    if read_mode == "dense":
        flop_per_decode = 2.0 * rows_x_steps * 256 * H
        achieved = flop_per_decode / L / head_s / 1e12
        res["roofline"] = {"bound": "mfma", "kernel": "k_lmhead", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None,
                           "flop_per_launch": flop_per_decode / L, "avg_launch_us": head_s * 1e6}
        log(f"[bench] lm_head leg: rows per step {rows_per_step}; lm_head avg {head_s * 1e6:.2f} us "
            f"({achieved:.0f} TFLOP/s), tile {res['tile_avg_us']:.2f} us, merge {res['merge_avg_us']:.2f} us")
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000, help="timed decodes")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b512x32_l4_4m_zipf_bf16")
    ap.add_argument("--pool-gib", type=float, default=1.0, help="size of each rotated input pool")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle baseline budget (0: skip)")
    ap.add_argument("--graph", type=int, default=1, help="replay each decode as a captured HIP graph")
    ap.add_argument("--lmhead", type=int, default=1, help="also run the SID-range lm_head leg")
    ap.add_argument("--score", type=int, default=1, help="also run the single-pass scoring leg")
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
    cpu = score_cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(wl, cat, args.cpu_seconds)
        log(f"[bench] oracle {cpu['value']:.0f} rows x steps/s ({cpu['cores']} processes)")
        if args.score:
            swl = synth.SCORE_WORKLOADS["score_u32_k512_l4_4m_zipf_d64"]
            score_cpu = score_cpu_baseline(swl, cat if swl.catalog_of == wl.name else swl.catalog(),
                                           max(3.0, args.cpu_seconds / 3))
            log(f"[bench] oracle scoring {score_cpu['value']:.3g} user-SID scores/s")

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = main_leg(args, wl, cat, dev)
    value = m["rows_x_steps"] * args.steps / m["elapsed"]
    unit_bytes = m["V"] * m["dsize"] + STATE_BYTES + TRIE_BYTES          # per row-step, tile kernel
    bytes_per_launch = m["rows_x_steps"] * unit_bytes / m["L"]
    achieved = bytes_per_launch / (m["tile_us"] * 1e-6) / 1e9
    traffic = recorded_traffic()
    log(f"[bench] {args.steps} decodes in {m['elapsed'] * 1e3:.1f} ms; tile kernel avg {m['tile_us']:.2f} us "
        f"({achieved:.0f} GB/s), merge kernel avg {m['merge_us']:.2f} us")
    lm = None
    if args.lmhead:
        lm = lmhead_leg(args, dev, "dense")
        lm["auto"] = lmhead_leg(args, dev, "auto")
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
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "requests": m["R"], "beam_width": m["B"], "L": m["L"],
                   "catalog": int(cat.shape[0]), "catalog_levels": "zipf(1.1) at every level",
                   "logits": ("bf16" if wl.bf16 else "f32") + f" N(0,{wl.sigma:g}^2), upcast to f32",
                   "rows_x_steps_per_decode": m["rows_x_steps"], "rows_per_step": m["rows_per_step"],
                   "graph": bool(args.graph), "input_pool_copies": m["pool"]},
        "roofline": {"bound": "hbm", "kernel": "k_tile", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None if traffic is None else traffic / (m["tile_us"] * 1e-6) / 1e9,
                     "traffic_bytes_per_launch": traffic, "bytes_per_row_step": unit_bytes, "bytes_per_launch": bytes_per_launch,
                     "avg_launch_us": m["tile_us"]},
        "hbm_GBps_wall": m["rows_x_steps"] * (unit_bytes + MERGE_WRITE_BYTES) * args.steps / m["elapsed"] / 1e9,
        "merge_avg_us": m["merge_us"],
        "lmhead": lm,
        "score": sc,
        "cpu_baseline": cpu,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
