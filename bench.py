#!/usr/bin/env python3
"""Throughput of the catalog-constrained wide-beam decode on one MI355X.

One bench step = one full decode of the workload's batch on the GPU: admit every
request at the root, run L constrained beam steps (masked log-softmax, per-request
top-n, parent-gather / trie-advance) and gather the ranked beams into device
buffers. Inputs (trie image, per-step logits) are resident in HBM before the timed
region; the logits of consecutive decodes come from a pool of identical copies
larger than the 256 MB Infinity Cache, so every decode streams them from HBM.

Prints one JSON line. Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
EXPAND_STATE_BYTES = 8           # node id + score per live row
EXPAND_TRIE_BYTES = 8            # first/last child id (or first child id + mask word) per row
MERGE_WRITE_BYTES = 18           # node, score, parent slot, back-pointer (+ code) per survivor


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000, help="timed decodes")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b512x32_l4_4m_zipf_bf16")
    ap.add_argument("--pool-gib", type=float, default=1.0, help="size of the rotated logits pool")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle baseline budget (0: skip)")
    ap.add_argument("--graph", type=int, default=0, help="replay each decode as a captured HIP graph")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): "
              "requests are independent, so the path shards by request with no per-step "
              "communication; run one process per GPU instead.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from trie_constrained_beam_amd import Beams, Trie, synth

    wl = synth.WORKLOADS[args.workload]
    if wl.slot_budget or wl.hidden:
        raise SystemExit(f"workload {wl.name} is a parity case, not a bench line")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    cat = wl.catalog()
    log(f"[bench] catalog {cat.shape} in {time.perf_counter() - t0:.1f}s")
    trie = Trie(cat, device=dev)
    widths = list(wl.widths)
    S, R, B = sum(widths), len(widths), max(widths)
    V, L = trie.V, trie.L
    beams = Beams(trie, S, R, B, device=dev)

    # ---------------------------------------------------------------- inputs in HBM
    ids, bases = beams.init(widths)
    host_steps = []
    for t in range(L):
        host = np.zeros((S, V), dtype=np.uint16 if wl.bf16 else np.float32)
        for i, (w, b) in enumerate(zip(widths, bases)):
            host[b:b + w] = synth.logits_rowkeyed(wl.seed, t, i, w, wl.sigma, bf16=wl.bf16)
        host_steps.append(host)

    def to_dev(h):
        if wl.bf16:
            return torch.from_numpy(h.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(h).to(dev)
    base_set = [to_dev(h) for h in host_steps]
    per_decode_bytes = sum(x.numel() * x.element_size() for x in base_set)
    n_copies = max(1, math.ceil(args.pool_gib * 2 ** 30 / per_decode_bytes))
    pool = [base_set] + [[x.clone() for x in base_set] for _ in range(n_copies - 1)]
    out = {"sids": torch.empty((R, B, L), dtype=torch.uint8, device=dev),
           "scores": torch.empty((R, B), dtype=torch.float32, device=dev),
           "items": torch.empty((R, B), dtype=torch.int64, device=dev),
           "counts": torch.empty(R, dtype=torch.int32, device=dev)}
    log(f"[bench] pool {n_copies} x {per_decode_bytes / 2**20:.1f} MiB of logits")

    # live rows per step (untimed decode, read back once)
    rows_per_step = []
    for t in range(L):
        ex = beams.export()
        rows_per_step.append(int(ex["rows"][torch.as_tensor(ids, device=dev).long()].sum().item()))
        beams.step(pool[0][t])
    beams.finalize_device(ids, out)
    torch.cuda.synchronize()
    rows_x_steps = sum(rows_per_step)
    log(f"[bench] live rows per step {rows_per_step} -> {rows_x_steps} rows x steps per decode")

    def decode(c):
        rid, _ = beams.init(widths)
        for t in range(L):
            beams.step(pool[c][t])
        beams.finalize_device(rid, out)

    graphs = None
    if args.graph:
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in range(n_copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    decode(c)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

    def run(d):
        if graphs is not None:
            graphs[d % n_copies].replay()
        else:
            decode(d % n_copies)

    for d in range(args.warmup):
        run(d)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed region
    if graphs is None:
        beams.enable_timing(args.steps * L)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for d in range(args.steps):
        run(d)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    if graphs is None:
        _, tile_ms, merge_ms, n_timed = beams.timing()
    else:
        # the same decodes again, eagerly, with per-kernel events (graph replays hide them)
        beams.enable_timing(args.steps * L)
        for d in range(args.steps):
            decode(d % n_copies)
        _, tile_ms, merge_ms, n_timed = beams.timing()
    beams.enable_timing(0)

    value = rows_x_steps * args.steps / elapsed
    dsize = 2 if wl.bf16 else 4
    expand_unit = V * dsize + EXPAND_STATE_BYTES + EXPAND_TRIE_BYTES
    expand_bytes_per_launch = rows_x_steps * expand_unit / L
    expand_avg_s = tile_ms / 1e3 / n_timed
    achieved = expand_bytes_per_launch / expand_avg_s / 1e9
    path_unit = expand_unit + MERGE_WRITE_BYTES
    wall_gbps = rows_x_steps * path_unit * args.steps / elapsed / 1e9
    log(f"[bench] {args.steps} decodes in {elapsed * 1e3:.1f} ms; tile kernel avg "
        f"{expand_avg_s * 1e6:.2f} us, merge kernel avg {merge_ms / n_timed * 1e3:.2f} us")

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        otrie = oracle.OracleTrie(cat)
        per_req = []
        for i, w in enumerate(widths):
            per_req.append([synth.logits_rowkeyed(wl.seed, t, i, w, wl.sigma, bf16=wl.bf16)
                            for t in range(L)])
        done_rows, n_req_done = 0, 0
        c0 = time.perf_counter()
        while time.perf_counter() - c0 < args.cpu_seconds and n_req_done < 10 * R:
            i = n_req_done % R
            xs = per_req[i]
            res = oracle.decode(otrie, widths[i],
                                lambda t, pref: oracle.widen_logits(xs[t][:len(pref)],
                                                                    "bf16" if wl.bf16 else "f32"))
            done_rows += sum(h["cand_parent"].max() + 1 for h in res["history"])
            n_req_done += 1
        cpu_s = time.perf_counter() - c0
        cpu = {"value": done_rows / cpu_s, "unit": "beam-rows x steps/s", "cores": 1, "kind": "oracle",
               "sample": f"{n_req_done} request decodes of this workload ({done_rows} beam-rows x steps, "
                         f"{cpu_s:.1f} s) on {platform.processor() or platform.machine()}, "
                         f"numpy float64, single thread"}
        log(f"[bench] oracle {cpu['value']:.0f} rows x steps/s over {cpu_s:.1f}s")

    line = {
        "metric": "constrained beam-rows x steps/sec (and achieved HBM GB/s) at B=512, 1 MI355X",
        "value": value,
        "unit": "beam-rows x steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "requests": R, "beam_width": B, "L": L, "catalog": int(cat.shape[0]),
                   "catalog_levels": "zipf(1.1)" if wl.level_dists[0] == "zipf" else "/".join(wl.level_dists),
                   "logits": ("bf16" if wl.bf16 else "f32") + f" N(0,{wl.sigma:g}^2)",
                   "rows_x_steps_per_decode": rows_x_steps, "rows_per_step": rows_per_step,
                   "graph": bool(args.graph), "logits_pool_copies": n_copies},
        "roofline": {"bound": "hbm", "kernel": "k_tile", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "bytes_per_row_step": expand_unit, "avg_launch_us": expand_avg_s * 1e6},
        "hbm_GBps_wall": wall_gbps,
        "merge_avg_us": merge_ms / n_timed * 1e3,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
