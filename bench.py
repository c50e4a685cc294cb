#!/usr/bin/env python3
"""Paged-KV split-KV decode attention benchmark on one MI355X.

One step = one full decode call (split kernel, plus the combine kernel when
more than one split is used) over one batch of synthetic, seeded input that
is already resident in HBM.  The default workload is the 1B-model decode shape
(B=8, Hq=24, Hkv=4, D=64, page 32, kv_lens uniform on [128, 2048]);
``--workload`` selects the other decode shapes.

Protocol: W untimed warmup steps; then K timed steps back to back on one
stream, each reading a different replica of the K/V pools (same logical
content, different addresses, replicas spanning >= 1 GiB so no step finds its
K/V in L2 or the 256 MB Infinity Cache).  A spin kernel queued first keeps the
host's launches ahead of the GPU, so the HIP events measure GPU time.  Events
between the kernels give each kernel's own average duration (on the stream
the kernels run on).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X published HBM3E peak
METRIC = "paged-decode attention µs/call and achieved HBM GB/s (% of peak), B=8..256"


def kernel_name(w, S, prob) -> str:
    import paged_kv_split_amd as pkv
    return pkv.kernel_family(prob)


def source_digest() -> str:
    """Digest of the kernel sources; counter figures taken on other sources
    are stale."""
    import hashlib
    csrc = os.path.join(ROOT, "paged_kv_split_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per call from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's reading), or
    None when there is none for this workload or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    e = data.get("workloads", {}).get(workload)
    if not e or data.get("source_digest") != source_digest():
        return None
    return e["hbm_bytes_per_call"]


def make_workload(name: str):
    import workloads
    if name in workloads.CONFIGS:
        return workloads.CONFIGS[name]()
    if name.startswith("sweep_d"):
        d, h = name[len("sweep_d"):].split("_h")
        return workloads.sweep(int(d), int(h))
    raise SystemExit(f"unknown workload {name}")


def describe(w, splits, replicas):
    L = w.kv_lens
    return {"workload": w.name, "B": w.B, "q_len": w.q_len, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
            "page_size": w.page_size, "kv_len_min": int(L.min()), "kv_len_max": int(L.max()),
            "kv_len_mean": round(float(L.mean()), 1), "mask": None if w.mask is None else list(w.mask.shape),
            "causal": w.causal_offsets is not None or w.causal_offset >= 0, "splits": splits,
            "replicas": replicas, "seed": w.seed}


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle on the host cores, on a bounded sample of the workload:
    the first n sequences (all their rows), n chosen so three timed runs take
    about budget_s seconds."""
    import oracle

    def head(n):
        return w.replace(B=n, q=w.q[:n], block_table=w.block_table[:n], kv_lens=w.kv_lens[:n],
                         causal_offsets=None if w.causal_offsets is None else w.causal_offsets[:n],
                         mask=None if w.mask is None else w.mask[:n])

    threads = oracle.max_threads()
    probe = head(1)
    t0 = time.perf_counter()
    oracle.decode(probe)
    sec_per_byte = max(time.perf_counter() - t0, 1e-5) / max(probe.kv_bytes(), 1)
    n = 1
    while n < w.B and head(n + 1).kv_bytes() * sec_per_byte * 3 <= budget_s:
        n += 1
    sub = head(n)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.decode(sub)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": round(sub.kv_bytes() / t / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "us_per_call": round(t * 1e6 * w.kv_bytes() / max(sub.kv_bytes(), 1), 1),
            "sample": f"first {n} of {w.B} sequences of {w.name} (all their rows), fp64 OpenMP oracle, "
                      f"median of 3 runs; us_per_call scaled to the full batch by K/V bytes"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_1b")
    ap.add_argument("--splits", type=int, default=0, help="0 = library heuristic")
    ap.add_argument("--replica-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--runs", type=int, default=5, help="timed repetitions (median reported)")
    ap.add_argument("--copy-calibration", type=float, default=0.0,
                    help="only run a plain device copy of this many bytes (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the paged decode kernel runs on one device's share "
              f"of the work (--gpus {args.gpus}, WORLD_SIZE {world} requested). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_split_amd as pkv

    torch.cuda.init()
    dev = torch.device("cuda:0")
    if args.copy_calibration > 0:
        n = int(args.copy_calibration) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "copies": 3}), flush=True)
        return
    w = make_workload(args.workload)
    print(f"bench: workload {w.name} built on host", file=sys.stderr, flush=True)

    def t(a, dtype):
        return torch.from_numpy(np.ascontiguousarray(a)).view(dtype).to(dev)

    q = t(w.q.view(np.int16), torch.bfloat16)
    bt = t(w.block_table, torch.int32)
    kl = t(w.kv_lens, torch.int32)
    co = None if w.causal_offsets is None else t(w.causal_offsets, torch.int32)
    mask = None if w.mask is None else t(w.mask, torch.float32)
    pool_bytes = 2 * w.k_cache.nbytes
    n_rep = max(2, math.ceil(args.replica_bytes / max(pool_bytes, 1)))
    kh = torch.from_numpy(w.k_cache.view(np.int16)).view(torch.bfloat16)
    vh = torch.from_numpy(w.v_cache.view(np.int16)).view(torch.bfloat16)
    ks = [kh.to(dev) for _ in range(n_rep)]
    vs = [vh.to(dev) for _ in range(n_rep)]
    del kh, vh

    msb, msq = w.mask_strides
    prob = pkv.make_problem(batch=w.B, q_len=w.q_len, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
                            page_size=w.page_size, num_pages=w.num_pages,
                            max_pages_per_seq=w.max_pages_per_seq, max_kv_len=w.max_kv_len,
                            scale=w.scale, causal_offset=w.causal_offset, num_splits=args.splits,
                            mask_stride_b=msb, mask_stride_q=msq)
    S = pkv.num_splits_for(prob)
    prob.num_splits = S
    out = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=dev)
    o_part, ml_part = pkv.alloc_workspace(prob, S, dev)      # ml_part zeroed (counter head)
    ob = 0 if o_part is None else o_part.numel() * 4
    mb = 0 if ml_part is None else ml_part.numel() * 4
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)

    P = pkv._ptr
    base = (P(q), P(bt), P(kl), P(co), P(mask))
    po, pm = P(o_part), P(ml_part)

    def step(r):
        st = pkv.paged_decode_raw(prob, base[0], P(ks[r]), P(vs[r]), base[1], base[2], base[3], base[4],
                                  po, ob, pm, mb, P(out), 0, sh)
        if st:
            raise pkv.PkvError(st, "pkv_paged_decode")

    # warmup
    for i in range(args.warmup):
        step(i % n_rep)
    torch.cuda.synchronize()
    print(f"bench: warmup done (S={S}, replicas={n_rep})", file=sys.stderr, flush=True)

    # spin length that covers the host's enqueue time of the timed loop
    t0 = time.perf_counter()
    for i in range(min(args.steps, 20)):
        step(i % n_rep)
    host_per_step = (time.perf_counter() - t0) / min(args.steps, 20)
    torch.cuda.synchronize()
    if not hasattr(torch.cuda, "_sleep"):
        raise SystemExit("torch.cuda._sleep is needed to keep the launch queue ahead of the GPU")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(1_000_000)
    e1.record()
    torch.cuda.synchronize()
    sleep_ms_per_unit = e0.elapsed_time(e1) / 1_000_000
    spin = int(min(2.0 * host_per_step * args.steps * 1e3 / max(sleep_ms_per_unit, 1e-9), 2**31 - 1))

    def timed(rotate=True):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(spin)
        start.record()
        for i in range(args.steps):
            r = i % n_rep if rotate else 0
            ev[i][0].record()
            step(r)
            ev[i][1].record()
        end.record()
        torch.cuda.synchronize()
        total = start.elapsed_time(end)
        call_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
        return total, call_ms

    runs = [timed(True) for _ in range(max(1, args.runs))]
    total_ms = statistics.median(r[0] for r in runs)
    call_ms = statistics.median(r[1] for r in runs)
    warm = timed(False)
    print("bench: timed runs done", file=sys.stderr, flush=True)

    graph_us = None
    if not args.no_graph:
        try:
            nrep_g = min(n_rep, 64)
            gs = torch.cuda.Stream()
            gs.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            sh_saved = sh
            with torch.cuda.stream(gs):
                sh = int(gs.cuda_stream)        # step() launches on the capture stream
                with torch.cuda.graph(g, stream=gs):
                    for r in range(nrep_g):
                        step(r)
            sh = sh_saved
            torch.cuda.current_stream().wait_stream(gs)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, args.steps // nrep_g)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            graph_us = a.elapsed_time(b) * 1e3 / (reps * nrep_g)
        except Exception as ex:  # graph timing is a side figure; report why it is missing
            print(f"bench: graph replay skipped: {ex}", file=sys.stderr, flush=True)

    kv_bytes = w.kv_bytes()
    us_call = total_ms * 1e3 / args.steps
    gbs = kv_bytes / (us_call * 1e-6) / 1e9
    kern_gbs = kv_bytes / (call_ms * 1e-3) / 1e9
    n_kernels = 1 if (S == 1 or pkv.merges_in_kernel(prob, S)) else 2
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": describe(w, S, n_rep),
        "us_per_call": round(us_call, 3),
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "kernels_per_call": n_kernels,
        "call_us_events": round(call_ms * 1e3, 3),
        "warm_us_per_call": round(warm[0] * 1e3 / args.steps, 3),
        "graph_us_per_call": None if graph_us is None else round(graph_us, 3),
        "kv_bytes_per_call": kv_bytes,
        "roofline": {"bound": "hbm", "kernel": kernel_name(w, S, prob), "achieved": round(kern_gbs, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(kern_gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(w.name)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
