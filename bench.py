#!/usr/bin/env python3
"""Paged-KV split-KV decode attention benchmark on one MI355X.

One step = one full pkv_paged_decode call (the split kernel, which also
merges the splits for small grids, or the split kernel then the combine
kernel) over one batch of synthetic, seeded input that is already resident in
HBM.  The default workload is the 1B-model decode shape (B=8, Hq=24, Hkv=4,
D=64, page 32, kv_lens uniform on [128, 2048]); ``--workload`` selects the
other decode shapes, and ``mixed`` a batch of chunked-prefill and decode
sequences with different query-token counts (pkv_paged_decode_varlen).

Protocol: W untimed warmup steps; then K timed eager steps back to back on
one stream, bracketed by two HIP events (median of --runs repetitions), each
step reading a different replica of the K/V pools (same logical content,
different addresses, replicas spanning >= 1 GiB so no step finds its K/V in
L2 or the 256 MB Infinity Cache).  A spin kernel queued first keeps the host's
launches ahead of the GPU, so the events measure GPU time.  `value` is K/V
bytes per call over that eager time per call.  The dominant kernel's own
average duration (for the roofline) comes from a hipGraph of back-to-back
launches of that kernel alone, replayed between two events on its stream.
Prints one JSON line.
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
PEAK_BF16_TFLOPS = 2500.0      # MI355X published dense bf16 matrix-core peak
METRIC = "paged-decode attention µs/call and achieved HBM GB/s (% of peak), B=8..256"


def kernel_name(w, S, prob) -> str:
    import paged_kv_split_amd as pkv
    return pkv.kernel_family(prob)


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
    from paged_kv_split_amd.profiling import source_digest
    if not e or data.get("source_digest") != source_digest():
        return None
    return e["hbm_bytes_per_call"]


def algorithmic_bytes(w) -> int:
    """Bytes the split kernel must move at minimum in one call: the K and V
    rows of every visible key, q, the bf16 output, the block-table entries of
    the pages in use and, when present, the mask entries of those keys."""
    import numpy as np
    L = w.kv_lens.astype(np.int64)
    n = w.q_lens.astype(np.int64) if w.q_lens is not None else np.full(w.B, w.q_len, dtype=np.int64)
    kv = int(L.sum()) * w.Hkv * w.D * 2 * 2
    qo = w.total_tokens * w.Hq * w.D * 2 * 2
    bt = int(((L + w.page_size - 1) // w.page_size).sum()) * 4
    mask = 0
    if w.mask is not None:
        mask = int((L * (n if w.mask.ndim == 3 else 1)).sum()) * 4
    return kv + qo + bt + mask


def algorithmic_flops(w) -> int:
    """Matrix flops one call must do at minimum: 4 * D per (query row, visible
    key) (q.k and p.v, a multiply and an add each), over every query head."""
    import numpy as np
    L = w.kv_lens.astype(np.int64)
    n = w.q_lens.astype(np.int64) if w.q_lens is not None else np.full(w.B, w.q_len, dtype=np.int64)
    pairs = 0
    for b in range(w.B):
        i = np.arange(int(n[b]), dtype=np.int64)
        if w.causal_offsets is not None:
            c = int(w.causal_offsets[b])
            vis = np.minimum(L[b], c + i + 1) if c >= 0 else np.full_like(i, L[b])
        elif w.causal_offset == -2:
            vis = np.minimum(L[b], L[b] - n[b] + i + 1)
        elif w.causal_offset >= 0:
            vis = np.minimum(L[b], w.causal_offset + i + 1)
        else:
            vis = np.full_like(i, L[b])
        pairs += int(np.maximum(vis, 0).sum())
    return pairs * w.Hq * w.D * 4


def make_workload(name: str):
    import workloads
    if name in workloads.CONFIGS:
        return workloads.CONFIGS[name]()
    if name.startswith("sweep_d"):
        d, h = name[len("sweep_d"):].split("_h")
        return workloads.sweep(int(d), int(h))
    raise SystemExit(f"unknown workload {name}")


def describe(w, splits, replicas, heads_per_block):
    L = w.kv_lens
    extra = {}
    if w.q_lens is not None:
        extra = {"q_tokens": w.total_tokens, "prefill_seqs": int((w.q_lens > 1).sum()),
                 "causal_last": w.causal_offset == -2}
    return {"workload": w.name, "B": w.B, "q_len": w.q_len, **extra, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
            "page_size": w.page_size, "kv_len_min": int(L.min()), "kv_len_max": int(L.max()),
            "kv_len_mean": round(float(L.mean()), 1), "mask": None if w.mask is None else list(w.mask.shape),
            "causal": w.causal_offsets is not None or w.causal_offset != -1, "splits": splits,
            "heads_per_block": heads_per_block,
            "replicas": replicas, "seed": w.seed}


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle on the host cores, on a bounded sample of the workload:
    the first n sequences (all their rows), n chosen so three timed runs take
    about budget_s seconds."""
    import oracle

    def head(n):
        return w.replace(B=n, q=w.q[:n], block_table=w.block_table[:n], kv_lens=w.kv_lens[:n],
                         causal_offsets=None if w.causal_offsets is None else w.causal_offsets[:n],
                         mask=None if w.mask is None else w.mask[:n],
                         q_lens=None if w.q_lens is None else w.q_lens[:n])

    run = oracle.decode_varlen if w.q_lens is not None or w.causal_offset < -1 else oracle.decode
    threads = oracle.max_threads()
    probe = head(1)
    t0 = time.perf_counter()
    run(probe)
    sec_per_byte = max(time.perf_counter() - t0, 1e-5) / max(probe.kv_bytes(), 1)
    n = 1
    while n < w.B and head(n + 1).kv_bytes() * sec_per_byte * 3 <= budget_s:
        n += 1
    sub = head(n)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        run(sub)
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
    ap.add_argument("--heads-per-block", type=int, default=0, help="kv heads per workgroup; 0 = library heuristic")
    ap.add_argument("--kv-layout", default="paged", choices=["paged", "blhd", "bhld"],
                    help="K/V in pages (pkv_paged_decode) or contiguous per sequence (pkv_contiguous_decode)")
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

    varlen = w.q_lens is not None
    if varlen:
        qp, cu = w.packed_q()
        q = t(qp.view(np.int16), torch.bfloat16)
        cu_t = t(cu, torch.int32)
        if args.kv_layout != "paged":
            raise SystemExit("varlen batches are paged only")
    else:
        q = t(w.q.view(np.int16), torch.bfloat16)
    bt = t(w.block_table, torch.int32)
    kl = t(w.kv_lens, torch.int32)
    co = None if w.causal_offsets is None else t(w.causal_offsets, torch.int32)
    mask = None if w.mask is None else t(w.mask, torch.float32)
    paged = args.kv_layout == "paged"
    if paged:
        kc, vc = w.k_cache, w.v_cache
    else:
        import workloads
        kc, vc = workloads.to_contiguous(w, args.kv_layout)
    cap = w.max_kv_len
    pool_bytes = 2 * kc.nbytes
    n_rep = max(2, math.ceil(args.replica_bytes / max(pool_bytes, 1)))
    kh = torch.from_numpy(kc.view(np.int16)).view(torch.bfloat16)
    vh = torch.from_numpy(vc.view(np.int16)).view(torch.bfloat16)
    ks = [kh.to(dev) for _ in range(n_rep)]
    vs = [vh.to(dev) for _ in range(n_rep)]
    del kh, vh, kc, vc

    msb, msq = w.mask_strides
    if paged:
        prob = pkv.make_problem(batch=w.B, q_len=w.q_len, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
                                page_size=w.page_size, num_pages=w.num_pages,
                                max_pages_per_seq=w.max_pages_per_seq, max_kv_len=w.max_kv_len,
                                scale=w.scale, causal_offset=w.causal_offset, num_splits=args.splits,
                                mask_stride_b=msb, mask_stride_q=msq, heads_per_block=args.heads_per_block)
    else:
        prob = pkv.contiguous_problem(batch=w.B, q_len=w.q_len, num_q_heads=w.Hq, num_kv_heads=w.Hkv,
                                      head_dim=w.D, kv_capacity=cap, max_kv_len=w.max_kv_len, scale=w.scale,
                                      causal_offset=w.causal_offset, num_splits=args.splits,
                                      mask_stride_b=msb, mask_stride_q=msq,
                                      heads_per_block=args.heads_per_block)
    plan = pkv.plan_varlen(prob, w.total_tokens) if varlen else pkv.plan(prob)
    S = plan.splits
    prob.num_splits = S
    prob.heads_per_block = plan.heads_per_block
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
        if varlen:
            st = pkv.paged_decode_varlen_raw(prob, P(cu_t), w.total_tokens, base[0], P(ks[r]), P(vs[r]), base[1],
                                             base[2], base[3], base[4], po, ob, pm, mb, P(out), 0, sh)
        elif paged:
            st = pkv.paged_decode_raw(prob, base[0], P(ks[r]), P(vs[r]), base[1], base[2], base[3], base[4],
                                      po, ob, pm, mb, P(out), 0, sh)
        else:
            st = pkv.contiguous_decode_raw(prob, pkv.KV_LAYOUTS[args.kv_layout], cap, base[0], P(ks[r]), P(vs[r]),
                                           base[2], base[3], base[4], po, ob, pm, mb, P(out), 0, sh)
        if st:
            raise pkv.PkvError(st, "pkv_paged_decode" if paged else "pkv_contiguous_decode")

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

    def timed(fn, rotate=True):
        """ms per call of `steps` back-to-back eager calls, bracketed by two events."""
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(spin)
        start.record()
        for i in range(args.steps):
            fn(i % n_rep if rotate else 0)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    runs = [timed(step) for _ in range(max(1, args.runs))]
    call_ms = statistics.median(runs)
    warm_ms = timed(step, rotate=False)
    print("bench: timed runs done", file=sys.stderr, flush=True)

    def graph_ms(fn):
        """ms per launch when one call per replica (up to 64) is captured into
        a hipGraph and the graph is replayed back to back, bracketed by two
        events on the stream the kernels run on: the launches' own average
        duration, without the host's per-launch gaps."""
        nonlocal sh
        nrep_g = min(n_rep, 64)
        cur = torch.cuda.current_stream()
        gs = torch.cuda.Stream()
        gs.wait_stream(cur)
        g = torch.cuda.CUDAGraph()
        saved = sh
        try:
            with torch.cuda.stream(gs):
                sh = int(gs.cuda_stream)        # the raw calls launch on the capture stream
                with torch.cuda.graph(g, stream=gs):
                    for r in range(nrep_g):
                        fn(r)
        finally:
            sh = saved
        cur.wait_stream(gs)
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
        return a.elapsed_time(b) / (reps * nrep_g)

    # The dominant kernel's own average duration: the whole call when it is
    # one kernel; otherwise the split kernel alone (the same kernel, run
    # through pkv_paged_decode_partials), and the combine kernel alone.
    # Contiguous K/V and varlen batches have no partials entry point: a
    # two-kernel call is timed whole there.
    n_kernels = plan.kernels if paged and not varlen else 1
    rows = w.total_tokens * w.Hq
    pob, pmb = pkv.partials_bytes(prob, S)
    po2 = torch.empty(max(pob // 4, 4), dtype=torch.float32, device=dev)
    pm2 = torch.empty(max(pmb // 4, 4), dtype=torch.float32, device=dev)

    def split_only(r):
        st = pkv.paged_decode_partials_raw(prob, base[0], P(ks[r]), P(vs[r]), base[1], base[2], base[3],
                                           base[4], P(po2), pob, P(pm2), pmb, sh)
        if st:
            raise pkv.PkvError(st, "pkv_paged_decode_partials")

    def combine_only(r):
        st = pkv.combine_raw(rows, S, w.D, P(po2), P(pm2), P(out), 0, sh)
        if st:
            raise pkv.PkvError(st, "pkv_combine")

    if n_kernels == 2:
        split_only(0)
        combine_only(0)
    timing = "graph"
    graph_call_ms = split_ms = None
    comb_ms = 0.0
    if not args.no_graph:
        try:
            graph_call_ms = graph_ms(step)
            if n_kernels == 1:
                split_ms = graph_call_ms
            else:
                split_ms = graph_ms(split_only)
                comb_ms = graph_ms(combine_only)
        except Exception as ex:  # report why, and fall back to eager timing
            print(f"bench: graph timing unavailable: {ex}", file=sys.stderr, flush=True)
            graph_call_ms = split_ms = None
    if split_ms is None:
        timing = "eager"
        split_ms = call_ms if n_kernels == 1 else timed(split_only)
        comb_ms = 0.0 if n_kernels == 1 else timed(combine_only)

    kv_bytes = w.kv_bytes()
    us_call = call_ms * 1e3
    gbs = kv_bytes / (us_call * 1e-6) / 1e9
    algo = algorithmic_bytes(w)
    kern_gbs = algo / (split_ms * 1e-3) / 1e9
    flops = algorithmic_flops(w)
    # the bound: matrix cores when the call's flops per byte exceed the
    # machine balance (dense bf16 peak / HBM peak), else HBM
    mfma_bound = flops / max(algo, 1) > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(call_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(describe(w, S, n_rep, plan.heads_per_block), kv_layout=args.kv_layout),
        "us_per_call": round(us_call, 3),
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "kernels_per_call": plan.kernels,
        "kernel_us": {"split": round(split_ms * 1e3, 3), "combine": round(comb_ms * 1e3, 3),
                      "timing": timing if n_kernels == plan.kernels else timing + ", split = whole call"},
        "algorithmic_bytes_per_call": algo,
        "warm_us_per_call": round(warm_ms * 1e3, 3),
        "graph_us_per_call": None if graph_call_ms is None else round(graph_call_ms * 1e3, 3),
        "kv_bytes_per_call": kv_bytes,
        "algorithmic_flops_per_call": flops,
        "roofline": ({"bound": "mfma", "kernel": kernel_name(w, S, prob),
                      "achieved": round(flops / (split_ms * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                      "unit": "TFLOP/s", "frac": round(flops / (split_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "traffic": measured_traffic(w.name if paged else f"{w.name}:{args.kv_layout}")}
                     if mfma_bound else
                     {"bound": "hbm", "kernel": kernel_name(w, S, prob), "achieved": round(kern_gbs, 2),
                      "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(kern_gbs / PEAK_HBM_GBS, 4),
                      "traffic": measured_traffic(w.name if paged else f"{w.name}:{args.kv_layout}")}),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
