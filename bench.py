#!/usr/bin/env python3
"""Paged-KV split-KV decode attention benchmark on one MI355X.

One step = one full pkv_paged_decode call (the split kernel, which also
merges the splits for small grids, or the split kernel then the combine
kernel) over one batch of synthetic, seeded input that is already resident in
HBM.  The default workload is the largest single-GPU decode configuration of
the B = 8..256 range: B = 256 sequences of 4 query tokens (Hq = 64, Hkv = 8,
D = 128, page 32) over lognormal kv lengths (median 1024, clipped to [32,
8192]), causal at each sequence's end.  ``--workload`` selects another shape
for the headline; the same JSON line also carries, under ``configs``, the
timing and roofline of every other benchmark shape (the 12 head-dim / GQA
sweep variants, the long-context shape at automatic, 1 and 64 splits, the
1B-model decode shape, the mixed chunked-prefill + decode batch and the
prefill chunks), each measured in this run with the same protocol.

Protocol (after the AstrAI GEMV benchmark notes: warmup, then back-to-back
iterations, medians): W untimed warmup steps; then K timed eager steps back
to back on one stream, bracketed by two HIP events (median of --runs
repetitions), each step reading a different replica of the K/V pools (same
logical content, different addresses, replicas spanning >= 1 GiB so no step
finds its K/V in L2 or the 256 MB Infinity Cache).  A spin kernel queued
first keeps the host's launches ahead of the GPU, so the events measure GPU
time.  `value` is K/V bytes per call over that eager time per call.  The
dominant kernel's own average duration (for the roofline) comes from a
hipGraph of back-to-back launches of that kernel alone, replayed between two
events on the stream the graph runs on.  Prints one JSON line.
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
DEFAULT_WORKLOAD = "ragged"

# Shapes timed beside the headline (name, forced split count or 0).
SECONDARY = ([(f"sweep_d{d}_h{h}", 0) for d in (32, 64, 128, 256) for h in (8, 32, 64)] +
             [("long_ctx", 0), ("long_ctx", 1), ("long_ctx", 64), ("decode_1b", 0), ("mixed", 0),
              ("prefill", 0), ("ragged", 0)])


def config_key(workload: str, splits: int) -> str:
    """Name of a (workload, forced split count) entry: 'long_ctx:s64'."""
    return workload if splits <= 0 else f"{workload}:s{splits}"


def measured_traffic(key: str):
    """HBM bytes per call from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's reading), or
    None when there is none for this entry or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    e = data.get("workloads", {}).get(key)
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


def _head(w, n):
    """The workload restricted to its first n sequences (pools shared)."""
    return w.replace(B=n, q=w.q[:n], block_table=w.block_table[:n], kv_lens=w.kv_lens[:n],
                     causal_offsets=None if w.causal_offsets is None else w.causal_offsets[:n],
                     mask=None if w.mask is None else w.mask[:n],
                     q_lens=None if w.q_lens is None else w.q_lens[:n])


def _oracle_run(w):
    import oracle
    return oracle.decode_varlen if w.q_lens is not None or w.causal_offset < -1 else oracle.decode


def oracle_time(w, threads: int, budget_s: float, runs: int = 3):
    """Median wall time of the oracle on the first n sequences of w (all
    their rows), n the largest that keeps `runs` runs within budget_s;
    returns (seconds, n)."""
    run = _oracle_run(w)
    probe = _head(w, 1)
    t0 = time.perf_counter()
    run(probe, threads)
    sec_per_byte = max(time.perf_counter() - t0, 1e-5) / max(probe.kv_bytes(), 1)
    n = 1
    while n < w.B and _head(w, n + 1).kv_bytes() * sec_per_byte * runs <= budget_s:
        n += 1
    sub = _head(w, n)
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        run(sub, threads)
        times.append(time.perf_counter() - t0)
    return statistics.median(times), n


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle on the host cores, on a bounded sample of the workload
    (its first n sequences, all their rows, n chosen so three timed runs take
    about budget_s seconds), scaled to the full call by K/V bytes; plus the
    oracle on one thread on the tiny, 1B-model decode and long-context shapes
    (whole batch, or its first sequences within a small budget)."""
    import oracle
    threads = oracle.max_threads()      # all host cores (before any single-thread run)
    t, n = oracle_time(w, threads, budget_s)
    sub = _head(w, n)
    res = {"value": round(sub.kv_bytes() / t / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "us_per_call": round(t * 1e6 * w.kv_bytes() / max(sub.kv_bytes(), 1), 1),
           "sample": f"first {n} of {w.B} sequences of {w.name} (all their rows), fp64 OpenMP oracle on "
                     f"{threads} threads, median of 3 runs; us_per_call scaled to the full batch by K/V bytes",
           "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(), "omp_threads": threads}
    single = {}
    for name in ("tiny", "decode_1b", "long_ctx"):
        ws = make_workload(name)
        t1, n1 = oracle_time(ws, 1, 3.0)
        single[name] = {"us_per_call": round(t1 * 1e6 * ws.kv_bytes() / max(_head(ws, n1).kv_bytes(), 1), 1),
                        "sample": f"first {n1} of {ws.B} sequences, 1 thread, median of 3 runs"
                                  + ("" if n1 == ws.B else ", scaled to the full batch by K/V bytes")}
    res["single_thread"] = single
    oracle.decode(make_workload("tiny"), threads)   # the OpenMP thread count stays set: back to all cores
    return res


class Bench:
    """Device state and timing of one workload: inputs resident in HBM, the
    K/V pools replicated across >= replica_bytes, one call per step."""

    def __init__(self, name, args, splits=0, heads_per_block=0, kv_layout="paged"):
        import numpy as np
        import torch

        import paged_kv_split_amd as pkv

        self.args = args
        self.pkv = pkv
        self.torch = torch
        dev = torch.device("cuda:0")
        w = self.w = make_workload(name)
        self.key = config_key(name, splits) if kv_layout == "paged" else f"{config_key(name, splits)}:{kv_layout}"
        self.kv_layout = kv_layout

        def t(a, dtype):
            return torch.from_numpy(np.ascontiguousarray(a)).view(dtype).to(dev)

        self.varlen = varlen = w.q_lens is not None
        if varlen:
            qp, cu = w.packed_q()
            q = t(qp.view(np.int16), torch.bfloat16)
            self.cu_t = t(cu, torch.int32)
            if kv_layout != "paged":
                raise SystemExit("varlen batches are paged only")
        else:
            q = t(w.q.view(np.int16), torch.bfloat16)
        self.q = q
        self.bt = t(w.block_table, torch.int32)
        self.kl = t(w.kv_lens, torch.int32)
        self.co = None if w.causal_offsets is None else t(w.causal_offsets, torch.int32)
        self.mask = None if w.mask is None else t(w.mask, torch.float32)
        self.paged = paged = kv_layout == "paged"
        if paged:
            kc, vc = w.k_cache, w.v_cache
        else:
            import workloads
            kc, vc = workloads.to_contiguous(w, kv_layout)
        self.cap = w.max_kv_len
        pool_bytes = 2 * kc.nbytes
        self.n_rep = n_rep = max(2, math.ceil(args.replica_bytes / max(pool_bytes, 1)))
        k0 = torch.from_numpy(kc.view(np.int16)).view(torch.bfloat16).to(dev)
        v0 = torch.from_numpy(vc.view(np.int16)).view(torch.bfloat16).to(dev)
        self.ks = [k0] + [k0.clone() for _ in range(n_rep - 1)]
        self.vs = [v0] + [v0.clone() for _ in range(n_rep - 1)]
        del kc, vc

        msb, msq = w.mask_strides
        if paged:
            prob = pkv.make_problem(batch=w.B, q_len=w.q_len, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
                                    page_size=w.page_size, num_pages=w.num_pages,
                                    max_pages_per_seq=w.max_pages_per_seq, max_kv_len=w.max_kv_len,
                                    scale=w.scale, causal_offset=w.causal_offset, num_splits=splits,
                                    mask_stride_b=msb, mask_stride_q=msq, heads_per_block=heads_per_block)
        else:
            prob = pkv.contiguous_problem(batch=w.B, q_len=w.q_len, num_q_heads=w.Hq, num_kv_heads=w.Hkv,
                                          head_dim=w.D, kv_capacity=self.cap, max_kv_len=w.max_kv_len,
                                          scale=w.scale, causal_offset=w.causal_offset, num_splits=splits,
                                          mask_stride_b=msb, mask_stride_q=msq, heads_per_block=heads_per_block)
        self.plan = plan = pkv.plan_varlen(prob, w.total_tokens) if varlen else pkv.plan(prob)
        self.S = S = plan.splits
        if not plan.paired_heads:
            # lock the reported plan in (the contiguous layouts then run the paged plan's
            # splits and grouping)
            prob.num_splits = S
            prob.heads_per_block = plan.heads_per_block
        # a paired plan stays automatic (as given on the command line), so every call runs the
        # plan reported here: a forced grouping is never paired, and forcing the split count
        # alone may change the grouping the heuristic picks; the [B, Hkv, L, D] layout runs
        # the same split count unpaired
        self.prob = prob
        self.out = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=dev)
        self.o_part, self.ml_part = pkv.alloc_workspace(prob, S, dev)     # ml_part zeroed (counter head)
        self.ob = 0 if self.o_part is None else self.o_part.numel() * 4
        self.mb = 0 if self.ml_part is None else self.ml_part.numel() * 4
        self.sh = int(torch.cuda.current_stream().cuda_stream)
        P = pkv._ptr
        self.base = (P(q), P(self.bt), P(self.kl), P(self.co), P(self.mask))
        self.po, self.pm = P(self.o_part), P(self.ml_part)
        # the split step alone (partials entry point), for two-kernel calls
        self.n_kernels = plan.kernels if paged and not varlen else 1
        self.rows = w.total_tokens * w.Hq
        self.pob, self.pmb = pkv.partials_bytes(prob, S)
        self.po2 = torch.empty(max(self.pob // 4, 4), dtype=torch.float32, device=dev)
        self.pm2 = torch.empty(max(self.pmb // 4, 4), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    def step(self, r):
        pkv, P, w, b = self.pkv, self.pkv._ptr, self.w, self.base
        if self.varlen:
            st = pkv.paged_decode_varlen_raw(self.prob, P(self.cu_t), w.total_tokens, b[0], P(self.ks[r]),
                                             P(self.vs[r]), b[1], b[2], b[3], b[4], self.po, self.ob, self.pm,
                                             self.mb, P(self.out), 0, self.sh)
        elif self.paged:
            st = pkv.paged_decode_raw(self.prob, b[0], P(self.ks[r]), P(self.vs[r]), b[1], b[2], b[3], b[4],
                                      self.po, self.ob, self.pm, self.mb, P(self.out), 0, self.sh)
        else:
            st = pkv.contiguous_decode_raw(self.prob, pkv.KV_LAYOUTS[self.kv_layout], self.cap, b[0],
                                           P(self.ks[r]), P(self.vs[r]), b[2], b[3], b[4], self.po, self.ob,
                                           self.pm, self.mb, P(self.out), 0, self.sh)
        if st:
            raise pkv.PkvError(st, "pkv_paged_decode" if self.paged else "pkv_contiguous_decode")

    def split_only(self, r):
        pkv, P, b = self.pkv, self.pkv._ptr, self.base
        st = pkv.paged_decode_partials_raw(self.prob, b[0], P(self.ks[r]), P(self.vs[r]), b[1], b[2], b[3],
                                           b[4], P(self.po2), self.pob, P(self.pm2), self.pmb, self.sh)
        if st:
            raise pkv.PkvError(st, "pkv_paged_decode_partials")

    def combine_only(self, r):
        pkv, P = self.pkv, self.pkv._ptr
        st = pkv.combine_raw(self.rows, self.S, self.w.D, P(self.po2), P(self.pm2), P(self.out), 0, self.sh)
        if st:
            raise pkv.PkvError(st, "pkv_combine")

    def measure(self, steps, warmup, runs, graph=True):
        """Timing of this workload: eager µs per call (median of `runs`
        repetitions of `steps` calls), warm (no rotation) µs per call, and the
        dominant kernel's own duration from graph replay."""
        torch = self.torch
        n_rep = self.n_rep
        for i in range(warmup):
            self.step(i % n_rep)
        torch.cuda.synchronize()
        # spin length that covers the host's enqueue time of the timed loop
        t0 = time.perf_counter()
        for i in range(min(steps, 20)):
            self.step(i % n_rep)
        host_per_step = (time.perf_counter() - t0) / min(steps, 20)
        torch.cuda.synchronize()
        if not hasattr(torch.cuda, "_sleep"):
            raise SystemExit("torch.cuda._sleep is needed to keep the launch queue ahead of the GPU")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        sleep_ms_per_unit = e0.elapsed_time(e1) / 1_000_000
        spin = int(min(2.0 * host_per_step * steps * 1e3 / max(sleep_ms_per_unit, 1e-9), 2**31 - 1))

        def timed(fn, rotate=True):
            """ms per call of `steps` back-to-back eager calls, bracketed by two events."""
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            torch.cuda._sleep(spin)
            start.record()
            for i in range(steps):
                fn(i % n_rep if rotate else 0)
            end.record()
            torch.cuda.synchronize()
            return start.elapsed_time(end) / steps

        call_ms = statistics.median([timed(self.step) for _ in range(max(1, runs))])
        warm_ms = timed(self.step, rotate=False)

        def graph_ms(fn):
            """ms per launch when calls cycling over the replicas (one per
            replica, up to 64, and at least 16 so that a replay's own launch
            gap is spread over many calls) are captured into a hipGraph and the
            graph is replayed back to back, bracketed by two events on the
            stream the replays run on."""
            nrep_g = max(min(n_rep, 64), 16)
            gs = torch.cuda.Stream()
            gs.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            saved = self.sh
            try:
                with torch.cuda.stream(gs):
                    self.sh = int(gs.cuda_stream)     # the raw calls launch on the capture stream
                    with torch.cuda.graph(g, stream=gs):
                        for r in range(nrep_g):
                            fn(r % n_rep)
            finally:
                self.sh = saved
            torch.cuda.current_stream().wait_stream(gs)
            torch.cuda.synchronize()
            reps = max(1, steps // nrep_g)
            with torch.cuda.stream(gs):
                g.replay()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(gs)
                for _ in range(reps):
                    g.replay()
                b.record(gs)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / (reps * nrep_g)

        if self.n_kernels == 2:
            self.split_only(0)
            self.combine_only(0)
        timing = "graph"
        graph_call_ms = split_ms = None
        comb_ms = 0.0
        if graph:
            try:
                graph_call_ms = graph_ms(self.step)
                if self.n_kernels == 1:
                    split_ms = graph_call_ms
                else:
                    split_ms = graph_ms(self.split_only)
                    comb_ms = graph_ms(self.combine_only)
            except Exception as ex:  # report why, and fall back to eager timing
                print(f"bench: graph timing unavailable: {ex}", file=sys.stderr, flush=True)
                graph_call_ms = split_ms = None
        if split_ms is None:
            timing = "eager"
            split_ms = call_ms if self.n_kernels == 1 else timed(self.split_only)
            comb_ms = 0.0 if self.n_kernels == 1 else timed(self.combine_only)
        return dict(call_ms=call_ms, warm_ms=warm_ms, graph_call_ms=graph_call_ms, split_ms=split_ms,
                    comb_ms=comb_ms, timing=timing)

    def report(self, m):
        """Figures of one measurement: K/V GB/s of the call, algorithmic
        bytes and flops, and the dominant kernel's roofline."""
        import paged_kv_split_amd as pkv
        w = self.w
        kv_bytes = w.kv_bytes()
        us_call = m["call_ms"] * 1e3
        gbs = kv_bytes / (us_call * 1e-6) / 1e9
        algo = algorithmic_bytes(w)
        flops = algorithmic_flops(w)
        split_s = m["split_ms"] * 1e-3
        # the bound: matrix cores when the call's flops per byte exceed the
        # machine balance (dense bf16 peak / HBM peak), else HBM
        mfma_bound = flops / max(algo, 1) > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
        kernel = pkv.kernel_family(self.prob)
        traffic = measured_traffic(self.key)
        if mfma_bound:
            ach = flops / split_s / 1e12
            roof = {"bound": "mfma", "kernel": kernel, "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
        else:
            ach = algo / split_s / 1e9
            roof = {"bound": "hbm", "kernel": kernel, "achieved": round(ach, 2), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}
        return dict(us_per_call=round(us_call, 3), kv_gbs=round(gbs, 2), pct_of_peak=round(100 * gbs / PEAK_HBM_GBS, 2),
                    kernel_us={"split": round(m["split_ms"] * 1e3, 3), "combine": round(m["comb_ms"] * 1e3, 3),
                               "timing": m["timing"] if self.n_kernels == self.plan.kernels
                               else m["timing"] + ", split = whole call"},
                    kernels_per_call=self.plan.kernels, splits=self.S, heads_per_block=self.plan.heads_per_block,
                    algorithmic_bytes_per_call=algo, kv_bytes_per_call=kv_bytes,
                    algorithmic_flops_per_call=flops, warm_us_per_call=round(m["warm_ms"] * 1e3, 3),
                    graph_us_per_call=None if m["graph_call_ms"] is None else round(m["graph_call_ms"] * 1e3, 3),
                    roofline=roof)

    def release(self):
        for name in ("ks", "vs", "q", "bt", "kl", "co", "mask", "out", "o_part", "ml_part", "po2", "pm2"):
            setattr(self, name, None)
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--splits", type=int, default=0, help="0 = library heuristic")
    ap.add_argument("--heads-per-block", type=int, default=0, help="kv heads per workgroup; 0 = library heuristic")
    ap.add_argument("--kv-layout", default="paged", choices=["paged", "blhd", "bhld"],
                    help="K/V in pages (pkv_paged_decode) or contiguous per sequence (pkv_contiguous_decode)")
    ap.add_argument("--replica-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--runs", type=int, default=5, help="timed repetitions (median reported)")
    ap.add_argument("--no-configs", action="store_true", help="time the headline workload only")
    ap.add_argument("--config-steps", type=int, default=200, help="timed calls per run, other shapes")
    ap.add_argument("--config-warmup", type=int, default=20)
    ap.add_argument("--config-runs", type=int, default=3)
    ap.add_argument("--copy-calibration", type=float, default=0.0,
                    help="only run a plain device copy of this many bytes (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the paged decode kernel runs on one device's share "
              f"of the work (--gpus {args.gpus}, WORLD_SIZE {world} requested). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

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

    bench = Bench(args.workload, args, args.splits, args.heads_per_block, args.kv_layout)
    print(f"bench: workload {bench.w.name} on the device (S={bench.S}, replicas={bench.n_rep})",
          file=sys.stderr, flush=True)
    m = bench.measure(args.steps, args.warmup, args.runs, graph=not args.no_graph)
    rep = bench.report(m)
    print("bench: timed runs done", file=sys.stderr, flush=True)
    line = {
        "metric": METRIC,
        "value": rep["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["call_ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(describe(bench.w, bench.S, bench.n_rep, bench.plan.heads_per_block),
                       kv_layout=args.kv_layout),
    }
    line.update({k: v for k, v in rep.items() if k not in ("splits", "heads_per_block", "kv_gbs")})
    headline_key = bench.key
    bench.release()
    del bench

    if not args.no_configs:
        configs = {}
        for name, splits in SECONDARY:
            key = config_key(name, splits)
            if key == headline_key:
                continue
            b = Bench(name, args, splits)
            mm = b.measure(args.config_steps, args.config_warmup, args.config_runs, graph=not args.no_graph)
            r = b.report(mm)
            configs[key] = {"us_per_call": r["us_per_call"], "kv_gbs": r["kv_gbs"], "pct_of_peak": r["pct_of_peak"],
                            "kernel_us": r["kernel_us"]["split"], "splits": r["splits"],
                            "heads_per_block": r["heads_per_block"], "roofline": r["roofline"]}
            print(f"bench: {key} {r['us_per_call']} us/call, roofline frac {r['roofline']['frac']}",
                  file=sys.stderr, flush=True)
            b.release()
        line["configs"] = {"steps": args.config_steps, "warmup": args.config_warmup, "runs": args.config_runs,
                           "results": configs}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(make_workload(args.workload), args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
