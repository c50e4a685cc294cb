"""Turn the output of collect.sh into short text summaries.

usage: python3 -m paged_kv_split_amd.profiling.summarize OUTDIR PROFILES_DIR WORKLOAD...

For each workload it writes PROFILES_DIR/<kernel>_<workload>.md: the
rocprofv3 per-kernel statistics of the library's kernels, the bench line's
own HIP-event timing of the same kernel (the two must agree), and the HBM
bytes per launch from the FETCH_SIZE and WRITE_SIZE counters, each scaled by
what the counter reads for a plain 1 GiB device copy, and (when collected)
the matrix-core busy fraction, bf16 MFMA throughput and LDS bank conflicts.  It also records those
bytes in PROFILES_DIR/traffic.json, keyed by the kernel-source digest, for
bench.py's roofline.traffic field.
"""
import csv
import glob
import json
import os
import sys

from . import source_digest

COPY_BYTES = 1 << 30
SIMDS = 256 * 4   # MI355X: 256 CUs x 4 SIMDs
XCDS = 8
OURS = ("split_decode", "split_prefill", "combine_kernel")


def _csv(pattern):
    files = sorted(glob.glob(pattern))
    if not files:
        raise SystemExit(f"missing {pattern}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _short(name: str) -> str:
    """'void pkv::(anonymous namespace)::split_decode_valu<128, 1, ...>(pkv::DecodeArgs)'
    -> 'split_decode_valu<128, 1, ...>'"""
    for tag in OURS:
        i = name.find(tag)
        if i >= 0:
            rest = name[i:]
            j = rest.find(">(")
            return rest[:j + 1] if j >= 0 else rest.split("(")[0]
    return name.split("(")[0]


def _family(name: str) -> str:
    return _short(name).split("<")[0]


def counter_per_dispatch(rows, counter):
    """{kernel name: mean counter value (KiB) per dispatch} for our kernels."""
    acc = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def calibration(out):
    fetch = _csv(f"{out}/copy_fetch/*counter_collection.csv")
    write = _csv(f"{out}/copy_write/*counter_collection.csv")
    f = counter_per_dispatch(fetch, "FETCH_SIZE")
    w = counter_per_dispatch(write, "WRITE_SIZE")
    copy_f = max(f.values())          # the copy is the only kernel that reads 1 GiB
    copy_names = [k for k in w if "copy" in k.lower()]
    copy_w = sum(w[k] for k in copy_names) / len(copy_names) if copy_names else max(w.values())
    return {"copy_bytes": COPY_BYTES, "fetch_kib": copy_f, "write_kib": copy_w,
            "fetch_scale": COPY_BYTES / (copy_f * 1024), "write_scale": COPY_BYTES / (copy_w * 1024)}


def summarize(out, profiles, key, cal, command):
    """Summary of one workload key (NAME or NAME:sN, a forced split count;
    its collected files are tagged NAME_sN)."""
    wl = key.replace(":", "_")
    stats = _csv(f"{out}/{wl}_trace/*kernel_stats.csv")
    ours = [r for r in stats if any(t in r["Name"] for t in OURS)]
    with open(f"{out}/{wl}_trace.out") as fh:
        bench = json.loads([ln for ln in fh.read().splitlines() if ln.startswith("{")][-1])
    fetch = counter_per_dispatch(_csv(f"{out}/{wl}_fetch/*counter_collection.csv"), "FETCH_SIZE")
    write = counter_per_dispatch(_csv(f"{out}/{wl}_write/*counter_collection.csv"), "WRITE_SIZE")
    split = max((r for r in ours if "split_" in r["Name"]), key=lambda r: float(r["TotalDurationNs"]))
    fam = _family(split["Name"])
    algo = bench["algorithmic_bytes_per_call"]
    ev_us = bench["kernel_us"]["split"]
    prof_us = float(split["AverageNs"]) / 1e3

    lines = [f"# {fam} — workload {wl}", "",
             "Command (run from the repository root on one MI355X):", "",
             f"    {command}", "",
             f"Kernel sources digest: `{source_digest()}`", "",
             "Workload: `" + json.dumps(bench["config"]) + "`", "",
             "## rocprofv3 --kernel-trace --stats (library kernels)", "",
             "| kernel | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
    for r in ours:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "## The same kernel timed by bench.py with HIP events", "",
              f"- split kernel: {ev_us:.2f} µs ({bench['kernel_us']['timing']} timing; rocprofv3 average "
              f"{prof_us:.2f} µs, ratio {ev_us / prof_us:.3f})",
              f"- whole call: {bench['us_per_call']:.2f} µs/call, {bench['value']:.1f} GB/s of K/V "
              f"({bench['kernels_per_call']} kernel(s) per call)",
              f"- algorithmic bytes per call: {algo:,}; algorithmic matrix flops per call: "
              f"{bench.get('algorithmic_flops_per_call', 0):,}",
              f"- roofline ({bench['roofline']['bound']} bound): achieved {bench['roofline']['achieved']:.1f} "
              f"{bench['roofline']['unit']} = {100 * bench['roofline']['frac']:.1f}% of "
              f"{bench['roofline']['peak']:.0f} {bench['roofline']['unit']}", "",
              "## HBM bytes per launch (FETCH_SIZE, WRITE_SIZE)", "",
              f"Calibration on a 1 GiB device copy: FETCH_SIZE reads {cal['fetch_kib']:.0f} KiB "
              f"(scale {cal['fetch_scale']:.4f}), WRITE_SIZE reads {cal['write_kib']:.0f} KiB "
              f"(scale {cal['write_scale']:.4f}).", "",
              "| kernel | FETCH KiB | WRITE KiB | HBM read bytes | HBM write bytes |", "|---|---|---|---|---|"]
    per_kernel = {}
    for name in sorted(set(fetch) | set(write)):
        if not any(t in name for t in OURS):
            continue
        fb = fetch.get(name, 0.0) * 1024 * cal["fetch_scale"]
        wb = write.get(name, 0.0) * 1024 * cal["write_scale"]
        per_kernel[_short(name)] = (fb, wb)
        lines.append(f"| `{_short(name)}` | {fetch.get(name, 0.0):.0f} | {write.get(name, 0.0):.0f} | "
                     f"{fb:,.0f} | {wb:,.0f} |")
    fb, wb = per_kernel[_short(split["Name"])]
    lines += ["", f"Split kernel: {fb + wb:,.0f} HBM bytes per launch = {(fb + wb) / algo:.3f} x the "
              f"algorithmic bytes.", ""]
    sq = None
    sq_files = glob.glob(f"{out}/{wl}_sq/*counter_collection.csv")
    if sq_files:
        rows = _csv(f"{out}/{wl}_sq/*counter_collection.csv")
        c = {n: counter_per_dispatch(rows, n) for n in
             ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_LDS_BANK_CONFLICT",
              "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE", "MfmaUtil")}
        name = next((k for k in c["GRBM_GUI_ACTIVE"] if _short(k) == _short(split["Name"])), None)
        if name is not None:
            busy = c["SQ_VALU_MFMA_BUSY_CYCLES"].get(name, 0.0)
            gui = c["GRBM_GUI_ACTIVE"][name]
            mops = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"].get(name, 0.0)
            conf = c["SQ_LDS_BANK_CONFLICT"].get(name, 0.0)
            lds = c["SQ_LDS_IDX_ACTIVE"].get(name, 0.0)
            # the per-dispatch GRBM_GUI_ACTIVE record is the sum over the XCDs' GRBM
            # instances; busy cycles are summed over all SIMDs
            util = 100.0 * busy / (gui / XCDS * SIMDS) if gui > 0 else 0.0
            derived = c["MfmaUtil"].get(name)
            tflops = mops * 512 / (prof_us * 1e-6) / 1e12
            sq = {"mfma_busy_pct": round(util, 2), "mfma_util_derived_pct": derived, "mfma_bf16_tflops": round(tflops, 2),
                  "lds_bank_conflict_pct": round(100.0 * conf / lds, 2) if lds > 0 else 0.0}
            lines += ["## Matrix cores and LDS (SQ counters, per launch of the split kernel)", "",
                      f"- MFMA busy: {util:.2f}% of SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES / "
                      f"(GRBM_GUI_ACTIVE / {XCDS} XCDs x {SIMDS} SIMDs))"
                      + (f"; rocprofv3's derived MfmaUtil: {derived:.2f}%" if derived is not None else ""),
                      f"- bf16 MFMA work: {mops * 512:,.0f} flop per launch = {tflops:.2f} TFLOP/s over the "
                      f"rocprofv3 average duration (dense bf16 peak 2500 TFLOP/s)",
                      f"- LDS bank conflicts: {conf:,.0f} cycles over {lds:,.0f} LDS-active cycles "
                      f"({sq['lds_bank_conflict_pct']:.2f}%)", ""]
    if glob.glob(f"{out}/{wl}_issue/*counter_collection.csv"):
        rows = _csv(f"{out}/{wl}_issue/*counter_collection.csv")
        names = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VALU_TRANS_F32", "SQ_ACTIVE_INST_VALU",
                 "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_WAVES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")
        c = {n: counter_per_dispatch(rows, n) for n in names}
        name = next((k for k in c["GRBM_GUI_ACTIVE"] if _short(k) == _short(split["Name"])), None)
        waves = c["SQ_WAVES"].get(name, 0.0) if name is not None else 0.0
        if waves > 0:
            g = {n: c[n].get(name, 0.0) for n in names}
            simd_cycles = g["GRBM_GUI_ACTIVE"] / XCDS * SIMDS
            lines += ["## Instruction issue (SQ counters, per launch of the split kernel)", "",
                      f"- per wave: {g['SQ_INSTS_VALU'] / waves:,.0f} VALU instructions (MFMAs included), "
                      f"{g['SQ_INSTS_MFMA'] / waves:,.0f} MFMAs, {g['SQ_INSTS_VALU_TRANS_F32'] / waves:,.0f} "
                      f"fp32 transcendentals, {g['SQ_INSTS_LDS'] / waves:,.0f} LDS instructions "
                      f"({waves:,.0f} waves)",
                      f"- VALU and matrix cores issuing together: "
                      f"{100.0 * g['SQ_VALU_MFMA_COEXEC_CYCLES'] / simd_cycles:.1f}% of SIMD cycles "
                      f"(SQ_VALU_MFMA_COEXEC_CYCLES / (GRBM_GUI_ACTIVE / {XCDS} XCDs x {SIMDS} SIMDs))",
                      f"- VALU instructions executing: {100.0 * g['SQ_ACTIVE_INST_VALU'] / g['SQ_WAVE_CYCLES']:.1f}% "
                      f"of wave cycles (SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES)", ""]
    path = os.path.join(profiles, f"{fam}_{wl}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    rec = {"kernel": _short(split["Name"]), "hbm_bytes_per_call": round(fb + wb),
           "fetch_bytes": round(fb), "write_bytes": round(wb), "algorithmic_bytes": algo,
           "rocprof_avg_us": round(prof_us, 3), "event_avg_us": ev_us}
    if sq:
        rec.update(sq)
    return rec


def main():
    out, profiles, wls = sys.argv[1], sys.argv[2], sys.argv[3:]
    os.makedirs(profiles, exist_ok=True)
    cal = calibration(out)
    command = f"bash paged_kv_split_amd/profiling/collect.sh {out} " + " ".join(wls)
    tpath = os.path.join(profiles, "traffic.json")
    data = {}
    if os.path.exists(tpath):
        with open(tpath) as fh:
            data = json.load(fh)
    if data.get("source_digest") != source_digest():
        data = {"source_digest": source_digest(), "workloads": {}}
    data["calibration"] = cal
    data["command"] = (command + f"; python3 -m paged_kv_split_amd.profiling.summarize {out} {profiles} "
                       + " ".join(wls))
    for wl in wls:
        data["workloads"][wl] = summarize(out, profiles, wl, cal, data["command"])
        print(wl, data["workloads"][wl])
    with open(tpath, "w") as fh:
        json.dump(data, fh, indent=1)


if __name__ == "__main__":
    main()
