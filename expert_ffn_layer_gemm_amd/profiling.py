"""Summaries of rocprofv3 output for the profiles/ folder (host-side tool).

    python -m expert_ffn_layer_gemm_amd.profiling trace  STATS_CSV OUT_TXT --cmd "..."
    python -m expert_ffn_layer_gemm_amd.profiling traffic --workload W --bench-kernel NAME \
        --rocprof-kernel SUBSTR --fetch CSV --write CSV --fetch-copy CSV --write-copy CSV \
        --copy-bytes N --cmd-fetch "..." --cmd-write "..." --cmd-copy "..."
    python -m expert_ffn_layer_gemm_amd.profiling busy --workload W --bench-kernel NAME \
        --rocprof-kernel SUBSTR --counters CSV --trace CSV --mfma-flop F --peak-tflops P --cmd "..."
    python -m expert_ffn_layer_gemm_amd.profiling stalls --workload W --bench-kernel NAME \
        --rocprof-kernel SUBSTR --counters CSV --cmd "..."

`trace` keeps the rows of this library's kernels from a --kernel-trace --stats
summary.  `traffic` turns two --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
dispatch) into HBM bytes per launch of one kernel, each counter scaled by what
it reads for a plain device copy of known size, and writes
profiles/traffic_<workload>.json (read by bench.py, tagged with the kernel
source hash so stale numbers are ignored) plus a text summary.  `busy` turns
one --kernel-trace --pmc run (GRBM_GUI_ACTIVE, SQ_BUSY_CYCLES,
SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA) into the kernel's clock (GPU-active
cycles per XCD over its duration), the fraction of SIMD cycles the matrix
cores were busy, and the MFMA rate its instruction count implies.  `stalls`
turns one --pmc run of wave-state counters (SQ_WAVE_CYCLES, SQ_WAIT_ANY,
SQ_WAIT_INST_ANY, SQ_WAIT_INST_LDS, SQ_ACTIVE_INST_ANY, SQ_ACTIVE_INST_VALU,
SQ_ACTIVE_INST_LDS, SQ_LDS_BANK_CONFLICT) into fractions of the kernel's wave
cycles.
"""
import argparse
import collections
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT_DIR = os.path.join(ROOT, "profiles")          # where the summaries are written


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def trace_summary(stats_csv: str, out_txt: str, cmd: str) -> None:
    rows = _rows(stats_csv)
    lines = [f"# rocprofv3 kernel trace summary", f"# command: {cmd}",
             "# kernel | calls | average us | min us | max us | share of GPU time %"]
    for r in rows:
        name = r["Name"]
        if "moe::" not in name:
            continue
        lines.append(f"{name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")


def _per_kernel_kib(path):
    agg = collections.defaultdict(list)
    for r in _rows(path):
        agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return agg


def _pick(agg, substr):
    hits = [k for k in agg if substr in k]
    if len(hits) != 1:
        raise SystemExit(f"kernel substring {substr!r} matches {hits}")
    v = agg[hits[0]]
    return hits[0], sum(v) / len(v), len(v)


def traffic_summary(a) -> None:
    sys.path.insert(0, ROOT)
    from bench import source_hash
    fk, fetch_kib, nf = _pick(_per_kernel_kib(a.fetch), a.rocprof_kernel)
    wk, write_kib, nw = _pick(_per_kernel_kib(a.write), a.rocprof_kernel)
    _, fcopy_kib, _ = _pick(_per_kernel_kib(a.fetch_copy), "copyBuffer")
    _, wcopy_kib, _ = _pick(_per_kernel_kib(a.write_copy), "copyBuffer")
    f_scale = a.copy_bytes / (fcopy_kib * 1024.0)
    w_scale = a.copy_bytes / (wcopy_kib * 1024.0)
    fetch_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    d = {"workload": a.workload, "kernel": a.bench_kernel, "rocprof_kernel": fk,
         "source_hash": source_hash(), "fetch_kib_per_dispatch": fetch_kib,
         "write_kib_per_dispatch": write_kib, "copy_bytes": a.copy_bytes,
         "copy_fetch_kib": fcopy_kib, "copy_write_kib": wcopy_kib,
         "fetch_scale": f_scale, "write_scale": w_scale,
         "traffic_bytes": fetch_b + write_b, "dispatches": [nf, nw],
         "commands": {"fetch": a.cmd_fetch, "write": a.cmd_write, "copy": a.cmd_copy}}
    out = os.path.join(OUT_DIR, f"traffic_{a.workload}.json")
    json.dump(d, open(out, "w"), indent=1)
    txt = os.path.join(OUT_DIR, f"{a.bench_kernel}_{a.workload}_hbm_traffic.txt")
    open(txt, "w").write(
        f"# HBM traffic of {fk} on {a.workload} (rocprofv3 --pmc, one counter per run)\n"
        f"# commands:\n#   {a.cmd_fetch}\n#   {a.cmd_write}\n#   {a.cmd_copy}  (each counter)\n"
        f"FETCH_SIZE per dispatch: {fetch_kib:.1f} KiB over {nf} dispatches\n"
        f"WRITE_SIZE per dispatch: {write_kib:.1f} KiB over {nw} dispatches\n"
        f"plain copy of {a.copy_bytes} bytes: FETCH_SIZE {fcopy_kib:.1f} KiB, WRITE_SIZE {wcopy_kib:.1f} KiB\n"
        f"scale factors (true bytes / counter bytes): fetch {f_scale:.4f}, write {w_scale:.4f}\n"
        f"traffic per launch: fetch {fetch_b / 1e9:.4f} GB + write {write_b / 1e9:.4f} GB = "
        f"{(fetch_b + write_b) / 1e9:.4f} GB\n")


XCDS, SIMDS = 8, 1024          # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def busy_summary(a) -> None:
    ctr = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for r in _rows(a.counters):
        if a.rocprof_kernel in r["Kernel_Name"]:
            ctr[r["Kernel_Name"]][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[r["Kernel_Name"]].add(r["Dispatch_Id"])
    if len(ctr) != 1:
        raise SystemExit(f"kernel substring {a.rocprof_kernel!r} matches {list(ctr)}")
    name = next(iter(ctr))
    nd = len(disp[name])
    c = {k: v / nd for k, v in ctr[name].items()}          # per dispatch
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in _rows(a.trace)
            if r["Kernel_Name"] == name]
    dur_ns = sum(durs) / len(durs)
    gui = c["GRBM_GUI_ACTIVE"] / XCDS                        # GPU-active cycles of one XCD
    clock_ghz = gui / dur_ns
    busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * gui)
    tflops = c["SQ_INSTS_MFMA"] * a.mfma_flop / (dur_ns * 1e-9) / 1e12
    txt = os.path.join(OUT_DIR, f"{a.bench_kernel}_{a.workload}_mfma_busy.txt")
    open(txt, "w").write(
        f"# MFMA activity of {name} on {a.workload} (rocprofv3 --kernel-trace --pmc, one run)\n"
        f"# command: {a.cmd}\n"
        f"dispatches: {nd}; average duration {dur_ns / 1e3:.1f} us\n"
        f"GRBM_GUI_ACTIVE per XCD {gui:.4g} cycles -> clock {clock_ghz:.3f} GHz\n"
        f"SQ_VALU_MFMA_BUSY_CYCLES {c['SQ_VALU_MFMA_BUSY_CYCLES']:.4g} -> matrix cores busy "
        f"{100 * busy:.1f} % of SIMD cycles\n"
        f"SQ_INSTS_MFMA {c['SQ_INSTS_MFMA']:.4g} x {a.mfma_flop:.0f} FLOP -> {tflops:.1f} TFLOP/s, "
        f"{100 * tflops / a.peak_tflops:.1f} % of the {a.peak_tflops:.0f} TFLOP/s nominal peak\n"
        f"SQ_BUSY_CYCLES {c['SQ_BUSY_CYCLES']:.4g}\n")


STALL_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
                  "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                  "SQ_LDS_BANK_CONFLICT")
STALL_MEANING = {
    "SQ_WAIT_ANY": "waiting at s_waitcnt / barrier",
    "SQ_WAIT_INST_ANY": "waiting to issue (dependency or busy unit)",
    "SQ_WAIT_INST_LDS": "waiting to issue an LDS instruction",
    "SQ_ACTIVE_INST_ANY": "issuing any instruction",
    "SQ_ACTIVE_INST_VALU": "issuing vector ALU (incl. MFMA issue)",
    "SQ_ACTIVE_INST_LDS": "issuing LDS instructions",
    "SQ_LDS_BANK_CONFLICT": "LDS bank-conflict cycles",
}


def stall_summary(a) -> None:
    ctr = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for r in _rows(a.counters):
        if a.rocprof_kernel in r["Kernel_Name"]:
            ctr[r["Kernel_Name"]][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[r["Kernel_Name"]].add(r["Dispatch_Id"])
    if len(ctr) != 1:
        raise SystemExit(f"kernel substring {a.rocprof_kernel!r} matches {list(ctr)}")
    name = next(iter(ctr))
    nd = len(disp[name])
    c = {k: v / nd for k, v in ctr[name].items()}
    missing = [k for k in STALL_COUNTERS if k not in c]
    if missing:
        raise SystemExit(f"counters missing from {a.counters}: {missing}")
    wc = c["SQ_WAVE_CYCLES"]
    lines = [f"# Wave states of {name} on {a.workload} (rocprofv3 --kernel-trace --pmc, one run)",
             f"# command: {a.cmd}",
             f"dispatches: {nd}; SQ_WAVE_CYCLES {wc:.4g} per dispatch",
             "counter | per dispatch | fraction of wave cycles | meaning"]
    for k in STALL_COUNTERS[1:]:
        lines.append(f"{k} | {c[k]:.4g} | {c[k] / wc:.3f} | {STALL_MEANING[k]}")
    txt = os.path.join(OUT_DIR, f"{a.bench_kernel}_{a.workload}_stalls.txt")
    open(txt, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out_txt")
    t.add_argument("--cmd", required=True)
    r = sub.add_parser("traffic")
    for n in ("workload", "bench-kernel", "rocprof-kernel", "fetch", "write", "fetch-copy",
              "write-copy", "cmd-fetch", "cmd-write", "cmd-copy"):
        r.add_argument("--" + n, required=True)
    r.add_argument("--copy-bytes", type=int, required=True)
    b = sub.add_parser("busy")
    for n in ("workload", "bench-kernel", "rocprof-kernel", "counters", "trace", "cmd"):
        b.add_argument("--" + n, required=True)
    b.add_argument("--mfma-flop", type=float, required=True)
    b.add_argument("--peak-tflops", type=float, required=True)
    st = sub.add_parser("stalls")
    for n in ("workload", "bench-kernel", "rocprof-kernel", "counters", "cmd"):
        st.add_argument("--" + n, required=True)
    a = ap.parse_args()
    if a.cmd_name == "trace":
        trace_summary(a.stats_csv, a.out_txt, a.cmd)
    elif a.cmd_name == "busy":
        busy_summary(a)
    elif a.cmd_name == "stalls":
        stall_summary(a)
    else:
        traffic_summary(a)


if __name__ == "__main__":
    main()
