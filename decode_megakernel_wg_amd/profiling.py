"""rocprofv3 passes over bench.py and their summaries (markdown, one file per kernel, workload and pass).

python -m decode_megakernel_wg_amd.profiling trace WORKLOAD [--steps 32] [--gemv mfma|valu]
python -m decode_megakernel_wg_amd.profiling hbm WORKLOAD [--gemv mfma|valu]      FETCH_SIZE and WRITE_SIZE, calibrated
python -m decode_megakernel_wg_amd.profiling counters WORKLOAD                     LDS bank conflicts, busy CUs, occupancy, MFMA
python -m decode_megakernel_wg_amd.profiling timeline WORKLOAD                     per-task timestamp pass (trace.py)
python -m decode_megakernel_wg_amd.profiling probe                                 synchronisation / streaming costs (hop_probe)

Each pass runs `rocprofv3 ... -- python3 bench.py --workload WORKLOAD ... --no-cpu-baseline` as a child process
under a time limit of its own, from /tmp, with the raw output under OUT (default gpurun_out/rocprof), and
writes its summary to OUT/summaries/mk_persistent_<workload>_<pass>.md: the command, the kernel source hash
(bench.kernel_source_hash), and the figures of the persistent kernel's dispatches (the decode steps; the fill
kernels that generate the synthetic inputs are listed in the trace but are not part of a step).

HBM traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the persistent kernel, each scaled by what the
same counter reads for a plain copy of exactly 1 GiB (hbm_calib.py: FETCH_SIZE reads half of the bytes on this
part, WRITE_SIZE all of them).  Counter figures of the other passes are sums over the counter's shader
engines and XCDs, per dispatch, averaged over the dispatches.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
KERNEL = "mk_persistent"
CALIB = "neg"  # the calibration copy: torch's elementwise negation kernel

COUNTER_PASSES = {
    "lds": ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_LDS", "GRBM_GUI_ACTIVE"],
    "occupancy": ["SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_WAVES",
                  "GRBM_GUI_ACTIVE"],
    "mfma": ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU",
             "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
}
N_CU = 256


def source_hash():
    sys.path.insert(0, ROOT)
    import bench

    return bench.kernel_source_hash()


def run(cmd, timeout, log):
    """Run a profiling command (a list) from /tmp with TMPDIR=/tmp; raise if it fails or times out."""
    env = dict(os.environ, TMPDIR="/tmp", PYTHONPATH=ROOT)
    print(f"[profiling] {' '.join(cmd)}", flush=True)
    with open(log, "w") as fh:
        r = subprocess.run(["timeout", "-k", "10", str(timeout)] + cmd, cwd="/tmp", env=env, stdout=fh, stderr=subprocess.STDOUT)
    # rocprofv3 itself may end with a segmentation fault (139) after the program finished and its files are
    # complete; the summaries then fail on missing files if they are not
    if r.returncode not in (0, 139):
        raise RuntimeError(f"{cmd[0]} failed ({r.returncode}); see {log}")


def bench_cmd(workload, steps, warmup, gemv):
    c = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload, "--steps", str(steps), "--warmup", str(warmup),
         "--no-cpu-baseline"]
    if gemv != "mfma":
        c += ["--gemv", gemv]
    return c


def rocprof(args, out_dir, name, prog, timeout, log):
    run(["rocprofv3"] + args + ["-f", "csv", "-d", out_dir, "-o", name, "--"] + prog, timeout, log)


def find(out_dir, suffix):
    hits = sorted(glob.glob(os.path.join(out_dir, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {out_dir}")
    return hits[-1]


def counter_rows(out_dir):
    """{(dispatch id, kernel name): {counter: summed value}} from a counter-collection CSV."""
    rows = {}
    with open(find(out_dir, "counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            d = rows.setdefault(key, {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return rows


def per_dispatch(rows, kernel_substr):
    ds = [v for (_, k), v in sorted(rows.items()) if kernel_substr in k]
    if not ds:
        raise RuntimeError(f"no dispatch of a kernel named *{kernel_substr}* in the counters")
    return ds


def header(title, commands, extra=""):
    lines = [f"# {title}", "", "Commands (run on one MI355X; `R` = repository root; each under `timeout`, from /tmp with TMPDIR=/tmp):",
             "", "```"] + commands + ["```", "", f"Kernel source hash (sha256 of decode_megakernel_wg_amd/csrc/*, first 16 hex): "
                                      f"`{source_hash()}`", ""]
    if extra:
        lines += [extra, ""]
    return lines


def show(cmd):
    return " ".join(c.replace(ROOT, "$R").replace(sys.executable, "python3") for c in cmd)


def do_trace(a, out):
    d = os.path.join(out, f"trace_{a.workload}_{a.gemv}")
    prog = bench_cmd(a.workload, a.steps, 2, a.gemv)
    args = ["--kernel-trace", "--stats"]
    rocprof(args, d, "t", prog, 900, os.path.join(out, f"trace_{a.workload}_{a.gemv}.log"))
    stats = find(d, "kernel_stats.csv")
    lines = header(f"rocprofv3 kernel trace: persistent decode kernel, workload {a.workload}" +
                   (f", GEMV tiles on the {a.gemv.upper()}" if a.gemv != "mfma" else ""),
                   [f"rocprofv3 {' '.join(args)} -f csv -d $OUT -o t -- {show(prog)}"])
    lines += ["| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    with open(stats) as fh:
        for r in csv.DictReader(fh):
            name = r["Name"]
            short = name if len(name) <= 90 else name[:87] + "..."
            lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                         f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
    lines += ["", f"The `{KERNEL}` row is the decode step (one launch per step; {a.steps} timed steps and 2 warm-up steps); the fill "
              "kernels generate the synthetic weights and KV cache before the timed region."]
    bl = [l for l in open(os.path.join(out, f"trace_{a.workload}_{a.gemv}.log")) if l.startswith("{")]
    if bl:
        lines += ["", "bench.py line of the same run:", "", "```", bl[-1].strip(), "```"]
    return f"mk_persistent_{a.workload}_kernel_trace" + ("" if a.gemv == "mfma" else f"_{a.gemv}"), lines


def calib(out, counter):
    d = os.path.join(out, f"calib_{counter}")
    prog = [sys.executable, "-m", "decode_megakernel_wg_amd.hbm_calib"]
    rocprof(["--pmc", counter], d, "c", prog, 300, os.path.join(out, f"calib_{counter}.log"))
    v = [x[counter] for x in per_dispatch(counter_rows(d), CALIB)]
    return max(v), prog


def do_hbm(a, out):
    prog = bench_cmd(a.workload, 3, 1, a.gemv)
    res, cmds = {}, []
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d = os.path.join(out, f"pmc_{counter}_{a.workload}_{a.gemv}")
        rocprof(["--pmc", counter], d, "p", prog, 600, os.path.join(out, f"pmc_{counter}_{a.workload}.log"))
        res[counter] = [x[counter] for x in per_dispatch(counter_rows(d), KERNEL)]
        cmds.append(f"rocprofv3 --pmc {counter} -f csv -d $OUT -o p -- {show(prog)}")
    cal = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        cal[counter], cprog = calib(out, counter)
        cmds.append(f"rocprofv3 --pmc {counter} -f csv -d $OUT -o c -- {show(cprog)}")
    gib_kib = 1024.0 * 1024.0
    f_fac, w_fac = gib_kib / cal["FETCH_SIZE"], gib_kib / cal["WRITE_SIZE"]
    fetch = sum(res["FETCH_SIZE"]) / len(res["FETCH_SIZE"])
    write = sum(res["WRITE_SIZE"]) / len(res["WRITE_SIZE"])
    rd, wr = fetch * f_fac * 1024, write * w_fac * 1024
    lines = header(f"HBM traffic counters: persistent decode kernel, workload {a.workload}" +
                   (f", GEMV tiles on the {a.gemv.upper()}" if a.gemv != "mfma" else ""), cmds,
                   "Two counter passes over the bench command (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), and the same two "
                   "passes over a calibration kernel that reads and writes exactly 1 GiB (hbm_calib.py).")
    lines += ["| quantity | value |", "|---|---|",
              f"| calibration FETCH_SIZE per dispatch (KiB), 1 GiB read | {cal['FETCH_SIZE']:.1f} (factor {f_fac:.4f}) |",
              f"| calibration WRITE_SIZE per dispatch (KiB), 1 GiB written | {cal['WRITE_SIZE']:.1f} (factor {w_fac:.4f}) |",
              f"| {KERNEL} FETCH_SIZE per dispatch (KiB), {len(res['FETCH_SIZE'])} dispatches | {fetch:.1f} (min "
              f"{min(res['FETCH_SIZE']):.1f}, max {max(res['FETCH_SIZE']):.1f}) |",
              f"| {KERNEL} WRITE_SIZE per dispatch (KiB), {len(res['WRITE_SIZE'])} dispatches | {write:.1f} (min "
              f"{min(res['WRITE_SIZE']):.1f}, max {max(res['WRITE_SIZE']):.1f}) |",
              f"| HBM bytes read per launch (calibrated) | {rd:.4e} |",
              f"| HBM bytes written per launch (calibrated) | {wr:.4e} |",
              f"| traffic_bytes_per_launch | {int(round(rd + wr))} |"]
    return f"mk_persistent_{a.workload}_hbm_counters" + ("" if a.gemv == "mfma" else f"_{a.gemv}"), lines


def do_counters(a, out):
    prog = bench_cmd(a.workload, 3, 1, a.gemv)
    vals, cmds = {}, []
    for name, counters in COUNTER_PASSES.items():
        d = os.path.join(out, f"pmc_{name}_{a.workload}")
        rocprof(["--pmc"] + counters, d, "p", prog, 600, os.path.join(out, f"pmc_{name}_{a.workload}.log"))
        ds = per_dispatch(counter_rows(d), KERNEL)
        for c in counters:
            vals[c] = sum(x.get(c, 0.0) for x in ds) / len(ds)
        cmds.append(f"rocprofv3 --pmc {' '.join(counters)} -f csv -d $OUT -o p -- {show(prog)}")
    gui = vals["GRBM_GUI_ACTIVE"]  # GPU clock cycles of the dispatch (summed over the 8 XCDs)
    cycles = gui / 8.0
    lines = header(f"rocprofv3 counters: persistent decode kernel, workload {a.workload} (LDS, busy CUs, occupancy, matrix cores)",
                   cmds, "Per dispatch, averaged over the dispatches of the persistent kernel (sums over shader engines and "
                         "XCDs).  GRBM_GUI_ACTIVE / 8 = cycles of the dispatch per XCD.")
    lds_acc = vals["SQ_LDS_IDX_ACTIVE"] - vals["SQ_LDS_BANK_CONFLICT"]
    lines += ["| figure | value | from |", "|---|---|---|",
              f"| dispatch cycles (per XCD) | {cycles:.4g} | GRBM_GUI_ACTIVE / 8 |",
              f"| LDS bank conflicts per LDS access cycle | {vals['SQ_LDS_BANK_CONFLICT'] / max(lds_acc, 1):.4f} | "
              "SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT) |",
              f"| share of CU time stalled by LDS bank conflicts | {vals['SQ_LDS_BANK_CONFLICT'] / (cycles * N_CU):.4f} | "
              "SQ_LDS_BANK_CONFLICT / (cycles x 256 CUs) |",
              f"| LDS instructions per dispatch | {vals['SQ_INSTS_LDS']:.4g} | SQ_INSTS_LDS |",
              f"| busy-CU share of the dispatch | {vals['SQ_BUSY_CU_CYCLES'] / (cycles * N_CU):.4f} | "
              "SQ_BUSY_CU_CYCLES / (cycles x 256 CUs) |",
              f"| mean resident waves per CU | {4 * vals['SQ_WAVE_CYCLES'] / (cycles * N_CU):.3f} (of 8 launched per CU) | "
              "4 x SQ_WAVE_CYCLES / (cycles x 256 CUs) |",
              f"| share of wave time waiting (any) | {vals['SQ_WAIT_ANY'] / max(vals['SQ_WAVE_CYCLES'], 1):.4f} | "
              "SQ_WAIT_ANY / SQ_WAVE_CYCLES |",
              f"| share of wave time issuing an instruction | {vals['SQ_ACTIVE_INST_ANY'] / max(vals['SQ_WAVE_CYCLES'], 1):.4f} | "
              "SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES |",
              f"| waves launched per dispatch | {vals['SQ_WAVES']:.0f} | SQ_WAVES |",
              f"| BF16 matrix-core ops per dispatch | {vals['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.4g} | "
              "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 |",
              f"| matrix-core busy share (per SIMD) | {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (cycles * N_CU * 4):.4f} | "
              "SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs) |",
              f"| MFMA instructions / VALU instructions per dispatch | {vals['SQ_INSTS_MFMA']:.4g} / {vals['SQ_INSTS_VALU']:.4g} | "
              "SQ_INSTS_MFMA, SQ_INSTS_VALU |"]
    return f"mk_persistent_{a.workload}_counters", lines


def do_timeline(a, out):
    from . import trace

    w, tasks, ts, plain, traced = trace.run(a.workload, 3)
    lines = header(f"Per-task timestamp pass: persistent decode kernel, workload {a.workload}",
                   [f"python3 -m decode_megakernel_wg_amd.trace --workload {a.workload}"],
                   "The kernel's own 100 MHz wall-clock timestamps (MK_DBG_TIMESTAMPS) of one step after 3 warm-up steps.")
    lines += trace.summarize(w, tasks, ts, plain, traced).split("\n")
    return f"mk_persistent_{a.workload}_timeline", lines


def do_probe(a, out):
    """Run the measurement program hop_probe (built in-tree by build.build_probe) and keep its tables."""
    prog = os.path.join(HERE, "hop_probe")
    if not os.path.exists(prog):
        raise RuntimeError("hop_probe is not built (decode_megakernel_wg_amd.build.build_probe)")
    log = os.path.join(out, "hop_probe.log")
    run([prog], 240, log)
    with open(log) as fh:
        body = [l.rstrip("\n") for l in fh if l.strip() != "done"]
    lines = header("Synchronisation and streaming costs on this part (hop_probe)",
                   ["decode_megakernel_wg_amd/hop_probe   (built from decode_megakernel_wg_amd/hop_probe.hip by build.build_probe)"],
                   "A standalone program, not the decode kernel: one dependency hop between workgroups on different XCDs "
                   "(counter protocol against a flag in the data), int64 atomic additions against plain stores, "
                   "re-reads of a buffer that fits the last-level cache, and reads of a payload another workgroup has "
                   "just published.  Wall-clock ticks at 100 MHz; HIP events.")
    return "mk_probe_sync_and_streaming", lines + body


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=("trace", "hbm", "counters", "timeline", "probe"))
    ap.add_argument("workload", nargs="?", default="b1_8k")
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--gemv", choices=("mfma", "valu"), default="mfma")
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "rocprof"))
    a = ap.parse_args()
    out = os.path.abspath(a.out)
    os.makedirs(os.path.join(out, "summaries"), exist_ok=True)
    name, lines = {"trace": do_trace, "hbm": do_hbm, "counters": do_counters, "timeline": do_timeline,
                   "probe": do_probe}[a.what](a, out)
    path = os.path.join(out, "summaries", name + ".md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"[profiling] wrote {path}", flush=True)


if __name__ == "__main__":
    main()
