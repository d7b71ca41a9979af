"""Per-task timestamp pass of the persistent kernel: the per-layer hop timeline and each compute unit's idle share.

python -m decode_megakernel_wg_amd.trace [--workload b1_8k] [--warmup 3]

Runs the workload's first steps, then one step with MK_DBG_TIMESTAMPS (every task records, on the 100 MHz
wall clock: its claim, the moment its dependency waits ended, its end, the compute unit it ran on, and up
to four sub-phase marks).  Prints a markdown summary:
 - the step's span and the time of the same step without timestamps (the recording's overhead);
 - per layer, medians over the layers other than the first and last, relative to the moment the layer's
   input was complete (the end of the last residual epilogue of the previous layer): when the tasks of each
   kind were claimed, when their waits ended and when they ended;
 - per compute unit, the share of the step spent inside task bodies with dependencies met, spinning in a
   dependency wait, and outside any task (taking the next task, the LM head's closing phase, drained).
Only the kernel's own clock is read; nothing here changes the schedule except the recording stores.
"""
from __future__ import annotations

import argparse
import time

import numpy as np

OPS = {1: "EMBED", 3: "QKV", 4: "ATTN", 5: "UP", 6: "OPROJ", 7: "DOWN", 8: "MERGE"}
TICK_US = 0.01  # 100 MHz


def run(workload: str, warmup: int):
    import torch

    from synth import workloads as W

    from . import mk
    from .session import Session

    w = W.make(workload, steps=warmup + 2)
    sess = Session(w)
    tasks = sess.h.mk_build_tasks(sess.seq_rows_host[0], want_tasks=True)
    for _ in range(warmup):
        sess.step()
    sess.status()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    sess.step()
    e1.record()
    sess.status()
    plain_ms = e0.elapsed_time(e1)
    sess.h.mk_debug_set(mk.MK_DBG_TIMESTAMPS)
    e0.record()
    sess.step()
    e1.record()
    sess.status()
    traced_ms = e0.elapsed_time(e1)
    ts = sess.h.mk_debug_read(mk.MK_DBGK_TIMESTAMPS, (len(tasks), 8), np.uint64).astype(np.int64)
    return w, tasks, ts, plain_ms, traced_ms


def summarize(w, tasks, ts, plain_ms, traced_ms):
    op = tasks[:, 0]
    layer = tasks[:, 1]
    claim, met, end = ts[:, 0], ts[:, 1], ts[:, 2]
    # tasks that ran (the expert tiles of slots a layer leaves unused are passed over and record nothing)
    ran = end > 0
    t_first = claim[ran].min()
    span_us = (end[ran].max() - t_first) * TICK_US
    L = w.shape.n_layers
    lines = [f"workload `{w.name}`, batch {w.B}, {len(tasks)} tasks, {int(ran.sum())} of them run (the others are "
             "expert tiles of unused slots, passed over)", "",
             f"step without timestamps {plain_ms * 1e3:.1f} us; with timestamps {traced_ms * 1e3:.1f} us; "
             f"span of the recorded tasks {span_us:.1f} us (the LM head's closing phase follows the last task)", ""]
    # layer input complete: the earliest moment a QKV tile of the layer saw all row tiles of its input
    # (their waits end when the last row tile's residual epilogue has counted itself)
    t0 = np.zeros(L, np.int64)
    for l in range(L):
        m = (op == 3) & (layer == l) & ran
        t0[l] = met[m][met[m] > 0].min()
    per = np.diff(t0) * TICK_US
    lines += [f"layer period (input complete to next input complete), median over layers 1..{L - 2}: "
              f"{np.median(per[1:]):.1f} us (min {per.min():.1f}, max {per.max():.1f})", "",
              "| task | count per layer | claimed (median, latest) | waits ended (median, latest) | ended (median, latest) | "
              "marks after the waits (median) |",
              "|---|---|---|---|---|---|"]
    mid = range(1, L - 1)
    for o in (3, 4, 5, 8, 6, 7):
        rows = {"claim": [], "met": [], "end": [], "cl_max": [], "met_max": [], "end_max": []}
        marks = [[] for _ in range(4)]
        cnt = 0  # tasks of the kind that ran in a layer (the last layer seen)
        for l in mid:
            m = (op == o) & (layer == l) & ran
            if not m.any():
                continue
            cnt = int(m.sum())
            base = t0[l]
            rel = lambda v: (v[m] - base) * TICK_US  # noqa: E731
            c, e = rel(claim), rel(end)
            mm = met[m]
            mt = (np.where(mm > 0, mm, claim[m]) - base) * TICK_US
            rows["claim"].append(np.median(c))
            rows["cl_max"].append(c.max())
            rows["met"].append(np.median(mt))
            rows["met_max"].append(mt.max())
            rows["end"].append(np.median(e))
            rows["end_max"].append(e.max())
            mabs = np.where(mm > 0, mm, claim[m])
            for k in range(4):
                mk_ = ts[m, 4 + k]
                ok = mk_ > 0
                if ok.any():
                    marks[k].append(np.median((mk_[ok] - mabs[ok]) * TICK_US))
        if cnt:
            md = {k: np.median(v) for k, v in rows.items()}
            mtxt = ", ".join(f"m{k} {np.median(v):+.1f}" for k, v in enumerate(marks) if v)
            lines.append(f"| {OPS[o]} | {cnt} | {md['claim']:+.1f}, {md['cl_max']:+.1f} | {md['met']:+.1f}, {md['met_max']:+.1f} | "
                         f"{md['end']:+.1f}, {md['end_max']:+.1f} | {mtxt} |")
    lines += ["", "Times in us relative to the layer's input being complete (negative: before it).  Marks: GEMV tiles "
              "m0 = inputs staged, m1 = tile computed, m2 (UP) = expert weights requested; attention m0 = queries "
              "staged, m1 = cached positions done, m2 = partials published, m3 = merge started (last split only, when no "
              "merge tasks); merge tasks m0 = waits ended, m1 = the splits' weights formed (partials landed)."]
    # per compute unit: time in task bodies (waits met), in waits, outside tasks, over the recorded span
    cu = (ts[:, 3] >> 32) * 65536 + ((ts[:, 3] >> 8) & 0xFFFF)
    keys = np.unique(cu[ran])
    wait_f, body_f, out_f = [], [], []
    span = end[ran].max() - t_first
    for k in keys:
        m = (cu == k) & ran
        c, mt, e = claim[m], met[m], end[m]
        mt = np.where(mt > 0, mt, c)
        wait = (mt - c).sum()
        body = (e - mt).sum()
        wait_f.append(wait / span)
        body_f.append(body / span)
        out_f.append(1 - (wait + body) / span)
    wait_f, body_f, out_f = map(np.array, (wait_f, body_f, out_f))
    lines += ["", f"compute units seen: {len(keys)}", "",
              "| share of the recorded span | mean over CUs | min | max |", "|---|---|---|---|",
              f"| in task bodies (dependencies met) | {body_f.mean():.3f} | {body_f.min():.3f} | {body_f.max():.3f} |",
              f"| spinning in dependency waits | {wait_f.mean():.3f} | {wait_f.min():.3f} | {wait_f.max():.3f} |",
              f"| outside tasks (taking tasks, drained) | {out_f.mean():.3f} | {out_f.min():.3f} | {out_f.max():.3f} |"]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="b1_8k")
    ap.add_argument("--warmup", type=int, default=3)
    a = ap.parse_args()
    t = time.time()
    w, tasks, ts, plain_ms, traced_ms = run(a.workload, a.warmup)
    print(summarize(w, tasks, ts, plain_ms, traced_ms))
    print(f"\n(run took {time.time() - t:.1f} s)")


if __name__ == "__main__":
    main()
