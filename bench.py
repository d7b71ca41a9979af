"""Decode throughput of the persistent megakernel on one MI355X, and its fraction of HBM speed-of-light.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload b1_8k] [--no-cpu-baseline] [--gemv mfma|valu]

A step is one decode step (one launch of the persistent kernel over the whole model) for the
workload's batch; inputs (weights, KV cache, page tables, lengths) are resident in HBM before the
timed region and every step feeds the previous step's greedy tokens back on the device.  Prints one
JSON line.  Speed-of-light bytes per step are the active weights (distinct experts counted once per
layer, from the kernel's own routing record) plus the K/V read over every attended position, at 8 TB/s.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD_TEXT = {
    "b1_8k": "48-layer parallel-transformer MoE decoder (d_model 2048, 32 q heads / 4 KV heads x 128, 128 SwiGLU experts "
             "top-8, d_ffn 768, vocab 262144, BF16 weights), batch 1, 8192 prior KV positions in 16-token pages, greedy decode",
    "b8_ragged_uniform": "same 48-layer model, batch 8, contexts log-uniform in [1024, 32768], shuffled pages, uniform routing",
    "b8_ragged_skewed": "same 48-layer model, batch 8, contexts log-uniform in [1024, 32768], shuffled pages, "
                        "router bias -1.5 ln(rank) (skewed routing)",
    "long_64k": "same 48-layer model, batch 1, 65536 prior positions, split-KV attention",
    "long_128k": "same 48-layer model, batch 1, 131072 prior positions, split-KV attention",
    "long_256k": "same 48-layer model, batch 1, 262144 prior positions, split-KV attention",
    "tp2_b1_8k": "one GPU's share of the same model under 2-way tensor parallelism (16 q heads / 2 KV heads x 128, "
                 "128 experts top-8 with d_ffn 384, vocab 131072, d_model 2048, 48 layers), batch 1, 8192 prior KV positions; "
                 "the per-layer exchanges between the two GPUs are not part of this single-GPU run",
    "continuous": "same 48-layer model under continuous batching: arrivals every ~64 steps (exponential gaps), "
                  "geometric output lengths (mean 256), prefixes log-uniform in [512, 65536], LIFO page free list, "
                  "live batch 1-8, task list rebuilt every step on the host while the previous step runs",
}


def kernel_source_hash():
    """sha256 (first 16 hex) over the persistent kernel's sources, names included, in name order."""
    import glob
    import hashlib

    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "decode_megakernel_wg_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload, gemv="mfma"):
    """Calibrated HBM bytes per launch of the persistent kernel from the committed counter summary of this
    workload (and GEMV engine), or None when there is none or it was taken on other kernel sources."""
    import re

    suffix = "" if gemv == "mfma" else f"_{gemv}"
    path = os.path.join(ROOT, "profiles", f"mk_persistent_{workload}_hbm_counters{suffix}.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        text = fh.read()
    h = re.search(r"Kernel source hash[^`]*`([0-9a-f]+)`", text)
    t = re.search(r"\| traffic_bytes_per_launch \| (\d+) \|", text)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return int(t.group(1))


def percentile(xs, q):
    """q-th percentile of the per-step times (nearest rank)."""
    v = sorted(xs)
    return v[min(len(v) - 1, max(0, -(-q * len(v) // 100) - 1))]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def unique_experts_per_layer(sess):
    import numpy as np

    from decode_megakernel_wg_amd import mk

    s = sess.shape
    sel = sess.h.mk_debug_read(mk.MK_DBGK_ROUTE_SEL, (s.n_layers, sess.B, s.top_k), np.int32)
    return [len(np.unique(sel[l])) for l in range(s.n_layers)]


def run_gpu(workload, steps, warmup, model=None, gemv="mfma"):
    import numpy as np
    import torch

    from decode_megakernel_wg_amd import roofline as R
    from decode_megakernel_wg_amd.session import Session
    from synth import workloads as W

    w = W.make(workload, steps=steps + warmup)
    t0 = time.time()
    if model is None or model.shape != w.shape:
        log(f"generating {w.shape.n_layers}-layer synthetic weights in HBM")
        model = W.DeviceModel(w.shape)
    log(f"generating KV prefixes {w.ctx}")
    sess = Session(w, model=model)
    if gemv == "valu":  # GEMV tiles on the VALU instead of the matrix cores (batch 1; engine comparison)
        from decode_megakernel_wg_amd import mk

        sess.h.mk_debug_set(mk.MK_DBG_VALU_GEMV)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f} s; warmup {warmup} steps")
    for _ in range(warmup):
        sess.step()
    sess.status()
    # bytes per timed step: weights with the distinct experts actually used + KV read at each step's lengths
    sess.rewind(0)
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    uniq = []
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(steps):
        sess.step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    sess.status()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    total_ms = evs[0].elapsed_time(evs[-1])
    # routing of the last step (the kernel records it every step); distinct tokens of the step
    uniq = unique_experts_per_layer(sess)
    n_tok = len(set(int(t) for t in sess.next_tokens())) if sess.B > 1 else 1
    bytes_steps = [R.step_bytes(w.shape, sess.seq_rows_host[i], uniq, n_tok) for i in range(steps)]
    avg_bytes = sum(bytes_steps) / steps
    ms_per_step = total_ms / steps
    return dict(w=w, sess=sess, model=model, ms_per_step=ms_per_step, per_step_ms=per, avg_bytes=avg_bytes, uniq=uniq,
                tok_s=steps * w.B / (total_ms * 1e-3), kernel_ms=sum(per) / steps)


def run_gpu_continuous(steps, warmup):
    """Continuous batching over the schedule's first `steps` steps, in two passes over the same steps.
    Pass 1 runs step by step and reads each step's routing back (distinct experts per layer, for the bytes).
    Pass 2 is the timed one: steps are enqueued back to back, the host rebuilding step t+1's task list while
    the GPU runs step t; tok/s = tokens / (wall time - GPU time of the admitted prefixes' writes), and each
    kernel is timed with HIP events on the launch stream (for the roofline).  Both passes must end on the
    same greedy tokens.  Warm-up: the first `warmup` steps, then a restart from step 0."""
    import numpy as np
    import torch

    from decode_megakernel_wg_amd import mk
    from decode_megakernel_wg_amd import roofline as R
    from decode_megakernel_wg_amd.continuous import ContinuousSession
    from synth import workloads as W

    t0 = time.time()
    log("generating 48-layer synthetic weights in HBM")
    sess = ContinuousSession(W.FULL, steps)
    log(f"setup {time.time() - t0:.1f} s; pool {sess.n_pages} pages; warmup {warmup} steps")
    for _ in range(min(warmup, steps)):
        sess.step()
    sess.status()
    sess.reset()
    s = W.FULL
    stream = torch.cuda.current_stream()
    kern, nbytes, ntok = [], [], 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)  # pass-1 kernel time (logged)
    orig = sess.h.mk_decode_step

    def timed_step(*a, **k):
        e0.record(stream)
        orig(*a, **k)
        e1.record(stream)

    sess.h.mk_decode_step = timed_step
    last = None
    for i in range(steps):
        sids, _, pos, nxt, _ = sess.step()
        B = len(sids)
        kern.append(e0.elapsed_time(e1))
        sel = sess.h.mk_debug_read(mk.MK_DBGK_ROUTE_SEL, (s.n_layers, B, s.top_k), np.int32)
        uniq = [len(np.unique(sel[l])) for l in range(s.n_layers)]
        nbytes.append(R.step_bytes(s, pos, uniq, len(set(int(t) for t in nxt))))
        ntok += B
        last = nxt
        if (i + 1) % 256 == 0:
            log(f"pass 1 step {i + 1}/{steps}: batch {B}")
    sess.status()
    sess.h.mk_decode_step = orig
    sess.reset()
    wall, fill_s, kern2 = sess.run_pipelined(steps, kernel_events=True)
    sess.status()
    B = len(sess.steps[steps - 1].sids)
    nxt = mk.read_device(sess.next_ptr, 4 * B)
    if not np.array_equal(nxt, last):
        raise RuntimeError("pipelined pass ended on other tokens than the step-by-step pass")
    log(f"pass 2: {wall:.3f} s wall, {fill_s:.3f} s of prefix writes")
    log(f"kernel time per step: pass 1 {sum(kern) / steps:.3f} ms, pass 2 {1e3 * sum(kern2) / steps:.3f} ms")
    return dict(sess=sess, wall_s=wall - fill_s, kernel_s=sum(kern2), kernel_ms=[1e3 * k for k in kern2], bytes=sum(nbytes), tokens=ntok,
                batch_sizes=[len(st.sids) for st in sess.steps[:steps]], max_ctx=int(max(max(st.pos) for st in sess.steps[:steps])))


def cpu_baseline_continuous(min_seconds=10.0, max_steps=16):
    """The CPU oracle on consecutive steps of the continuous-batching schedule (free-running on its own tokens),
    until `min_seconds` of timed work or `max_steps` steps; prefix writes and weight generation not timed."""
    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import oracle as O
    from oracle_runner import OracleRun
    from synth import continuous as CB
    from synth import synth
    from synth import workloads as W

    steps, seqs, n_pages, max_pages = CB.schedule(max_steps, n_pages=8192)
    s = W.FULL
    orc = OracleRun(W.Workload("continuous", s, [], max_steps), np.zeros((0, max_pages), np.int32), n_pages, keep_all=False)
    last, timed, n, ntok = {}, 0.0, 0, 0
    for st in steps:
        if timed >= min_seconds:
            break
        for sid in st.admitted:
            q = seqs[sid]
            synth.fill_kv_host(orc.kv, 0, s.n_kv_heads, s.d_head, W.PAGE, np.array(q.pages, np.int32), sid, 0, q.prefix, W.SEED_KV,
                               W.KV_SIGMA)
        pt = CB.page_table(st, seqs, max_pages)
        toks = np.array([last.get(sid, synth.token(W.SEED_TOK, sid, s.vocab)) for sid in st.sids], np.int32)
        pos = st.pos.astype(np.int64)
        B = len(st.sids)
        x = O.embed(orc.D, W.host_embed_rows(s, toks), np.arange(B, dtype=np.int32))
        for l in range(s.n_layers):
            hl = orc.layer_weights(l, [])
            nrm = np.stack([O.rmsnorm(x[b], hl.arrs[0]) for b in range(B)])
            need = set()
            for b in range(B):
                sel, _, _ = O.router(nrm[b], hl.arrs[5], s.top_k, None)
                need.update(int(e) for e in sel)
            Wl = orc.layer_weights(l, sorted(need))
            t1 = time.perf_counter()
            x, _ = O.layer(orc.D, Wl, pos, pt, orc.kv[l], x)
            timed += time.perf_counter() - t1
        t1 = time.perf_counter()
        _, nxt = O.head(orc.D, x, orc.final_norm, orc.lm_head)
        timed += time.perf_counter() - t1
        for b, sid in enumerate(st.sids):
            last[sid] = int(nxt[b])
        n += 1
        ntok += B
        log(f"oracle step {n}: timed {timed:.2f} s")
    return {"value": round(ntok / timed, 4), "unit": "tok/s", "cores": O.num_threads(), "kind": "oracle", **host_info(),
            "sample": f"the continuous-batching schedule's first {n} steps ({ntok} tokens, live batch "
                      f"{min(len(st.sids) for st in steps[:n])}-{max(len(st.sids) for st in steps[:n])}); fp64-accumulating C oracle "
                      f"with OpenMP; {timed:.2f} s of timed CPU work; prefix writes and host weight generation excluded"}


def host_info():
    """CPU model, sockets, logical CPUs and RAM of the host (lscpu, /proc/meminfo)."""
    info = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in ("Model name", "Socket(s)", "CPU(s)"):
                info[k.strip()] = v.strip()
    except Exception:  # noqa: BLE001 - reporting only
        pass
    try:
        with open("/proc/meminfo") as fh:
            kb = int(fh.readline().split()[1])
        info["ram_gib"] = round(kb / 2 ** 20, 1)
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": info.get("Model name"), "sockets": info.get("Socket(s)"), "logical_cpus": info.get("CPU(s)"),
            "ram_gib": info.get("ram_gib")}


def cpu_baseline(workload, min_seconds=10.0, max_steps=16):
    """The CPU oracle timed on consecutive greedy decode steps of the same workload (all layers and the LM head
    per step), until at least `min_seconds` of timed work or `max_steps` steps.  Each layer's synthetic weights
    are generated on the host before its timed call (generation is not timed)."""
    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import oracle as O
    from oracle_runner import OracleRun
    from synth import workloads as W

    w = W.make(workload, steps=max_steps)
    pt, n_pages = W.page_tables(w)
    t0 = time.time()
    orc = OracleRun(w, pt, n_pages, keep_all=False)
    log(f"oracle setup (KV + LM head generation) {time.time() - t0:.1f} s")
    s = w.shape
    tokens = np.array(w.tokens, np.int32)
    pos = np.array(w.ctx, np.int64)
    timed, steps = 0.0, 0
    while steps < max_steps and timed < min_seconds:
        x = O.embed(orc.D, W.host_embed_rows(s, tokens), np.arange(w.B, dtype=np.int32))
        for l in range(s.n_layers):
            hl = orc.layer_weights(l, [])
            n = np.stack([O.rmsnorm(x[b], hl.arrs[0]) for b in range(w.B)])
            need = set()
            for b in range(w.B):
                sel, _, _ = O.router(n[b], hl.arrs[5], s.top_k, w.router_bias)
                need.update(int(e) for e in sel)
            Wl = orc.layer_weights(l, sorted(need))
            t1 = time.perf_counter()
            x, _ = O.layer(orc.D, Wl, pos, pt, orc.kv[l], x)
            timed += time.perf_counter() - t1
        t1 = time.perf_counter()
        _, nxt = O.head(orc.D, x, orc.final_norm, orc.lm_head)
        timed += time.perf_counter() - t1
        tokens = np.asarray(nxt, np.int32)
        pos = pos + 1
        steps += 1
        log(f"oracle step {steps}: timed {timed:.2f} s")
    cores = O.num_threads()
    return {"value": round(steps * w.B / timed, 4), "unit": "tok/s", "cores": cores, "kind": "oracle", **host_info(),
            "sample": f"{steps} consecutive greedy decode steps of {workload} (all {s.n_layers} layers + LM head, batch {w.B}); "
                      f"fp64-accumulating C oracle with OpenMP; {timed:.2f} s of timed CPU work; host weight generation excluded"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="b1_8k", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gemv", choices=("mfma", "valu"), default="mfma",
                    help="engine of the GEMV tiles at batch 1: matrix cores (default) or VALU, for comparing the two")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from decode_megakernel_wg_amd import roofline as R

    if args.workload == "continuous":
        return main_continuous(args)
    r = run_gpu(args.workload, args.steps, args.warmup, gemv=args.gemv)
    w = r["w"]
    achieved = r["avg_bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
    sol_tok_s = R.sol_tokens_per_s(r["avg_bytes"], w.B)
    line = {
        "metric": "decode tok/s + % HBM speed-of-light, batch 1 @8K ctx and batch 8 ragged",
        "value": round(r["tok_s"], 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOAD_TEXT[args.workload]}", "global_batch": w.B,
                   "seq_len": int(max(w.ctx)), "parallelism": "single GPU, persistent megakernel"},
        "gemv_engine": args.gemv if w.B == 1 else "mfma",
        "sol_tok_s": round(sol_tok_s, 1),
        "pct_of_sol": round(100 * r["tok_s"] / sol_tok_s, 2),
        "sol_bytes_per_step": int(r["avg_bytes"]),
        "step_ms_p50": round(percentile(r["per_step_ms"], 50), 4),
        "step_ms_p99": round(percentile(r["per_step_ms"], 99), 4),
        "unique_experts_per_layer": int(round(sum(r["uniq"]) / len(r["uniq"]))),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(achieved / 8000.0, 4), "traffic": counter_traffic(args.workload, args.gemv)},
    }
    if not args.no_cpu_baseline:
        del r
        torch.cuda.empty_cache()
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)


def main_continuous(args):
    import torch

    r = run_gpu_continuous(args.steps, args.warmup)
    tok_s = r["tokens"] / r["wall_s"]
    achieved = r["bytes"] / r["kernel_s"] / 1e9
    sol_s = r["bytes"] / 8.0e12
    bs = r["batch_sizes"]
    line = {
        "metric": "decode tok/s + % HBM speed-of-light, batch 1 @8K ctx and batch 8 ragged",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * r["wall_s"] / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"continuous: {WORKLOAD_TEXT['continuous']}", "global_batch": max(bs),
                   "mean_batch": round(sum(bs) / len(bs), 3), "seq_len": r["max_ctx"], "parallelism": "single GPU, persistent megakernel"},
        "sol_tok_s": round(r["tokens"] / sol_s, 1),
        "pct_of_sol": round(100 * sol_s / r["wall_s"], 2),
        "sol_bytes_per_step": int(r["bytes"] / args.steps),
        "kernel_ms_per_step": round(1e3 * r["kernel_s"] / args.steps, 4),
        "kernel_ms_p50": round(percentile(r["kernel_ms"], 50), 4),
        "kernel_ms_p99": round(percentile(r["kernel_ms"], 99), 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(achieved / 8000.0, 4), "traffic": counter_traffic("continuous")},
    }
    if not args.no_cpu_baseline:
        del r
        torch.cuda.empty_cache()
        line["cpu_baseline"] = cpu_baseline_continuous()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
