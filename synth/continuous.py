"""Continuous-batching schedule: which sequences are live at each decode step, at which positions, in
which pages (no method arithmetic; shared by the oracle side and the GPU side).

Serving on the pages admits requests into the running decode batch and releases them when they end
(aimodeling.com "Cohere megakernel engine: one CUDA file, 1.58x vLLM on H100", section "Caveats": the
engine supports continuous batching over paged, ragged sequences).  The pages give no arrival process;
the reading used here:

* time is counted in decode steps; sequence 0 arrives at time 0 and the gaps between arrivals are
  exponential with mean 64 steps, rounded up (so at least one step);
* a sequence brings a synthetic KV prefix of log-uniform length in [512, 65536] positions and decodes
  a geometric number of tokens on {1, 2, ...} with p = 1/256 (mean 256);
* arrived sequences wait in FIFO order and are admitted while fewer than 8 are live; the live batch
  keeps admission order;
* an admitted sequence takes ceil((prefix + outputs) / 16) pages from a LIFO free list (initially
  pages 0, 1, 2, ... in order) and returns them after its last step;
* when nothing is live and nothing waits, the clock jumps to the next arrival (idle steps are not
  decode steps).

Draws: arrival gaps u01(seed 6, stream 0, i), output lengths u01(seed 7, stream 0, i), prefix lengths
loguniform(seed 3, stream 2) for sequence i.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import synth
from .workloads import PAGE, SEED_ARRIVE, SEED_LEN, SEED_OUTLEN

MEAN_GAP = 64.0
P_END = 1.0 / 256.0
PREFIX_LO, PREFIX_HI = 512, 65536
MAX_BATCH = 8


@dataclass
class Seq:
    sid: int
    arrive: int
    prefix: int
    out_len: int
    pages: list = field(default_factory=list)
    admitted_step: int = -1
    last_step: int = -1


@dataclass
class Step:
    sids: list          # live sequences in batch order
    pos: np.ndarray     # int32 [B]: prior positions of each (the new token's position)
    admitted: list      # sequences admitted just before this step (their prefixes must be written first)
    finished: list      # sequences whose last step this is (pages return to the free list after it)
    clock: int = 0      # arrival-process time of the step


def draws(n: int, lo: int = PREFIX_LO, hi: int = PREFIX_HI, mean_gap: float = MEAN_GAP):
    """Arrival times, prefix lengths and output lengths of sequences 0..n-1."""
    ug = synth.u01(SEED_ARRIVE, 0, 0, n)
    uo = synth.u01(SEED_OUTLEN, 0, 0, n)
    arrive = np.zeros(n, np.int64)
    for i in range(1, n):
        arrive[i] = arrive[i - 1] + max(1, math.ceil(-mean_gap * math.log1p(-float(ug[i]))))
    out_len = np.array([max(1, math.ceil(math.log1p(-float(u)) / math.log1p(-P_END))) for u in uo], np.int64)
    prefix = synth.loguniform_ints(SEED_LEN, 2, n, lo, hi)
    return arrive, prefix, out_len


def pages_for(prefix: int, out_len: int) -> int:
    return -(-(prefix + out_len) // PAGE)


def pool_pages(hi: int = PREFIX_HI, max_batch: int = MAX_BATCH) -> int:
    """A pool that holds max_batch sequences of the longest prefix and 4096 outputs each."""
    return max_batch * -(-(hi + 4096) // PAGE)


def schedule(n_steps: int, n_pages: int | None = None, lo: int = PREFIX_LO, hi: int = PREFIX_HI, max_batch: int = MAX_BATCH,
             mean_gap: float = MEAN_GAP):
    """The first n_steps decode steps.  Returns (steps, seqs, n_pages, max_pages_per_seq).  mean_gap: mean
    arrival gap in steps (64 for the workload; smaller gaps keep the batch full, for tests)."""
    n_pages = pool_pages(hi, max_batch) if n_pages is None else n_pages
    n_draw = n_steps + 64
    arrive, prefix, out_len = draws(n_draw, lo, hi, mean_gap)
    seqs = [Seq(i, int(arrive[i]), int(prefix[i]), int(out_len[i])) for i in range(n_draw)]
    free = list(range(n_pages - 1, -1, -1))  # stack: pop() gives page 0 first
    waiting, live, steps = [], [], []
    nxt, clock = 0, 0
    while len(steps) < n_steps:
        while nxt < n_draw and seqs[nxt].arrive <= clock:
            waiting.append(seqs[nxt])
            nxt += 1
        if not live and not waiting:
            if nxt >= n_draw:
                raise RuntimeError("ran out of drawn arrivals")
            clock = seqs[nxt].arrive  # idle: jump to the next arrival
            continue
        admitted = []
        while waiting and len(live) < max_batch:
            s = waiting[0]
            need = pages_for(s.prefix, s.out_len)
            if need > len(free):
                break  # FIFO: the head waits for pages
            waiting.pop(0)
            s.pages = [free.pop() for _ in range(need)]
            s.admitted_step = len(steps)
            live.append(s)
            admitted.append(s.sid)
        if not live:
            raise RuntimeError("page pool too small for the next sequence")
        t = len(steps)
        produced = {s.sid: t - s.admitted_step for s in live}
        pos = np.array([s.prefix + produced[s.sid] for s in live], np.int32)
        finished = [s.sid for s in live if produced[s.sid] + 1 == s.out_len]
        steps.append(Step([s.sid for s in live], pos, admitted, finished, clock))
        for s in [s for s in live if s.sid in finished]:
            s.last_step = t
            free.extend(reversed(s.pages))  # LIFO: the freed pages are the next ones handed out
            live.remove(s)
        clock += 1
    used = [s for s in seqs if s.admitted_step >= 0]
    max_pages = max(len(s.pages) for s in used)
    return steps, seqs, n_pages, max_pages


def page_table(steps_entry: Step, seqs, max_pages: int) -> np.ndarray:
    """int32 [B][max_pages]: the page lists of the step's sequences (-1 padded)."""
    pt = np.full((len(steps_entry.sids), max_pages), -1, np.int32)
    for b, sid in enumerate(steps_entry.sids):
        p = seqs[sid].pages
        pt[b, :len(p)] = p
    return pt
