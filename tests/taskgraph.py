"""CPU model of the task list's counter protocol, shared by the host tests and the GPU tests.

A task list is a topological order of 32-word descriptors; each task waits on up to four (counter, target)
pairs and, when it completes, arrives on / signals counters.  `complete` applies one task's counter effects,
`simulate` runs a list under the kernel's schedule with random interleavings, and `check_device_counters`
holds the device's counters at the end of a step (the kernel copies them just before resetting them,
MK_DBGK_COUNTERS) to the values the plan gives.  The descriptor word numbers and the counter-block order mirror the
library's layout (csrc/mk_desc.h); these tests fail if the two drift apart.
"""
from __future__ import annotations

import numpy as np

W_OP, W_LAYER, W_A, W_B, W_C, W_D, W_R0, W_R1, W_WAIT0, W_SIG, W_SIGN, W_ARR, W_ARRN, W_SIGR = 0, 1, 2, 3, 4, 5, 6, 7, 8, 16, 17, 18, 19, 20
W_RT, W_ARR2, W_ARRN2, W_RSIG, W_RSIGR = 22, 24, 25, 26, 27
OP_EMBED, OP_QKV, OP_ATTN, OP_UP, OP_OPROJ, OP_DOWN, OP_MERGE = 1, 3, 4, 5, 6, 7, 8
UNUSED_SLOT = 0x80000000


def counter_layout(L, Hkv, B, n_slots, n_rt):
    """Index of the first counter of each block, in the library's order."""
    o = 0
    lay = {}
    for name, size in (("ticket", 32), ("done", 32), ("xready", L + 1), ("qkv_done", L * Hkv),
                       ("router_arrive", L), ("slot_ready", L * n_slots), ("slots_used", L), ("attn_arrive", L * B * Hkv),
                       ("attn_done", L * Hkv),
                       ("up_done", L * n_slots), ("resid_arrive", L * n_rt), ("lm_arrive", 1), ("lm_pool", 1)):
        lay[name] = (o, size)
        o += size
    lay["total"] = (o + 31) & ~31
    return lay


def complete(w, ctr):
    """Counter effects of a finished task: an arrival (only the last arriver goes on), then the signal of
    W_SIGR consecutive counters; a task that completes a residual row tile then arrives with its router
    partial, and the last row tile releases the next layer's expert-slot counters (each receives a routing
    value >= 1)."""
    if w[W_ARR] >= 0:
        ctr[w[W_ARR]] += 1
        if ctr[w[W_ARR]] != w[W_ARRN]:
            return
    if w[W_SIG] >= 0:
        ctr[w[W_SIG]:w[W_SIG] + w[W_SIGR]] += w[W_SIGN]
    if w[W_ARR2] >= 0:
        ctr[w[W_ARR2]] += 1
        if ctr[w[W_ARR2]] == w[W_ARRN2]:
            ctr[w[W_RSIG]:w[W_RSIG] + w[W_RSIGR]] += 1


def phases_of(tasks):
    """The list's phases: maximal runs of one operation and layer, in list order."""
    phases = []
    for t in range(len(tasks)):
        key = (tasks[t, W_OP], tasks[t, W_LAYER])
        if not phases or phases[-1][0] != key:
            phases.append((key, []))
        phases[-1][1].append(t)
    return [p for _, p in phases]


def simulate(tasks, n_counters, n_workers, rng):
    """Every workgroup runs one task at a time and takes the next untaken task of the list (one pool, list
    order) when it has none.  Rounds visit the workgroups in random order; each takes its next task if it has
    none and runs its task if the waits are met.  A round that runs nothing while tasks remain is a deadlock.
    Returns final counters and completion counts."""
    ctr = np.zeros(n_counters, np.int64)
    done = np.zeros(len(tasks), np.int64)
    taken = 0
    cur = [None] * n_workers
    completed = 0

    def ready(t):
        w = tasks[t]
        for i in range(4):
            c, tgt = w[W_WAIT0 + 2 * i], w[W_WAIT0 + 2 * i + 1]
            if c >= 0 and ctr[c] < tgt:
                return False
        return True

    while completed < len(tasks):
        progressed = False
        for wk in rng.permutation(n_workers):
            if cur[wk] is None and taken < len(tasks):
                cur[wk] = taken
                taken += 1
            t = cur[wk]
            if t is None or not ready(t):
                continue
            cur[wk] = None
            done[t] += 1
            completed += 1
            complete(tasks[t], ctr)
            progressed = True
        assert progressed, f"deadlock: no workgroup can run its current task ({completed} of {len(tasks)} done)"
    return ctr, done


def in_order(tasks, n_counters):
    """Counter values after every task has completed once, in list order."""
    ctr = np.zeros(n_counters, np.int64)
    for w in tasks:
        complete(w, ctr)
    return ctr


def check_device_counters(got, tasks, n_counters, lay, grid, vocab, slot_values, n_slots):
    """The device's final counters of a step (MK_DBGK_COUNTERS) against the plan, exactly:
    - every dependency, arrival and readiness counter equals its planned final value (the in-order
      simulation of the list), except that the up-projection counter of an unused expert slot stays 0 (its
      tiles signal nothing); a row tile's residual counter still ends at Hkv + n_slots (the routing
      workgroup arrives for the unused slots);
    - expert-slot counters hold their slot's routing (expert + 1 in bits 0..15, token mask in bits 16..23;
      an unused slot 0x80000000), `slot_values` computed from the slot table, and each layer's used-slot
      counter the number of used slots;
    - the ticket (the one pool the workgroups take the list from) ends at (tasks + grid): it passes every
      task once, by a take or by the move past an expert phase's unused tail, and then each workgroup's
      last take finds the list's end;
    - the kernel's exit counter and the LM head's arrival counter equal the grid; the LM head's chunk pool was
      claimed at least once per vocabulary chunk."""
    got = np.asarray(got, np.int64)
    exp = in_order(tasks, n_counters)
    s0, ns = lay["slot_ready"]
    exp[s0:s0 + ns] = slot_values
    L = ns // n_slots
    used = np.asarray(slot_values).reshape(L, n_slots) != UNUSED_SLOT
    u0, _ = lay["slots_used"]
    exp[u0:u0 + L] = used.sum(1)
    d0, _ = lay["up_done"]
    exp[d0:d0 + L * n_slots][~used.ravel()] = 0
    exp[lay["ticket"][0]] = len(tasks) + grid
    exp[lay["done"][0]] = grid
    exp[lay["lm_arrive"][0]] = grid
    lm = lay["lm_pool"][0]
    nch = -(-vocab // 128)
    assert nch <= got[lm] <= nch + 4 * grid, f"LM head chunk pool claimed {got[lm]} times for {nch} chunks"
    exp[lm] = got[lm]
    bad = np.nonzero(got[:n_counters] != exp)[0]
    assert len(bad) == 0, f"counters differ from the plan at {bad[:8].tolist()}: device {got[bad[:8]].tolist()} plan {exp[bad[:8]].tolist()}"


def tasks_ran(done, tasks, slot_values, n_slots):
    """Completion counts of a step: every task once, except the expert tiles of unused slots, which run at most
    once (a workgroup that took one before its layer was routed runs it as an empty task)."""
    done = np.asarray(done)
    unused = np.zeros(len(tasks), bool)
    sv = np.asarray(slot_values).reshape(-1, n_slots)
    moe = (tasks[:, W_OP] == OP_UP) | (tasks[:, W_OP] == OP_DOWN)
    unused[moe] = sv[tasks[moe, W_LAYER], tasks[moe, W_A]] == UNUSED_SLOT
    assert np.all(done[~unused] == 1), f"tasks not run exactly once: {np.nonzero((done != 1) & ~unused)[0][:10]}"
    assert np.all(done[unused] <= 1), "an unused slot's tile ran twice"
