"""Host-side checks of the C-ABI library: it loads, exports every declared entry point, validates shapes,
and its task lists are deadlock-free topological orders (CPU simulation of the counter protocol)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from decode_megakernel_wg_amd import mk
from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# descriptor words (mirrors the library's layout)
W_OP, W_LAYER, W_A, W_B, W_C, W_D, W_R0, W_R1, W_WAIT0, W_SIG, W_SIGN, W_ARR, W_ARRN, W_SIGR = 0, 1, 2, 3, 4, 5, 6, 7, 8, 16, 17, 18, 19, 20
W_ARR2, W_ARRN2, W_RSIG, W_RSIGR = 24, 25, 26, 27
OP_EMBED, OP_ATTN, OP_LMHEAD = 1, 4, 9


def declared(header):
    txt = open(os.path.join(ROOT, "include", header)).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b((?:mk|synth)_[a-z0-9_]+)\s*\(", txt)))


def test_libraries_load_and_export_every_declared_symbol():
    L = mk.lib()
    for name in declared("mk.h"):
        assert hasattr(L, name), name
    assert set(declared("mk.h")) == set(mk.EXPORTS)
    from synth import synth

    H = synth.host()
    D = C.CDLL(synth.DEV_LIB)
    for name in declared("synth.h"):
        assert hasattr(D if name.startswith("synth_dev_") else H, name), name


def desc_for(shape, B=1, pages=64, n_pages=1024, **over):
    d = mk.make_desc(shape, B, pages, n_pages)
    for k, v in over.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("field,value,code", [("d_head", 96, mk.MK_E_UNSUPPORTED), ("page_size", 32, mk.MK_E_UNSUPPORTED),
                                              ("max_batch", 9, mk.MK_E_UNSUPPORTED), ("n_q_heads", 6, mk.MK_E_UNSUPPORTED),
                                              ("abi_version", 99, mk.MK_E_INVAL), ("n_layers", 0, mk.MK_E_INVAL),
                                              ("top_k", 9, mk.MK_E_UNSUPPORTED)])
def test_shape_validation(field, value, code):
    d = desc_for(W.TINY, **{field: value})
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan_tasks(d, [10])
    assert e.value.code == code


def test_batch_validation():
    d = desc_for(W.TINY, B=2, pages=4)
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan_tasks(d, [1, 2, 3])
    assert e.value.code == mk.MK_E_INVAL
    with pytest.raises(mk.MkError):
        mk.mk_plan_tasks(d, [10, 64])   # 64 // 16 = 4 pages: beyond max_pages_per_seq
    with pytest.raises(mk.MkError):
        mk.mk_plan_tasks(d, [-1])


def phases_of(tasks):
    """The launcher's phases: maximal runs of one operation and layer, in list order."""
    phases = []
    for t in range(len(tasks)):
        key = (tasks[t, W_OP], tasks[t, W_LAYER])
        if not phases or phases[-1][0] != key:
            phases.append((key, []))
        phases[-1][1].append(t)
    return [p for _, p in phases]


def simulate(tasks, n_counters, n_workers, rng):
    """Every workgroup runs one task at a time.  One workgroup claims the list in order; two or more take
    tasks from the phase pools in order, one at a time, moving to the next phase once a take finds the pool
    empty.  Rounds visit the workgroups in random order; each picks its next task if it has none and runs
    its task if the waits are met.  A round that runs nothing while tasks remain is a deadlock.  Returns
    final counters and completion counts."""
    phases = phases_of(tasks) if n_workers >= 2 else [list(range(len(tasks)))]
    ctr = np.zeros(n_counters, np.int64)
    done = np.zeros(len(tasks), np.int64)
    taken = [0] * len(phases)
    cur = [None] * n_workers
    ph = [0] * n_workers
    completed = 0

    def ready(t):
        w = tasks[t]
        for i in range(4):
            c, tgt = w[W_WAIT0 + 2 * i], w[W_WAIT0 + 2 * i + 1]
            if c >= 0 and ctr[c] < tgt:
                return False
        return True

    def pick(wk):
        while ph[wk] < len(phases):
            p = ph[wk]
            if taken[p] < len(phases[p]):
                taken[p] += 1
                return phases[p][taken[p] - 1]
            ph[wk] += 1
        return None

    while completed < len(tasks):
        progressed = False
        for wk in rng.permutation(n_workers):
            if cur[wk] is None:
                cur[wk] = pick(wk)
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


@pytest.mark.parametrize("name,B_lens", [("tiny", [128]), ("tiny", [5, 300, 17, 0]), ("full", [8192]),
                                         ("full", [1024, 30000, 4000, 70000, 2000, 9000, 1500, 12000])])
def test_task_list_is_a_deadlock_free_topological_order(name, B_lens):
    shape = W.TINY if name == "tiny" else W.FULL
    maxp = max(B_lens) // 16 + 2
    d = desc_for(shape, B=len(B_lens), pages=maxp, n_pages=maxp * len(B_lens))
    tasks, n_ctr = mk.mk_plan_tasks(d, B_lens)
    assert tasks.shape[1] == mk.MK_DESC_WORDS
    assert np.array_equal(tasks[:, 31], np.arange(len(tasks)))
    # every wait is reachable from earlier tasks only
    sim = np.zeros(n_ctr, np.int64)
    for t, w in enumerate(tasks):
        for i in range(4):
            c, tgt = w[W_WAIT0 + 2 * i], w[W_WAIT0 + 2 * i + 1]
            if c >= 0:
                assert sim[c] >= tgt, f"task {t} waits on counter {c} beyond earlier signals"
        complete(w, sim)
    rng = np.random.default_rng(0)
    for workers in (1, 2, 3, 256):
        if name == "full" and workers != 256 and len(B_lens) > 1:
            continue
        ctr, done = simulate(tasks, n_ctr, workers, rng)
        assert np.all(done == 1)
        for w in tasks:
            for i in range(4):
                c, tgt = w[W_WAIT0 + 2 * i], w[W_WAIT0 + 2 * i + 1]
                if c >= 0:
                    assert ctr[c] == tgt or ctr[c] >= tgt


def test_dropped_producer_is_detected_by_the_simulator():
    d = desc_for(W.TINY, B=1, pages=16)
    tasks, n_ctr = mk.mk_plan_tasks(d, [100])
    t = tasks.copy()
    first = int(np.nonzero(t[:, W_OP] == 6)[0][0])
    t[first, W_ARR] = t[first, W_SIG] = -1   # an O-projection tile that never arrives
    with pytest.raises(AssertionError, match="deadlock"):
        simulate(t, n_ctr, 4, np.random.default_rng(1))


def test_task_counts_full_model():
    d = desc_for(W.FULL, B=1, pages=600, n_pages=600)
    tasks, _ = mk.mk_plan_tasks(d, [8192])
    ops = np.bincount(tasks[:, W_OP], minlength=10)
    assert ops[OP_LMHEAD] == 0   # the LM head is the kernel's closing phase, not tasks
    # about 96 splits per layer: 8192 cached positions x 4 KV groups / 96 = 341 -> 384 positions (3 chunks of
    # 128) per split, 22 splits per KV group; the last split of each (sequence, group) takes the rest (128
    # cached positions) and the new token
    assert ops[OP_ATTN] == 48 * 4 * 22
    attn = tasks[tasks[:, W_OP] == 4]
    assert (attn[:, W_R0] == 384).all() and (attn[:, W_D] == 22).all()
    # long contexts: about 192 splits per layer (ctx x 4 / 192 positions rounded to 128), at most 4096 each
    for ctx, pos in ((65536, 1408), (131072, 2688), (262144, 4096)):
        dl = desc_for(W.FULL, B=1, pages=ctx // 16 + 64, n_pages=ctx // 16 + 64)
        tl, _ = mk.mk_plan_tasks(dl, [ctx])
        al = tl[(tl[:, W_OP] == 4) & (tl[:, 1] == 0)]
        assert (al[:, W_R0] == pos).all() and len(al) == 4 * -(-ctx // pos)
    # expert up-projection tiles: 48 gate + 48 up rows at batches of 1-2 (16 tiles per expert), 64 + 64 above
    up = tasks[tasks[:, W_OP] == 5]
    assert ops[5] == 48 * 8 * 16 and ((up[:, W_R1] - up[:, W_R0]) == 48).all()
    d8 = desc_for(W.FULL, B=8, pages=600 * 8, n_pages=600 * 8)
    t8, _ = mk.mk_plan_tasks(d8, [8192] * 8)
    up8 = t8[t8[:, W_OP] == 5]
    assert ((up8[:, W_R1] - up8[:, W_R0]) == 64).all() and len(up8) == 48 * 64 * 12


@pytest.mark.parametrize("name,B_lens", [("tiny", [128]), ("tiny", [5, 300, 17, 0]), ("full", [8192]),
                                         ("full", [1024, 30000, 4000, 70000, 2000, 9000, 1500, 12000])])
def test_task_list_has_the_regular_phase_structure(name, B_lens):
    """The launcher runs the list as phases only when it is the embedding tiles followed, layer by layer, by
    the same sequence of operation runs with the same sizes (otherwise it falls back to in-order claims):
    every planned list must have that structure."""
    shape = W.TINY if name == "tiny" else W.FULL
    maxp = max(B_lens) // 16 + 2
    d = desc_for(shape, B=len(B_lens), pages=maxp, n_pages=maxp * len(B_lens))
    tasks, _ = mk.mk_plan_tasks(d, B_lens)
    runs = phases_of(tasks)
    assert all(tasks[t, W_OP] == OP_EMBED for t in runs[0])
    L = shape.n_layers
    assert (len(runs) - 1) % L == 0
    npl = (len(runs) - 1) // L
    assert 1 <= npl <= 7
    first = [(int(tasks[r[0], W_OP]), len(r)) for r in runs[1:1 + npl]]
    for l in range(L):
        layer_runs = runs[1 + l * npl:1 + (l + 1) * npl]
        assert [(int(tasks[r[0], W_OP]), len(r)) for r in layer_runs] == first
        assert all(int(tasks[t, W_LAYER]) == l for r in layer_runs for t in r)
