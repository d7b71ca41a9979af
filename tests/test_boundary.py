"""Host-side checks of the C-ABI library: it loads, exports every declared entry point, validates shapes,
and its task lists are deadlock-free topological orders (CPU simulation of the counter protocol)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from decode_megakernel_wg_amd import mk
from synth import workloads as W
from taskgraph import (OP_ATTN, OP_EMBED, OP_MERGE, W_ARR, W_C, W_D, W_LAYER, W_OP, W_R0, W_R1, W_SIG, W_WAIT0, complete, counter_layout,
                       phases_of, simulate)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


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


@pytest.mark.parametrize("name,B_lens", [("tiny", [128]), ("tiny", [5, 300, 17, 0]), ("tiny", [16384]), ("full", [8192]),
                                         ("full", [65536]),
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
        # every interleaving ends every counter at its planned value, and every wait's target is exactly
        # that final value (a consumer waits for all of its producers)
        assert np.array_equal(ctr, sim)
        for w in tasks:
            for i in range(4):
                c, tgt = w[W_WAIT0 + 2 * i], w[W_WAIT0 + 2 * i + 1]
                if c >= 0:
                    assert ctr[c] == tgt, f"counter {c} ends at {ctr[c]}, a wait targets {tgt}"


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
    # the LM head, the router and the residual add are not tasks
    assert set(np.unique(tasks[:, W_OP]).tolist()) == {1, 3, 4, 5, 6, 7}
    # about 96 splits per layer: 8192 cached positions x 4 KV groups / 96 = 341 -> 384 positions (3 chunks of
    # 128) per split, 22 splits per KV group; the last split of each (sequence, group) takes the rest (128
    # cached positions) and the new token
    assert ops[OP_ATTN] == 48 * 4 * 22
    attn = tasks[tasks[:, W_OP] == 4]
    assert (attn[:, W_R0] == 384).all() and (attn[:, W_D] == 22).all()
    # long contexts: about 192 splits per layer (ctx x 4 / 192 positions rounded to 128), about 224 from 2048
    # positions per split on, at most 4096 positions each
    for ctx, pos in ((65536, 1408), (131072, 2304), (262144, 4096)):
        dl = desc_for(W.FULL, B=1, pages=ctx // 16 + 64, n_pages=ctx // 16 + 64)
        tl, _ = mk.mk_plan_tasks(dl, [ctx])
        al = tl[(tl[:, W_OP] == 4) & (tl[:, 1] == 0)]
        assert (al[:, W_R0] == pos).all() and len(al) == 4 * -(-ctx // pos)
    # merge tasks from 33 splits of one sequence on (long contexts): one per head of each (sequence, KV group), after
    # the up-projection tiles; the splits then only count themselves, and each O-projection tile waits for its
    # group's eight merges
    assert ops[8] == 0
    for ctx in (65536, 131072, 262144):
        dl = desc_for(W.FULL, B=1, pages=ctx // 16 + 64, n_pages=ctx // 16 + 64)
        tl, _ = mk.mk_plan_tasks(dl, [ctx])
        m0 = tl[(tl[:, W_OP] == 8) & (tl[:, 1] == 0)]
        a0 = tl[(tl[:, W_OP] == 4) & (tl[:, 1] == 0)]
        ns = len(a0) // 4
        assert len(m0) == 32 and sorted(m0[:, W_C].tolist()) == sorted(list(range(8)) * 4)
        assert (m0[:, W_R0] == 1).all() and (m0[:, W_D] == ns).all() and (a0[:, W_ARR] == -1).all()
        assert (ctx, ns) in ((65536, 47), (131072, 57), (262144, 64))
        o0 = tl[(tl[:, W_OP] == 6) & (tl[:, 1] == 0)]
        assert (o0[:, W_WAIT0 + 1] == 8).all()
        runs = [int(tl[r[0], W_OP]) for r in phases_of(tl)[1:7]]
        assert runs == [3, 4, 5, 8, 6, 7]
    # expert up-projection tiles: 48 gate + 48 up rows at batches of 1-2 (16 tiles per expert), 64 + 64 above
    up = tasks[tasks[:, W_OP] == 5]
    assert ops[5] == 48 * 8 * 16 and ((up[:, W_R1] - up[:, W_R0]) == 48).all()
    d8 = desc_for(W.FULL, B=8, pages=600 * 8, n_pages=600 * 8)
    t8, _ = mk.mk_plan_tasks(d8, [8192] * 8)
    up8 = t8[t8[:, W_OP] == 5]
    assert ((up8[:, W_R1] - up8[:, W_R0]) == 64).all() and len(up8) == 48 * 64 * 12


@pytest.mark.parametrize("name,B_lens", [("tiny", [128]), ("tiny", [5, 300, 17, 0]), ("tiny", [16384]), ("full", [8192]),
                                         ("full", [65536]),
                                         ("full", [1024, 30000, 4000, 70000, 2000, 9000, 1500, 12000])])
def test_task_list_has_the_regular_phase_structure(name, B_lens):
    """The kernel classifies its takes by the list's phase table (and passes over the expert tiles of unused
    slots) only when the list is the embedding tiles followed, layer by layer, by the same sequence of
    operation runs with the same sizes (otherwise it runs those tiles as empty tasks): every planned list
    must have that structure."""
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


@pytest.mark.parametrize("shape,lens", [(W.TINY, [128]), (W.TINY, [5, 300, 17, 0]), (W.TINY, [16384]), (W.FULL, [8192]),
                                        (W.FULL, [100] * 8)])
def test_counter_layout_mirror(shape, lens):
    """The tests' copy of the counter layout gives the library's counter count, and every counter a descriptor
    names lies in the block its role belongs to."""
    maxp = max(lens) // 16 + 2
    d = desc_for(shape, B=len(lens), pages=maxp, n_pages=maxp * len(lens))
    tasks, n_ctr = mk.mk_plan_tasks(d, lens)
    B, L = len(lens), shape.n_layers
    n_slots = min(shape.n_experts, B * shape.top_k)
    n_rt = shape.d_model // (128 if shape.d_model >= 1024 else 32)
    lay = counter_layout(L, shape.n_kv_heads, B, n_slots, n_rt)
    assert lay["total"] == n_ctr

    def inside(c, block):
        o, n = lay[block]
        return o <= c < o + n

    for w in tasks:
        op = w[W_OP]
        if op == 3:
            assert inside(w[W_WAIT0], "xready") and inside(w[W_SIG], "qkv_done")
        if op == OP_ATTN and w[W_ARR] >= 0:
            assert inside(w[W_WAIT0], "qkv_done") and inside(w[W_ARR], "attn_arrive") and inside(w[W_SIG], "attn_done")
        if op == OP_ATTN and w[W_ARR] < 0:  # merged by merge tasks: the split only counts itself
            assert inside(w[W_WAIT0], "qkv_done") and inside(w[W_SIG], "attn_arrive")
        if op == OP_MERGE:
            assert inside(w[W_WAIT0], "attn_arrive") and inside(w[W_SIG], "attn_done")
        if op == 6:
            assert inside(w[W_WAIT0], "attn_done")
        if op == 5:
            assert inside(w[W_WAIT0], "slot_ready") and inside(w[W_SIG], "up_done")
        if op in (6, 7):
            assert inside(w[W_ARR], "resid_arrive") and inside(w[W_SIG], "xready")


def test_chunk_map_validation_and_planning():
    """first_of: entries of a chunk are consecutive, in position order, and its attention splits cover only the
    cached prefix below the chunk's first position."""
    d = desc_for(W.TINY, B=8, pages=64, n_pages=512)
    lens = [300, 301, 302, 303, 40, 41, 7, 500]
    first = [0, 0, 0, 0, 4, 4, 6, 7]
    tasks, _ = mk.mk_plan_tasks(d, lens, first)
    plain, _ = mk.mk_plan_tasks(d, [300, 300, 300, 300, 40, 40, 7, 500])
    # the splits depend only on the cached lengths: a chunk plans like its first entry repeated
    assert np.array_equal(tasks, plain)
    for bad_first, bad_lens in (([0, 0, 1, 3, 4, 4, 6, 7], lens),        # an entry whose first is not a chunk head
                                ([0, 1, 0, 3, 4, 4, 6, 7], lens),        # a chunk interrupted by another sequence
                                ([1, 1, 2, 3, 4, 4, 6, 7], lens),        # first after the entry
                                ([0, 0, 0, 0, 4, 4, 6, 7], [300, 301, 303, 303, 40, 41, 7, 500]),  # positions not consecutive
                                ([0, 0, 0, 0, 4, 4, 4, 7], lens)):       # an entry's position outside its chunk's run
        with pytest.raises(mk.MkError) as e:
            mk.mk_plan_tasks(d, bad_lens, bad_first)
        assert e.value.code == mk.MK_E_INVAL
    # prefill from an empty context: one split per entry, covering no cached position
    t0, _ = mk.mk_plan_tasks(d, list(range(8)), [0] * 8)
    attn = t0[t0[:, W_OP] == OP_ATTN]
    assert (attn[:, W_D] == 1).all()
