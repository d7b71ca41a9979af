"""Continuous-batching schedule (host logic, no GPU): arrival process, FIFO admission, page free list.

The schedule is input generation shared by both sides; these checks pin it to its stated rules
(arrivals exponential with mean 64 steps rounded up, outputs geometric with p = 1/256 on {1, 2, ...},
prefixes log-uniform in [512, 65536], at most 8 live, FIFO admission, LIFO page reuse, idle jumps).
"""
import math

import numpy as np

from synth import continuous as CB

STEPS = 1024


def _sched():
    return CB.schedule(STEPS)


def test_deterministic():
    a, sa, na, ma = _sched()
    b, sb, nb, mb = _sched()
    assert (na, ma) == (nb, mb)
    for x, y in zip(a, b):
        assert x.sids == y.sids and np.array_equal(x.pos, y.pos) and x.admitted == y.admitted and x.finished == y.finished


def test_draw_statistics():
    n = 20000
    arrive, prefix, out_len = CB.draws(n)
    gaps = np.diff(arrive)
    assert gaps.min() >= 1
    # ceil(Exp(64)) has mean 64 + ~0.5
    assert abs(gaps.mean() - 64.5) < 0.05 * 64
    assert out_len.min() >= 1
    assert abs(out_len.mean() - 256) < 0.05 * 256
    # geometric tail: P(L > 256) = (1 - p)^256
    assert abs((out_len > 256).mean() - (1 - CB.P_END) ** 256) < 0.02
    lo, hi = CB.PREFIX_LO, CB.PREFIX_HI
    assert prefix.min() >= lo and prefix.max() <= hi
    assert abs(prefix.mean() - (hi - lo) / math.log(hi / lo)) < 0.05 * (hi - lo) / math.log(hi / lo)
    # log-uniform: the median is the geometric mean of the bounds
    assert abs(math.log(np.median(prefix)) - 0.5 * math.log(lo * hi)) < 0.1


def test_batches_positions_and_lifetimes():
    steps, seqs, n_pages, max_pages = _sched()
    seen_first, count = {}, {}
    prev = None
    for t, st in enumerate(steps):
        B = len(st.sids)
        assert 1 <= B <= CB.MAX_BATCH and len(set(st.sids)) == B
        for b, sid in enumerate(st.sids):
            q = seqs[sid]
            assert q.arrive <= st.clock, "admitted before its arrival"
            if sid not in seen_first:
                seen_first[sid] = t
                assert sid in st.admitted and int(st.pos[b]) == q.prefix
            count[sid] = count.get(sid, 0) + 1
            assert int(st.pos[b]) == q.prefix + (t - seen_first[sid])
            assert -(-(int(st.pos[b]) + 1) // 16) <= len(q.pages) <= max_pages
        # admission order: admitted sequences join at the end, in arrival (= id) order
        assert st.sids[B - len(st.admitted):] == st.admitted and st.admitted == sorted(st.admitted)
        if prev is not None:
            cont = [s for s in prev.sids if s not in prev.finished]
            assert st.sids[:len(cont)] == cont
        prev = st
    for sid, n in count.items():
        q = seqs[sid]
        if q.last_step >= 0:
            assert n == q.out_len
    # FIFO: sequences are admitted in arrival order
    adm = [s.sid for s in sorted((s for s in seqs if s.admitted_step >= 0), key=lambda s: s.admitted_step)]
    assert adm == sorted(adm)
    mean_live = np.mean([len(st.sids) for st in steps])
    assert 1.5 < mean_live < 6.0  # offered load 256 / 64 = 4 (fewer at the start)


def test_pages_disjoint_and_lifo():
    steps, seqs, n_pages, _ = _sched()
    for st in steps:
        used = [p for sid in st.sids for p in seqs[sid].pages]
        assert len(used) == len(set(used)) and min(used) >= 0 and max(used) < n_pages
    for q in seqs:
        if q.admitted_step >= 0:
            assert len(q.pages) == CB.pages_for(q.prefix, q.out_len)
    # the first admission takes pages 0, 1, 2, ... in order
    q0 = seqs[0]
    assert q0.pages == list(range(len(q0.pages)))
    # LIFO reuse: the first sequence admitted after a release with no admission in between starts with the
    # first page of the last sequence released (pages go back in reverse, so they come out in order)
    checked, last_freed = 0, None
    for st in steps:
        if st.admitted and last_freed is not None:
            assert seqs[st.admitted[0]].pages[0] == seqs[last_freed].pages[0]
            checked += 1
        if st.admitted:
            last_freed = None
        if st.finished:
            last_freed = st.finished[-1]
    assert checked >= 1


def test_idle_jump():
    # with a tiny pool of decode steps the clock still advances one per step while anything is live
    steps, seqs, _, _ = _sched()
    for a, b in zip(steps, steps[1:]):
        assert b.clock > a.clock
        if b.clock > a.clock + 1:  # an idle jump: nothing was live after a, and b admits the next arrival
            assert set(a.sids) == set(a.finished) and b.admitted and seqs[b.admitted[0]].arrive == b.clock
