"""Bit-exact checks of the integer work of a decode step, from the kernel's own debug records.

After a step (read through the C ABI's debug kinds):
 - routing: each (layer, token)'s selection is exactly the top-k of the GPU's own router logits, ordered by
   (logit descending, index ascending), NaN ranking lowest; its gates are the softmax of those selected
   logits (fp32 rounding); the slot table holds exactly the distinct selected experts in ascending id, each
   with its tokens in ascending order, their ranks and bit-identical gates, and unused slots are empty;
 - page walks (MK_DBG_PAGE_WALK): every (layer, entry, KV group) read the pages of the cached positions
   below its chunk's first position, in logical order, once each (count and checksum of a brute-force walk
   of the page table), attended to every position up to its own, and wrote its K/V to the slot of its own
   position;
 - task graph: every task ran exactly once (an unused expert slot's tiles at most once) and every counter
   ended at its planned value (taskgraph).
"""
from __future__ import annotations

import numpy as np

from taskgraph import UNUSED_SLOT, check_device_counters, counter_layout, tasks_ran


def topk_exact(logits, k):
    key = np.where(np.isnan(logits), -np.inf, logits).astype(np.float64)
    order = np.lexsort((np.arange(len(key)), -key))
    return order[:k]


def check_routing(h, shape, B):
    from decode_megakernel_wg_amd import mk

    L, k, E = shape.n_layers, shape.top_k, shape.n_experts
    rl = h.mk_debug_read(mk.MK_DBGK_ROUTER_LOGITS, (L, B, E), np.float32)
    sel = h.mk_debug_read(mk.MK_DBGK_ROUTE_SEL, (L, B, k), np.int32)
    gate = h.mk_debug_read(mk.MK_DBGK_ROUTE_GATE, (L, B, k), np.float32)
    n_slots = min(E, B * k)
    slots = h.mk_debug_read(mk.MK_DBGK_SLOTS, (L, n_slots, 32), np.int32)
    slot_values = np.zeros(L * n_slots, np.int64)
    for l in range(L):
        for b in range(B):
            want = topk_exact(rl[l, b], k)
            assert np.array_equal(sel[l, b], want), f"layer {l} token {b}: selection {sel[l, b]} is not the top-k {want} of its logits"
            z = rl[l, b, want].astype(np.float64)
            g = np.exp(z - z.max())
            assert np.allclose(gate[l, b], g / g.sum(), rtol=2e-6, atol=1e-7), f"layer {l} token {b}: gates"
        experts = sorted(set(int(e) for e in sel[l].ravel()))
        for s in range(n_slots):
            ent = slots[l, s]
            if s >= len(experts):
                assert ent[0] == -1 and ent[1] == 0, f"layer {l} slot {s} should be unused: {ent[:4]}"
                slot_values[l * n_slots + s] = UNUSED_SLOT
                continue
            e = experts[s]
            toks = [(b, j) for b in range(B) for j in range(k) if sel[l, b, j] == e]
            assert ent[0] == e and ent[1] == len(toks), f"layer {l} slot {s}: expert {ent[0]} x{ent[1]}, want {e} x{len(toks)}"
            mask = 0
            for i, (b, j) in enumerate(toks):
                assert ent[2 + 3 * i] == b and ent[3 + 3 * i] == j, f"layer {l} slot {s} entry {i}"
                assert ent[4 + 3 * i] == gate[l, b, j:j + 1].view(np.int32)[0], f"layer {l} slot {s} entry {i}: gate bits"
                mask |= 1 << b
            slot_values[l * n_slots + s] = (mask << 16) | (e + 1)
    return slot_values


def check_page_walks(h, shape, pt, lens, first_of=None):
    """pt: the step's page-table rows [B][max_pages]; lens: the step's seq_lens."""
    from decode_megakernel_wg_amd import mk

    B = len(lens)
    L, Hkv = shape.n_layers, shape.n_kv_heads
    rec = h.mk_debug_read(mk.MK_DBGK_PAGE_WALK, (L, B, Hkv, 4), np.uint32)
    for b in range(B):
        f = b if first_of is None else int(first_of[b])
        len0, ln = int(lens[f]), int(lens[b])
        n = -(-len0 // 16)
        cs = int(sum((j + 1) * int(pt[b][j]) for j in range(n)) % (1 << 32))
        want = np.array([n, cs, ln + 1, 1 + int(pt[b][ln // 16]) * 16 + ln % 16], np.uint32)
        for l in range(L):
            for g in range(Hkv):
                assert np.array_equal(rec[l, b, g], want), f"layer {l} entry {b} KV group {g}: walk {rec[l, b, g]} want {want}"


def check_task_graph(h, shape, desc, lens, grid, slot_values, first_of=None, tasks=None):
    """lens / first_of: those the handle's task list was built with (a list stays valid while lengths grow);
    tasks: the handle's own list when it was planned with a debug switch that changes it (default: the list
    mk_plan_tasks gives for lens)."""
    from decode_megakernel_wg_amd import mk

    planned, n_ctr = mk.mk_plan_tasks(desc, lens, first_of)
    tasks = planned if tasks is None else tasks
    B = len(lens)
    n_slots = min(shape.n_experts, B * shape.top_k)
    done = h.mk_debug_read(mk.MK_DBGK_TASK_DONE, (len(tasks),), np.uint32)
    tasks_ran(done, tasks, slot_values, n_slots)
    n_rt = shape.d_model // (128 if shape.d_model >= 1024 else 32)
    lay = counter_layout(shape.n_layers, shape.n_kv_heads, B, n_slots, n_rt)
    got = h.mk_debug_read(mk.MK_DBGK_COUNTERS, (n_ctr,), np.uint32)
    check_device_counters(got, tasks, n_ctr, lay, grid, shape.vocab, slot_values, n_slots)


def device_grid():
    import torch

    return min(torch.cuda.get_device_properties(0).multi_processor_count, 1024)


def check_step(h, shape, desc, pt, lens, grid=None, first_of=None, walks=True, plan_lens=None, tasks=None):
    """All of the above for the step just run (the handle must have MK_DBG_PAGE_WALK set when walks);
    plan_lens: the lengths the task list was built with (default: this step's); tasks: the handle's list
    (check_task_graph)."""
    B = len(lens)
    slot_values = check_routing(h, shape, B)
    if walks:
        check_page_walks(h, shape, pt, lens, first_of)
    check_task_graph(h, shape, desc, lens if plan_lens is None else plan_lens, device_grid() if grid is None else grid, slot_values,
                     first_of, tasks)


KV_DRIFT_FIRST = 1e-5
KV_DRIFT_DEEP = 1e-3


def kv_layers_close(g, o, what=""):
    """Whole caches or per-layer slices [L][...][dh]: layer 0 at KV_DRIFT_FIRST, the others at KV_DRIFT_DEEP."""
    for l in range(g.shape[0]):
        r = kv_close(g[l], o[l], KV_DRIFT_FIRST if l == 0 else KV_DRIFT_DEEP)
        assert r <= 1.0, f"{what} layer {l}: K/V differ from the oracle's beyond one BF16 step + drift (ratio {r:.3g})"


def bf16_step(x):
    """Spacing of BF16 values at |x| (one rounding step): 2^(e - 7) for |x| in [2^e, 2^(e+1))."""
    a = np.abs(np.asarray(x, np.float32))
    e = np.floor(np.log2(np.where(a > 0, a, np.float32(2.0 ** -126))))
    return np.exp2(e - 7).astype(np.float32)


def kv_close(g, o, drift):
    """K/V head vectors (last axis) g from the GPU and o from the oracle, both BF16 values as fp32: every element
    within one BF16 rounding step of the oracle's plus drift times the head vector's RMS.  The two sides round
    fp32 values that agree to ~1e-6 of the vector in the first layer (KV_DRIFT_FIRST); deeper layers' inputs
    already carry the residual stream's drift, which a context of a few positions (no averaging in the
    attention) can raise to a few 1e-4 (KV_DRIFT_DEEP).  Returns the worst ratio of difference to bound
    (<= 1 passes)."""
    g = np.asarray(g, np.float32)
    o = np.asarray(o, np.float32)
    rms = np.sqrt(np.mean(o.astype(np.float64) ** 2, axis=-1, keepdims=True))
    bound = bf16_step(o) + drift * rms + 1e-30
    return float(np.max(np.abs(g.astype(np.float64) - o) / bound))
