"""GPU parity at the full model size, in the launch configuration the benchmark times (one workgroup per
compute unit, phase pools; the debug records read here do not change the schedule).

The 48-layer synthetic model (d_model 2048, 32 q / 4 KV heads x 128, 128 experts top-8, d_ffn 768, vocab
262144) runs consecutive greedy decode steps per workload; the oracle (fp64-accumulating C, weights
generated per layer on the host from the same seeded generator) runs the same steps, teacher-forced with the
GPU's tokens.  Bar, every step and sequence: logits relative L2 <= 1e-2; greedy tokens equal unless the
oracle's top-2 gap is below 1e-2, with >= 99 % agreement; routing identical except at oracle near-ties
(follow mode, at most 1 % of the routings); integer work bit-exact (selection = top-k of the GPU's own
logits, slot table, page walks, every task once, every counter at its planned value); the new K/V written
equal to the oracle's up to BF16 rounding (every element within one BF16 step plus 1e-5 of its head vector's
RMS in layer 0, plus 1e-3 of it in the deeper layers, whose inputs already differ slightly).  Long contexts run one oracle step with each
layer's cache generated when the layer runs.  The d_head-128 attention's results do not depend on the grid
or on where the pages of the cache lie (bit for bit).
"""
import numpy as np
import pytest
import torch

from gpu_checks import KV_DRIFT_DEEP, KV_DRIFT_FIRST, check_step, kv_close
from oracle_runner import OracleRun, rel_l2, top2_gap
from synth import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("cuda")]

LOGIT_TOL = 1e-2
TOKEN_GAP = 1e-2


def _gpu_kv_at(sess, l, b, pos):
    """K and V (fp32) the GPU cache holds for sequence b at position pos of layer l: [2][Hkv][dh]."""
    from oracle import oracle as O

    page = int(sess.kvc.pt_host[b, pos // 16])
    kv = sess.kvc.kv[l, page, :, :, pos % 16, :].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return O.bf16_to_f32(kv)


def _oracle_kv_at(orc, l, b, pos):
    from oracle import oracle as O

    page = int(orc.pt[b, pos // 16])
    kvl = orc.kept[l] if orc.lazy_kv else orc.kv[l]
    return O.bf16_to_f32(kvl[page, :, :, pos % 16, :])


def _compare_step(sess, orc, w, step, tokens, layers_kv):
    from decode_megakernel_wg_amd import mk

    s = w.shape
    logits = sess.logits.cpu().numpy()
    nxt = sess.next_tokens()
    check_step(sess.h, s, sess.desc, sess.kvc.pt_host, sess.seq_rows_host[step], plan_lens=sess.seq_rows_host[0])
    gsel = sess.h.mk_debug_read(mk.MK_DBGK_ROUTE_SEL, (s.n_layers, w.B, s.top_k), np.int32)
    pos = sess.seq_rows_host[step]
    ol, onx, _, _ = orc.step(tokens, pos, gpu_sel=gsel)
    agree, worst = 0, 0.0
    for b in range(w.B):
        e = rel_l2(logits[b], ol[b])
        worst = max(worst, e)
        assert e <= LOGIT_TOL, f"{w.name} step {step} seq {b}: logits rel L2 {e:.3e}"
        if nxt[b] == onx[b]:
            agree += 1
        else:
            assert top2_gap(ol[b]) < TOKEN_GAP, f"{w.name} step {step} seq {b}: token {nxt[b]} vs oracle {onx[b]}"
        assert nxt[b] == int(np.argmax(logits[b]))
    for l in layers_kv:
        for b in range(w.B):
            g, o = _gpu_kv_at(sess, l, b, int(pos[b])), _oracle_kv_at(orc, l, b, int(pos[b]))
            r = kv_close(g, o, KV_DRIFT_FIRST if l == 0 else KV_DRIFT_DEEP)
            assert r <= 1.0, f"{w.name} layer {l} seq {b}: new K/V beyond one BF16 step + drift (ratio {r:.3g})"
    return [int(t) for t in nxt], agree, worst


def _teacher_forced_router(sess, w):
    """The oracle's router applied to the GPU's own normalised inputs gives the GPU's router logits (all
    layers; the GPU's selection is then the exact top-k of those, checked by check_step)."""
    from decode_megakernel_wg_amd import mk
    from oracle import oracle as O

    s = w.shape
    n_gpu = sess.h.mk_debug_read(mk.MK_DBGK_NORM_IN, (s.n_layers, w.B, s.d_model), np.float32)
    rl = sess.h.mk_debug_read(mk.MK_DBGK_ROUTER_LOGITS, (s.n_layers, w.B, s.n_experts), np.float32)
    for l in range(s.n_layers):
        wr = W.host_matrix(7, l, s.n_experts, s.d_model)
        for b in range(w.B):
            _, _, lg = O.router(n_gpu[l, b], wr, s.top_k, w.router_bias)
            assert np.allclose(lg, rl[l, b], rtol=1e-5, atol=1e-6), f"{w.name}: router logits differ at layer {l} seq {b}"


def _run(name, steps, teacher_forced_step=None, lazy=False, extra_flags=0):
    from decode_megakernel_wg_amd import mk
    from decode_megakernel_wg_amd.session import Session

    w = W.make(name, steps=steps)
    pt, n_pages = W.page_tables(w)
    sess = Session(w, pt=pt, n_pages=n_pages)
    L = w.shape.n_layers
    layers_kv = (0, L // 2, L - 1)
    orc = OracleRun(w, pt, n_pages, keep_all=False, lazy_kv=lazy, keep_kv_layers=layers_kv)
    tokens = list(w.tokens)
    agree, worst = 0, 0.0
    for step in range(steps):
        flags = mk.MK_DBG_PAGE_WALK | mk.MK_DBG_COUNT_TASKS | extra_flags | (mk.MK_DBG_DUMP_N if step == teacher_forced_step else 0)
        sess.h.mk_debug_set(flags)
        sess.step()
        sess.status()
        if step == teacher_forced_step:
            _teacher_forced_router(sess, w)
        tokens, a, e = _compare_step(sess, orc, w, step, tokens, layers_kv)
        agree += a
        worst = max(worst, e)
        print(f"{name} step {step}: logits rel L2 {e:.2e}", flush=True)
    assert agree >= 0.99 * steps * w.B
    assert orc.near_ties <= max(1, 0.01 * orc.route_checked), f"{orc.near_ties} routing near-ties in {orc.route_checked}"
    print(f"{name}: {steps} steps, worst logits rel L2 {worst:.2e}, oracle follow-mode near-ties {orc.near_ties}/{orc.route_checked}")


@pytest.mark.timeout(900)
def test_full_b1_8k():
    _run("b1_8k", steps=16, teacher_forced_step=1)


@pytest.mark.timeout(600)
def test_full_b1_8k_valu_gemv():
    """The VALU engine of the GEMV tiles at batch 1 (MK_DBG_VALU_GEMV), same bar."""
    from decode_megakernel_wg_amd import mk

    _run("b1_8k", steps=2, teacher_forced_step=0, extra_flags=mk.MK_DBG_VALU_GEMV)


@pytest.mark.timeout(600)
def test_full_tp2_shard_b1_8k():
    """One GPU's share of the model under 2-way tensor parallelism (16 q / 2 KV heads, d_ffn 384, vocab 131072):
    the same kernel classes at the shard's shape, same bar."""
    _run("tp2_b1_8k", steps=4, teacher_forced_step=0)


@pytest.mark.timeout(600)
def test_full_b1_8k_gains():
    """Non-unit RMSNorm gains at full size (every layer's gain and the final norm's differ)."""
    _run("b1_8k_gains", steps=3, teacher_forced_step=0)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["b8_ragged_uniform", "b8_ragged_skewed"])
def test_full_b8_ragged(name):
    _run(name, steps=4, teacher_forced_step=0)


@pytest.mark.timeout(600)
def test_full_long_64k():
    _run("long_64k", steps=2)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["long_128k", "long_256k"])
def test_full_long_one_step(name):
    """128K and 256K contexts: one whole step against the oracle's whole step (logits, routing, K/V)."""
    _run(name, steps=1, lazy=True)


@pytest.mark.timeout(600)
def test_full_grid_and_page_order_invariance():
    """b8 skewed (the d_head-128 wave-independent attention, ragged contexts): the step's logits, tokens and new
    K/V are bit-identical on 256 and on 97 workgroups, and with the cache's pages placed in a second seeded
    shuffled order."""
    from decode_megakernel_wg_amd.session import Session

    w = W.make("b8_ragged_skewed", steps=1)
    pt, n_pages = W.page_tables(w)
    model = W.DeviceModel(w.shape)
    perm = np.random.default_rng(11).permutation(n_pages).astype(np.int32)
    pt2 = np.where(pt >= 0, perm[np.maximum(pt, 0)], -1).astype(np.int32)
    results = []
    for grid, table in ((0, pt), (97, pt), (0, pt2)):
        sess = Session(w, model=model, pt=table, n_pages=n_pages)
        sess.h.mk_set_grid(grid)
        sess.step()
        sess.status()
        new_kv = np.stack([np.stack([_gpu_kv_at(sess, l, b, w.ctx[b]) for b in range(w.B)]) for l in (0, w.shape.n_layers - 1)])
        results.append((sess.logits.cpu().numpy().copy(), sess.next_tokens().copy(), new_kv))
        del sess
        torch.cuda.empty_cache()
    for r in results[1:]:
        assert np.array_equal(r[0], results[0][0]) and np.array_equal(r[1], results[0][1]) and np.array_equal(r[2], results[0][2])


@pytest.mark.timeout(600)
def test_full_merge_tasks_bit_identical():
    """b8 skewed (ragged contexts, 1 to 14 splits per sequence): the split-KV partials merged by separate merge
    tasks over slices of each group's heads (MK_DBG_MERGE_TASKS; staged in LDS 16 bytes per lane at d_head 128)
    give the last-arriver merge's logits, tokens and new K/V bit for bit."""
    from decode_megakernel_wg_amd import mk
    from decode_megakernel_wg_amd.session import Session

    w = W.make("b8_ragged_skewed", steps=2)
    pt, n_pages = W.page_tables(w)
    model = W.DeviceModel(w.shape)
    results = []
    for flags in (0, mk.MK_DBG_MERGE_TASKS):
        sess = Session(w, model=model, pt=pt, n_pages=n_pages)
        sess.h.mk_debug_set(flags | mk.MK_DBG_PAGE_WALK | mk.MK_DBG_COUNT_TASKS)
        tasks = sess.h.mk_build_tasks(sess.seq_rows_host[0], want_tasks=True)
        assert ((tasks[:, 0] == 8).sum() > 0) == bool(flags)
        out = []
        for step in range(w.steps):
            sess.step()
            sess.status()
            check_step(sess.h, w.shape, sess.desc, pt, sess.seq_rows_host[step], plan_lens=sess.seq_rows_host[0], tasks=tasks)
            new_kv = np.stack([np.stack([_gpu_kv_at(sess, l, b, int(sess.seq_rows_host[step][b])) for b in range(w.B)])
                               for l in (0, w.shape.n_layers - 1)])
            out.append((sess.logits.cpu().numpy().copy(), sess.next_tokens().copy(), new_kv))
        results.append(out)
        del sess
        torch.cuda.empty_cache()
    for a, b in zip(results[0], results[1]):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
