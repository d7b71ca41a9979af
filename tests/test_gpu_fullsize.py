"""GPU parity at the full model size, in the launch configuration the benchmark times (one workgroup per
compute unit, phase pools, no debug switches unless a check needs them).

The 48-layer synthetic model (d_model 2048, 32 q / 4 KV heads x 128, 128 experts top-8, d_ffn 768, vocab
262144) runs one or two decode steps per workload; the oracle (fp64-accumulating C, weights generated per
layer on the host from the same seeded generator) runs the same steps, teacher-forced with the GPU's tokens.
Same bar as the small cases: logits relative L2 <= 1e-2, greedy tokens equal unless the oracle's top-2 gap
is below 1e-2, routing identical except at oracle near-ties (follow mode), new K/V written equal to the
oracle's (layer 0: within one BF16 rounding step; deeper layers: each head vector within relative L2
1e-2, since the residual stream there already differs by ~1e-4).  At 256K context the oracle computes the first
layer only (its KV cache alone is 537 MB) and is compared with the GPU's normalised input of layer 1.
"""
import numpy as np
import pytest
import torch

from oracle_runner import OracleRun, rel_l2, tie_ok, top2_gap
from synth import workloads as W

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-2
TOKEN_GAP = 1e-2
ROUTE_EPS = 1e-5


def _gpu_kv_at(sess, l, b, pos):
    """K and V (fp32) the GPU cache holds for sequence b at position pos of layer l: [2][Hkv][dh]."""
    from oracle import oracle as O

    page = int(sess.kvc.pt_host[b, pos // 16])
    kv = sess.kvc.kv[l, page, :, :, pos % 16, :].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return O.bf16_to_f32(kv)


def _oracle_kv_at(orc, l, b, pos):
    from oracle import oracle as O

    page = int(orc.pt[b, pos // 16])
    return O.bf16_to_f32(orc.kv[l][page, :, :, pos % 16, :])


def _compare_step(sess, orc, w, step, tokens, layers_kv=(0,)):
    from decode_megakernel_wg_amd import mk

    s = w.shape
    logits = sess.logits.cpu().numpy()
    nxt = sess.next_tokens()
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
            if l == 0:  # the first layer's projections agree to ~1e-6: at most one BF16 rounding step apart
                assert np.allclose(g, o, rtol=2 ** -7, atol=1e-4), f"{w.name} layer 0 seq {b}: new K/V differ"
            # deeper layers inherit the residual stream's ~1e-4 relative difference; each K and V head vector
            # is held to the logits' bar
            for kvh in np.ndindex(g.shape[:2]):
                e = rel_l2(g[kvh], o[kvh])
                assert e <= LOGIT_TOL, f"{w.name} layer {l} seq {b} {'KV'[kvh[0]]} head {kvh[1]}: rel L2 {e:.3e}"
    return [int(t) for t in nxt], agree, worst


def _teacher_forced_routing(sess, w):
    """Router of the GPU's own normalised inputs reproduces the GPU's selection (all layers)."""
    from decode_megakernel_wg_amd import mk
    from oracle import oracle as O

    s = w.shape
    n_gpu = sess.h.mk_debug_read(mk.MK_DBGK_NORM_IN, (s.n_layers, w.B, s.d_model), np.float32)
    gsel = sess.h.mk_debug_read(mk.MK_DBGK_ROUTE_SEL, (s.n_layers, w.B, s.top_k), np.int32)
    ties = 0
    for l in range(s.n_layers):
        wr = W.host_matrix(7, l, s.n_experts, s.d_model)
        for b in range(w.B):
            sel, _, lg = O.router(n_gpu[l, b], wr, s.top_k, w.router_bias)
            if not np.array_equal(sel, gsel[l, b]):
                assert tie_ok(lg, gsel[l, b], s.top_k, ROUTE_EPS), f"{w.name}: teacher-forced routing differs at layer {l} seq {b}"
                ties += 1
    assert ties <= max(1, 0.01 * s.n_layers * w.B)


def _run(name, steps, teacher_forced_step=None):
    from decode_megakernel_wg_amd import mk
    from decode_megakernel_wg_amd.session import Session

    w = W.make(name, steps=steps)
    pt, n_pages = W.page_tables(w)
    sess = Session(w, pt=pt, n_pages=n_pages)
    sess.h.mk_debug_set(0)  # per-task completion counts only (one counter increment per task)
    orc = OracleRun(w, pt, n_pages, keep_all=False)
    tokens = list(w.tokens)
    agree, worst = 0, 0.0
    for step in range(steps):
        if step == teacher_forced_step:
            sess.h.mk_debug_set(mk.MK_DBG_DUMP_N)
        sess.step()
        sess.status()
        done = sess.h.mk_debug_read(mk.MK_DBGK_TASK_DONE, (sess.h.n_tasks,), np.uint32)
        assert np.all(done == 1), f"{name} step {step}: tasks not run exactly once"
        if step == teacher_forced_step:
            _teacher_forced_routing(sess, w)
            sess.h.mk_debug_set(0)
        tokens, a, e = _compare_step(sess, orc, w, step, tokens, layers_kv=(0, w.shape.n_layers // 2, w.shape.n_layers - 1))
        agree += a
        worst = max(worst, e)
    assert agree >= 0.99 * steps * w.B
    print(f"{name}: worst logits rel L2 {worst:.2e}, oracle follow-mode near-ties {orc.near_ties}/{orc.route_checked}")


@pytest.mark.timeout(600)
def test_full_b1_8k():
    _run("b1_8k", steps=2, teacher_forced_step=1)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["b8_ragged_uniform", "b8_ragged_skewed"])
def test_full_b8_ragged(name):
    _run(name, steps=1)


@pytest.mark.timeout(600)
def test_full_long_64k():
    _run("long_64k", steps=1)


@pytest.mark.timeout(600)
def test_full_long_256k_first_layer():
    """256K context: the whole step on the GPU; the oracle computes layer 0 (attention over 262145 positions
    and the MoE) and its result is compared with the GPU's normalised input of layer 1 and its new layer-0 K/V."""
    from decode_megakernel_wg_amd import mk
    from decode_megakernel_wg_amd.session import Session
    from oracle import oracle as O

    w = W.make("long_256k", steps=1)
    pt, n_pages = W.page_tables(w)
    sess = Session(w, pt=pt, n_pages=n_pages)
    sess.h.mk_debug_set(mk.MK_DBG_DUMP_N)
    sess.step()
    sess.status()
    s = w.shape
    logits = sess.logits.cpu().numpy()
    assert np.isfinite(logits).all()
    done = sess.h.mk_debug_read(mk.MK_DBGK_TASK_DONE, (sess.h.n_tasks,), np.uint32)
    assert np.all(done == 1)
    n_gpu = sess.h.mk_debug_read(mk.MK_DBGK_NORM_IN, (s.n_layers, w.B, s.d_model), np.float32)
    gsel = sess.h.mk_debug_read(mk.MK_DBGK_ROUTE_SEL, (s.n_layers, w.B, s.top_k), np.int32)
    orc = OracleRun(w, pt, n_pages, keep_all=False, kv_layers=1)
    x1, sels, ns = orc.layers(list(w.tokens), np.array(w.ctx, np.int64), 1, gpu_sel=gsel)
    assert rel_l2(n_gpu[0, 0], ns[0][0]) < 1e-6, "layer-0 normalised input differs"
    n1 = O.rmsnorm(x1[0], np.full(s.d_model, W.ONE_BF16, np.uint16))
    e = rel_l2(n_gpu[1, 0], n1)
    assert e < 1e-4, f"layer-1 input after 256K attention: rel L2 {e:.3e}"
    g, o = _gpu_kv_at(sess, 0, 0, w.ctx[0]), _oracle_kv_at(orc, 0, 0, w.ctx[0])
    assert np.allclose(g, o, rtol=2 ** -7, atol=1e-4)
    print(f"long_256k: layer-1 input rel L2 {e:.2e}")
