"""The allocation-free decode step (mk_decode_step_static) against mk_decode_step, through the C ABI.

Both run the same kernel on the same inputs, so their logits, greedy tokens and written K/V are equal bit for
bit; checked on two calls in a row on one handle (a ragged batch of 8, then a smaller batch of 3 with other
lengths, whose scratch layout differs), and on the full-size model at batch 1.
"""
import numpy as np
import pytest
import torch

from synth import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("cuda")]


def _both(sess, seq_lens, rows, B):
    """The regular step, then the static one, on the same handle and inputs; returns both results."""
    from decode_megakernel_wg_amd import mk

    h = sess.h
    toks = torch.tensor(sess.w.tokens[:B], dtype=torch.int32, device="cuda")
    lens = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    pt = torch.from_numpy(np.ascontiguousarray(rows)).cuda()
    h.mk_build_tasks(seq_lens)
    out = []
    for static in (False, True):
        logits = torch.full((B, sess.shape.vocab), float("nan"), dtype=torch.float32, device="cuda")
        (h.mk_decode_step_static if static else h.mk_decode_step)(toks, lens, pt, sess.kvc.kv, logits)
        h.mk_status()
        nxt = mk.read_device(h.mk_next_tokens(), 4 * B)
        kv = sess.kvc.kv.view(torch.int16).clone()
        out.append((logits.cpu().numpy(), nxt, kv))
    return out


def test_static_step_equals_regular_step_twice():
    from decode_megakernel_wg_amd.session import Session

    w = W.make("tiny_ragged", steps=1)
    pt, n_pages = W.page_tables(w)
    sess = Session(w, pt=pt, n_pages=n_pages)
    for B, lens in ((8, list(w.ctx)), (3, [w.ctx[0] + 1, 5, w.ctx[2] + 1])):
        (l0, n0, kv0), (l1, n1, kv1) = _both(sess, np.array(lens, np.int32), pt[:B], B)
        assert np.isfinite(l0).all()
        assert np.array_equal(l0, l1) and np.array_equal(n0, n1), f"batch {B}: static step differs"
        assert torch.equal(kv0, kv1), f"batch {B}: K/V written differently"


def test_static_step_full_size_batch_1():
    from decode_megakernel_wg_amd.session import Session

    w = W.make("b1_8k", steps=1)
    sess = Session(w)
    (l0, n0, _), (l1, n1, _) = _both(sess, np.array(w.ctx, np.int32), sess.kvc.pt_host, 1)
    assert np.array_equal(l0, l1) and np.array_equal(n0, n1)


def test_static_step_long_context_merge_tasks():
    """A 16384-position context of the tiny model, whose plan merges the splits in merge tasks: the static step
    equals the regular one bit for bit."""
    from decode_megakernel_wg_amd import mk
    from decode_megakernel_wg_amd.session import Session

    w = W.make("tiny_long", steps=1)
    sess = Session(w)
    tasks, _ = mk.mk_plan_tasks(sess.desc, w.ctx)
    assert (tasks[:, 0] == 8).any()
    (l0, n0, kv0), (l1, n1, kv1) = _both(sess, np.array(w.ctx, np.int32), sess.kvc.pt_host, 1)
    assert np.isfinite(l0).all()
    assert np.array_equal(l0, l1) and np.array_equal(n0, n1) and torch.equal(kv0, kv1)
