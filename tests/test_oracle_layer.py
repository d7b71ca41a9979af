"""Pins of the oracle's layer and step composition: the parallel-layer algebra, the KV write,
self-attention of the new token, routing renormalisation, ragged batches and zero branches."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from synth import synth, workloads as W

RNG = np.random.default_rng(99)
ONE = np.uint16(0x3F80)


def rand_bf16(*shape, scale=0.02):
    return O.f32_to_bf16(RNG.normal(0, scale, size=shape).astype(np.float32))


def small_dims():
    return O.Dims(n_layers=2, d_model=64, n_q_heads=4, n_kv_heads=2, d_head=16, n_experts=6, top_k=2, d_ffn=32, vocab=100)


def small_layer(D, scale=0.1, identical_experts=False, zero_attn=False, zero_moe=False):
    d, dh = D.d_model, D.d_head
    wo = np.zeros((d, D.n_q_heads * dh), np.uint16) if zero_attn else rand_bf16(d, D.n_q_heads * dh, scale=scale)
    base = (rand_bf16(D.d_ffn, d, scale=scale), rand_bf16(D.d_ffn, d, scale=scale), rand_bf16(d, D.d_ffn, scale=scale))
    experts = {}
    for e in range(D.n_experts):
        t = base if identical_experts else (rand_bf16(D.d_ffn, d, scale=scale), rand_bf16(D.d_ffn, d, scale=scale),
                                            rand_bf16(d, D.d_ffn, scale=scale))
        if zero_moe:
            t = (t[0], t[1], np.zeros_like(t[2]))
        experts[e] = t
    return O.LayerWeights(np.full(d, ONE, np.uint16), rand_bf16(D.n_q_heads * dh, d, scale=scale),
                          rand_bf16(D.n_kv_heads * dh, d, scale=scale), rand_bf16(D.n_kv_heads * dh, d, scale=scale), wo,
                          rand_bf16(D.n_experts, d, scale=scale), experts, D.n_experts)


def fresh_cache(D, n_ctx, n_pages=8, seed=5, pt=None):
    kv = np.zeros((1, n_pages, 2, D.n_kv_heads, 16, D.d_head), np.uint16)
    pt = np.arange(n_pages, dtype=np.int32) if pt is None else pt
    synth.fill_kv_host(kv, 0, D.n_kv_heads, D.d_head, 16, pt, 0, 0, n_ctx, seed)
    return kv[0], pt


def test_layer_algebra_and_kv_write():
    D = small_dims()
    Wl = small_layer(D)
    p = 37
    kv, pt = fresh_cache(D, p)
    kv0 = kv.copy()
    x = RNG.normal(size=(1, D.d_model)).astype(np.float32)
    x2, aux = O.layer(D, Wl, [p], pt[None], kv, x)
    # x' = x + Attn(n) + MoE(n), each branch recomputed from the oracle's parts
    n = O.rmsnorm(x[0], Wl.arrs[0])
    assert np.array_equal(n, aux["n"][0])
    q = O.rope(O.matvec(Wl.arrs[1], n).reshape(D.n_q_heads, D.d_head), p)
    k = O.rope(O.matvec(Wl.arrs[2], n).reshape(D.n_kv_heads, D.d_head), p)
    v = O.matvec(Wl.arrs[3], n).reshape(D.n_kv_heads, D.d_head)
    ph, slot = pt[p // 16], p % 16
    assert np.array_equal(kv[ph, 0, :, slot], O.f32_to_bf16(k))
    assert np.array_equal(kv[ph, 1, :, slot], O.f32_to_bf16(v))
    mask = np.ones(kv.shape, bool)
    mask[ph, :, :, slot] = False
    assert np.array_equal(kv[mask], kv0[mask])
    o = O.attention(D, q, kv, pt, p + 1)
    a = O.matvec(Wl.arrs[4], o.reshape(-1))
    assert np.array_equal(a, aux["attn"][0])
    sel, gate, _ = O.router(n, Wl.arrs[5], D.top_k)
    assert np.array_equal(sel, aux["sel"][0]) and np.array_equal(gate, aux["gate"][0])
    m = sum(np.float64(gate[j]) * O.expert(n, *Wl.exp[sel[j]]).astype(np.float64) for j in range(D.top_k))
    assert np.array_equal(m.astype(np.float32), aux["moe"][0])
    ref = (x[0].astype(np.float64) + a.astype(np.float64) + aux["moe"][0].astype(np.float64)).astype(np.float32)
    assert np.array_equal(x2[0], ref)


def test_first_position_attends_only_to_itself():
    D = small_dims()
    Wl = small_layer(D)
    kv, pt = fresh_cache(D, 0)
    x = RNG.normal(size=(1, D.d_model)).astype(np.float32)
    _, aux = O.layer(D, Wl, [0], pt[None], kv, x)
    n = aux["n"][0]
    v = O.bf16_to_f32(O.f32_to_bf16(O.matvec(Wl.arrs[3], n))).reshape(D.n_kv_heads, D.d_head)
    grp = D.n_q_heads // D.n_kv_heads
    o = np.stack([v[h // grp] for h in range(D.n_q_heads)])
    assert np.array_equal(aux["attn"][0], O.matvec(Wl.arrs[4], o.reshape(-1)))


def test_zero_branches_leave_the_residual():
    D = small_dims()
    Wl = small_layer(D, zero_attn=True, zero_moe=True)
    kv, pt = fresh_cache(D, 20)
    x = RNG.normal(size=(1, D.d_model)).astype(np.float32)
    x2, _ = O.layer(D, Wl, [20], pt[None], kv, x)
    assert np.array_equal(x2, x)


def test_identical_experts_make_moe_independent_of_routing():
    # holds only when the gates are renormalised over the k selected experts
    D = small_dims()
    Wl = small_layer(D, identical_experts=True, zero_attn=True)
    kv, pt = fresh_cache(D, 5)
    x = RNG.normal(size=(1, D.d_model)).astype(np.float32)
    _, aux = O.layer(D, Wl, [5], pt[None], kv, x)
    y = O.expert(aux["n"][0], *Wl.exp[0])
    assert np.allclose(aux["moe"][0], y, rtol=1e-6, atol=1e-8)
    _, aux2 = O.layer(D, Wl, [5], pt[None], fresh_cache(D, 5)[0], x, sel_force=np.array([[4, 1]], np.int32))
    assert aux2["sel"][0].tolist() == [4, 1]
    lg = aux2["router_logits"][0].astype(np.float64)
    g = np.exp(lg[[4, 1]] - lg[[4, 1]].max())
    assert np.allclose(aux2["gate"][0], g / g.sum(), rtol=1e-6)
    assert np.allclose(aux2["moe"][0], y, rtol=1e-6, atol=1e-8)


def test_ragged_batch_equals_per_sequence_runs():
    D = small_dims()
    Wl = small_layer(D)
    pos = [3, 40, 17]
    n_pages = 12
    pts = np.stack([RNG.permutation(n_pages).astype(np.int32) for _ in pos])
    x = RNG.normal(size=(3, D.d_model)).astype(np.float32)
    caches = [fresh_cache(D, p, n_pages, seed=10 + i, pt=pts[i])[0] for i, p in enumerate(pos)]
    singles = []
    for i, p in enumerate(pos):
        c = caches[i].copy()
        xi, ai = O.layer(D, Wl, [p], pts[i:i + 1], c, x[i:i + 1])
        singles.append((xi[0], ai["sel"][0], c))
    # batch: all three sequences in one cache, disjoint pages via offset tables
    big = np.zeros((3 * n_pages,) + caches[0].shape[1:], np.uint16)
    pt_big = np.stack([pts[i] + i * n_pages for i in range(3)]).astype(np.int32)
    for i in range(3):
        big[i * n_pages:(i + 1) * n_pages] = caches[i]
    xb, ab = O.layer(D, Wl, pos, pt_big, big, x)
    for i in range(3):
        assert np.array_equal(xb[i], singles[i][0])
        assert np.array_equal(ab["sel"][i], singles[i][1])
        assert np.array_equal(big[i * n_pages:(i + 1) * n_pages], singles[i][2])


def test_step_with_zero_branches_is_embedding_through_the_head():
    D = small_dims()
    layers = [small_layer(D, zero_attn=True, zero_moe=True) for _ in range(D.n_layers)]
    emb = rand_bf16(D.vocab, D.d_model, scale=1.0)
    lm = rand_bf16(D.vocab, D.d_model, scale=0.5)
    fn = np.full(D.d_model, ONE, np.uint16)
    tok = [7, 42]
    kv = np.zeros((D.n_layers, 8, 2, D.n_kv_heads, 16, D.d_head), np.uint16)
    pt = np.stack([np.arange(4), np.arange(4, 8)]).astype(np.int32)
    x = O.embed(D, emb, tok)
    for l in range(D.n_layers):
        x, _ = O.layer(D, layers[l], [10, 3], pt, kv[l], x)
    logits, nxt = O.head(D, x, fn, lm)
    for b, t in enumerate(tok):
        e = O.bf16_to_f32(emb[t]).astype(np.float64)
        n = (e / math.sqrt(np.mean(e ** 2) + 1e-6)).astype(np.float32).astype(np.float64)
        ref = O.bf16_to_f32(lm).astype(np.float64) @ n
        assert np.allclose(logits[b], ref, rtol=1e-5, atol=1e-6)
        assert nxt[b] == np.argmax(logits[b])


def test_decode_step_equals_layer_by_layer_composition_on_the_tiny_model():
    w = W.make("tiny", steps=1)
    s = w.shape
    D = O.Dims(s.n_layers, s.d_model, s.n_q_heads, s.n_kv_heads, s.d_head, s.n_experts, s.top_k, s.d_ffn, s.vocab)
    pt, n_pages = W.page_tables(w)
    kv = W.host_kv(w, pt, n_pages)
    layers = []
    for l in range(s.n_layers):
        hl = W.host_layer(s, l)
        ex = {e: W.host_expert(s, l, e) for e in range(s.n_experts)}
        layers.append(O.LayerWeights(hl["attn_norm"], hl["wq"], hl["wk"], hl["wv"], hl["wo"], hl["w_router"], ex, s.n_experts))
    emb, lm = W.host_embed(s), W.host_lm_head(s)
    fn = np.full(s.d_model, ONE, np.uint16)
    # composition through the Python helpers
    kv1 = kv.copy()
    x = O.embed(D, emb, w.tokens)
    for l in range(s.n_layers):
        x, _ = O.layer(D, layers[l], w.ctx, pt, kv1[l], x)
    logits1, nxt1 = O.head(D, x, fn, lm)
    # one C call
    import ctypes as C
    arr = (O.OrLayerW * s.n_layers)(*[L.c for L in layers])
    kv2 = kv.copy()
    logits2 = np.empty((1, s.vocab), np.float32)
    nxt2 = np.empty(1, np.int32)
    tok = np.array(w.tokens, np.int32)
    pos = np.array(w.ctx, np.int64)
    dc = D.c()
    rc = O.lib().or_decode_step(C.byref(dc), C.cast(arr, C.c_void_p), O._p(emb), O._p(fn), O._p(lm), 1, O._p(tok), O._p(pos), O._p(pt),
                                pt.shape[1], O._p(kv2), n_pages, O._p(logits2), O._p(nxt2), None, None, None)
    assert rc == 0
    assert np.array_equal(logits1, logits2) and np.array_equal(nxt1, nxt2) and np.array_equal(kv1, kv2)
