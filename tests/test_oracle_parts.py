"""Pins of the CPU oracle's parts against library routines, closed forms, invariants and brute force.

Nothing here retypes the oracle's formulas: each check uses an independent
library routine (numpy / scipy / torch on the CPU in float64), a closed form
or an invariant that a dropped term, wrong sign, wrong index or transposed
operand would break.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import softmax

from oracle import oracle as O

RNG = np.random.default_rng(1234)


def rand_bf16(*shape, scale=0.02):
    return O.f32_to_bf16(RNG.normal(0, scale, size=shape).astype(np.float32))


def f64(b):
    return O.bf16_to_f32(b).astype(np.float64)


def dims(**kw):
    base = dict(n_layers=1, d_model=64, n_q_heads=4, n_kv_heads=2, d_head=16, n_experts=6, top_k=2, d_ffn=32, vocab=100,
                page_size=16)
    base.update(kw)
    return O.Dims(**base)


# ---------------------------------------------------------------- bf16 conversion

def test_bf16_rounding_matches_torch():
    x = np.concatenate([RNG.normal(0, 1, 10000), [0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 65504.0, 1e-40]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16(x), ref)
    lib = O.lib()
    for v in x[:50]:
        assert lib.or_f32_to_bf16(float(v)) == O.f32_to_bf16(np.array([v]))[0]


# ---------------------------------------------------------------- matvec

def test_matvec_matches_numpy_float64():
    W = rand_bf16(37, 300)
    x = RNG.normal(size=300).astype(np.float32)
    y = O.matvec(W, x)
    ref = (f64(W) @ x.astype(np.float64)).astype(np.float32)
    assert np.array_equal(y, ref) or np.max(np.abs(y - ref) / np.abs(ref)) < 1e-6


def test_matvec_orientation():
    # W [rows][cols] row-major: a one-hot x picks a column
    W = rand_bf16(5, 7)
    x = np.zeros(7, np.float32)
    x[3] = 1.0
    assert np.array_equal(O.matvec(W, x), O.bf16_to_f32(W[:, 3]))


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_vector_closed_form():
    d, c, eps = 256, 0.37, 1e-6
    x = np.full(d, c, np.float32)
    g = np.full(d, 0x3F80, np.uint16)
    n = O.rmsnorm(x, g, eps)
    expect = np.float32(np.float32(c) / math.sqrt(float(np.float32(c)) ** 2 + eps))
    assert np.allclose(n, expect, rtol=1e-7, atol=0)


def test_rmsnorm_scale_invariance_gain_and_unit_rms():
    x = RNG.normal(size=512).astype(np.float32)
    g1 = np.full(512, 0x3F80, np.uint16)
    n1 = O.rmsnorm(x, g1)
    n2 = O.rmsnorm(x * 8.0, g1)
    assert np.allclose(n1, n2, rtol=1e-6)
    assert abs(np.mean(n1.astype(np.float64) ** 2) - 1.0) < 1e-5
    g = rand_bf16(512, scale=1.0)
    ng = O.rmsnorm(x, g)
    assert np.allclose(ng, n1 * O.bf16_to_f32(g), rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------- RoPE

def test_rope_identity_at_position_zero():
    v = RNG.normal(size=(3, 16)).astype(np.float32)
    assert np.array_equal(O.rope(v, 0), v)


def test_rope_two_dims_is_a_plane_rotation():
    # d_head = 2: one pair, frequency base^0 = 1, angle = position
    v = np.array([[1.0, 0.0]], np.float32)
    for p in (1, 5, 1000):
        r = O.rope(v, p)
        assert np.allclose(r[0], [math.cos(p), math.sin(p)], atol=1e-7)
        assert abs(math.atan2(r[0, 1], r[0, 0]) - math.atan2(math.sin(p), math.cos(p))) < 1e-6


def test_rope_frequencies_and_pairing():
    # d_head = 8, base 10000: pair i = (i, i+4) turns by p * 10000^(-2i/8)
    dh = 8
    for i in range(dh // 2):
        v = np.zeros((1, dh), np.float32)
        v[0, i] = 1.0
        p = 3
        r = O.rope(v, p)
        ang = math.atan2(r[0, i + dh // 2], r[0, i])
        want = (p * 10000.0 ** (-2 * i / dh) + math.pi) % (2 * math.pi) - math.pi
        assert abs(ang - want) < 1e-6
        others = [j for j in range(dh) if j not in (i, i + dh // 2)]
        assert np.all(r[0, others] == 0)


def test_rope_norm_and_relative_position():
    q = RNG.normal(size=(2, 64)).astype(np.float32)
    k = RNG.normal(size=(2, 64)).astype(np.float32)
    for p in (7, 300):
        r = O.rope(q, p)
        a, b = r[:, :32], r[:, 32:]
        assert np.allclose(a ** 2 + b ** 2, q[:, :32] ** 2 + q[:, 32:] ** 2, rtol=1e-5)
    d1 = (O.rope(q, 100).astype(np.float64) * O.rope(k, 90)).sum(-1)
    d2 = (O.rope(q, 1010).astype(np.float64) * O.rope(k, 1000)).sum(-1)
    assert np.allclose(d1, d2, rtol=1e-4, atol=1e-4)


# ---------------------------------------------------------------- attention

def paged_cache(D, K, V, page_table, n_pages):
    """K, V: [n_ctx][Hkv][dh] uint16 -> paged cache [n_pages][2][Hkv][ps][dh]."""
    kv = np.zeros((n_pages, 2, D.n_kv_heads, D.page_size, D.d_head), np.uint16)
    for j in range(K.shape[0]):
        ph = page_table[j // D.page_size]
        kv[ph, 0, :, j % D.page_size] = K[j]
        kv[ph, 1, :, j % D.page_size] = V[j]
    return kv


def sdpa_ref(D, q, K, V):
    grp = D.n_q_heads // D.n_kv_heads
    qt = torch.from_numpy(q.astype(np.float64))[:, None, :]                     # [Hq][1][dh]
    kt = torch.from_numpy(f64(K)).permute(1, 0, 2).repeat_interleave(grp, 0)    # [Hq][n][dh]
    vt = torch.from_numpy(f64(V)).permute(1, 0, 2).repeat_interleave(grp, 0)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous())[:, 0].numpy()


@pytest.mark.parametrize("n_ctx", [1, 15, 16, 17, 200])
def test_attention_matches_torch_sdpa(n_ctx):
    D = dims()
    K = rand_bf16(n_ctx, D.n_kv_heads, D.d_head, scale=1.0)
    V = rand_bf16(n_ctx, D.n_kv_heads, D.d_head, scale=1.0)
    q = RNG.normal(size=(D.n_q_heads, D.d_head)).astype(np.float32)
    n_pages = -(-n_ctx // 16) + 2
    pt = RNG.permutation(n_pages).astype(np.int32)
    kv = paged_cache(D, K, V, pt, n_pages)
    out = O.attention(D, q, kv, pt, n_ctx)
    ref = sdpa_ref(D, q, K, V)
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_attention_special_cases():
    D = dims()
    q = RNG.normal(size=(D.n_q_heads, D.d_head)).astype(np.float32)
    pt = np.arange(4, dtype=np.int32)
    # a single position returns V exactly
    K = rand_bf16(1, D.n_kv_heads, D.d_head, scale=1.0)
    V = rand_bf16(1, D.n_kv_heads, D.d_head, scale=1.0)
    out = O.attention(D, q, paged_cache(D, K, V, pt, 4), pt, 1)
    grp = D.n_q_heads // D.n_kv_heads
    for h in range(D.n_q_heads):
        assert np.array_equal(out[h], O.bf16_to_f32(V[0, h // grp]))
    # equal keys give the mean of V
    K = np.repeat(rand_bf16(1, D.n_kv_heads, D.d_head, scale=1.0), 40, axis=0)
    V = rand_bf16(40, D.n_kv_heads, D.d_head, scale=1.0)
    out = O.attention(D, q, paged_cache(D, K, V, pt, 4), pt, 40)
    for h in range(D.n_q_heads):
        assert np.allclose(out[h], f64(V[:, h // grp]).mean(0), atol=1e-6)


def test_attention_paged_equals_contiguous_and_positions_are_a_set():
    D = dims()
    n = 70
    K = rand_bf16(n, D.n_kv_heads, D.d_head, scale=1.0)
    V = rand_bf16(n, D.n_kv_heads, D.d_head, scale=1.0)
    q = RNG.normal(size=(D.n_q_heads, D.d_head)).astype(np.float32)
    ident = np.arange(5, dtype=np.int32)
    shuf = np.array([3, 0, 4, 1, 2], np.int32)
    a = O.attention(D, q, paged_cache(D, K, V, ident, 5), ident, n)
    b = O.attention(D, q, paged_cache(D, K, V, shuf, 5), shuf, n)
    assert np.array_equal(a, b)
    # positions are an unordered set for decode attention (no mask inside the window)
    perm = RNG.permutation(n)
    c = O.attention(D, q, paged_cache(D, K[perm], V[perm], ident, 5), ident, n)
    assert np.allclose(a, c, atol=1e-6)


def test_attention_rejects_bad_pages():
    D = dims()
    kv = np.zeros((2, 2, D.n_kv_heads, 16, D.d_head), np.uint16)
    with pytest.raises(ValueError):
        O.attention(D, np.zeros((D.n_q_heads, D.d_head), np.float32), kv, np.array([0, 5], np.int32), 20)


# ---------------------------------------------------------------- router

def test_router_matches_sort_and_softmax():
    E, d, k = 16, 64, 4
    w = rand_bf16(E, d, scale=0.2)
    n = RNG.normal(size=d).astype(np.float32)
    bias = RNG.normal(size=E).astype(np.float32)
    sel, gate, logits = O.router(n, w, k, bias)
    raw = (f64(w) @ n.astype(np.float64)).astype(np.float32)
    assert np.array_equal(logits, raw + bias)
    order = np.lexsort((np.arange(E), -logits.astype(np.float64)))[:k]
    assert np.array_equal(sel, order)
    assert np.allclose(gate, softmax(logits[sel].astype(np.float64)), rtol=1e-6)


def test_router_k_equal_E_and_k_one():
    E, d = 8, 32
    w = rand_bf16(E, d, scale=0.3)
    n = RNG.normal(size=d).astype(np.float32)
    sel, gate, logits = O.router(n, w, E)
    full = softmax(logits.astype(np.float64))
    assert np.allclose(gate, full[sel], rtol=1e-6)
    sel1, gate1, _ = O.router(n, w, 1)
    assert gate1[0] == 1.0 and sel1[0] == int(np.argmax(logits))


def test_router_ties_go_to_the_lower_index_and_permutation_equivariance():
    E, d = 8, 16
    w = np.zeros((E, d), np.uint16)
    row = rand_bf16(d, scale=0.3)
    for e in (2, 5, 6):
        w[e] = row
    n = RNG.normal(size=d).astype(np.float32)
    if (f64(row) @ n) < 0:
        n = -n
    sel, gate, _ = O.router(n, w, 2)
    assert sel.tolist() == [2, 5] and np.allclose(gate, [0.5, 0.5])
    w2 = rand_bf16(E, d, scale=0.3)
    perm = RNG.permutation(E)
    s1, g1, _ = O.router(n, w2, 3)
    s2, g2, _ = O.router(n, w2[perm], 3)
    assert np.array_equal(perm[s2], s1) and np.array_equal(g1, g2)


# ---------------------------------------------------------------- expert

def test_expert_matches_torch_silu():
    d, F = 48, 40
    wg, wu, wd = rand_bf16(F, d, scale=0.3), rand_bf16(F, d, scale=0.3), rand_bf16(d, F, scale=0.3)
    n = RNG.normal(size=d).astype(np.float32)
    y = O.expert(n, wg, wu, wd)
    g = torch.from_numpy(f64(wg) @ n.astype(np.float64))
    u = torch.from_numpy(f64(wu) @ n.astype(np.float64))
    ref = f64(wd) @ (torch.nn.functional.silu(g) * u).numpy()
    assert np.allclose(y, ref, rtol=1e-5, atol=1e-7)


def test_expert_zero_cases():
    d, F = 16, 8
    n = RNG.normal(size=d).astype(np.float32)
    wu, wd = rand_bf16(F, d, scale=0.3), rand_bf16(d, F, scale=0.3)
    assert np.all(O.expert(n, np.zeros((F, d), np.uint16), wu, wd) == 0)       # silu(0) = 0
    assert np.all(O.expert(n, rand_bf16(F, d), wu, np.zeros((d, F), np.uint16)) == 0)


# ---------------------------------------------------------------- head

def test_head_matches_numpy_and_first_argmax():
    D = dims(vocab=50)
    x = RNG.normal(size=(3, D.d_model)).astype(np.float32)
    g = np.full(D.d_model, 0x3F80, np.uint16)
    lm = rand_bf16(50, D.d_model, scale=0.3)
    lm[17] = lm[4]   # a duplicated row: ties resolve to the lower index
    logits, nxt = O.head(D, x, g, lm)
    for b in range(3):
        n = x[b].astype(np.float64) / math.sqrt(np.mean(x[b].astype(np.float64) ** 2) + 1e-6)
        ref = f64(lm) @ n.astype(np.float32).astype(np.float64)
        assert np.allclose(logits[b], ref, rtol=1e-5, atol=1e-6)
        assert nxt[b] == int(np.argmax(logits[b]))
    x2 = np.zeros((1, D.d_model), np.float32)
    x2[0, 0] = 1.0
    lm2 = np.zeros((50, D.d_model), np.uint16)
    lm2[[9, 30], 0] = 0x3F80
    _, nx2 = O.head(D, x2, g, lm2)
    assert nx2[0] == 9
