"""Pins of the oracle on chunked prefill: a step whose batch holds consecutive positions of one sequence.

The oracle's layer takes a batch in order and, for each token, writes its K/V before it attends, so a chunk
of P consecutive positions of one sequence (entries sharing a page-table row) is causal by construction:
token i sees the cache below the chunk plus the chunk's tokens 0..i.  Pinned here by
 - equality with P single-token steps (the same tokens decoded one after another), bit for bit, for the
   layer outputs and the cache;
 - brute-force causal attention (torch's scaled-dot-product attention in fp64 on the CPU, an explicit
   lower-triangular mask over the chunk, KV heads repeated per GQA group) on a layer whose output
   projection is the identity, so the layer's attention output is the attention result itself.
"""
import math

import numpy as np
import torch

from oracle import oracle as O
from test_oracle_layer import ONE, fresh_cache, rand_bf16, small_dims, small_layer

RNG = np.random.default_rng(2024)


def rope64(v, pos, base=10000.0):
    """Rotate-half RoPE in fp64 at position pos on [heads][d_head]."""
    v = np.asarray(v, np.float64).copy()
    half = v.shape[1] // 2
    i = np.arange(half)
    th = pos * base ** (-2.0 * i / v.shape[1])
    c, s = np.cos(th), np.sin(th)
    a, b = v[:, :half].copy(), v[:, half:].copy()
    v[:, :half] = a * c - b * s
    v[:, half:] = a * s + b * c
    return v


def test_chunk_equals_single_token_steps():
    D = small_dims()
    layers = [small_layer(D) for _ in range(2)]
    p0, P = 21, 11   # the chunk starts mid-page and crosses a page boundary
    kv_a = [fresh_cache(D, p0, seed=7 + l)[0] for l in range(2)]
    kv_b = [k.copy() for k in kv_a]
    pt = np.arange(8, dtype=np.int32)
    x0 = RNG.normal(size=(P, D.d_model)).astype(np.float32)
    pos = p0 + np.arange(P)
    # one step: the whole chunk
    xa = x0.copy()
    for l in range(2):
        xa, _ = O.layer(D, layers[l], pos, np.repeat(pt[None], P, axis=0), kv_a[l], xa)
    # P steps of one token each
    xb = np.empty_like(x0)
    for i in range(P):
        x = x0[i:i + 1].copy()
        for l in range(2):
            x, _ = O.layer(D, layers[l], pos[i:i + 1], pt[None], kv_b[l], x)
        xb[i] = x[0]
    assert np.array_equal(xa, xb)
    for l in range(2):
        assert np.array_equal(kv_a[l], kv_b[l])


def test_chunk_attention_is_causal_brute_force():
    D = small_dims()
    d, dh, Hq, Hkv = D.d_model, D.d_head, D.n_q_heads, D.n_kv_heads
    assert d == Hq * dh
    base = small_layer(D, zero_moe=True)
    eye = np.zeros((d, d), np.uint16)
    eye[np.arange(d), np.arange(d)] = ONE
    Wl = O.LayerWeights(base.arrs[0], base.arrs[1], base.arrs[2], base.arrs[3], eye, base.arrs[5], base.exp, D.n_experts)
    p0, P = 37, 9
    kv, pt = fresh_cache(D, p0)
    x = RNG.normal(size=(P, d)).astype(np.float32)
    pos = p0 + np.arange(P)
    _, aux = O.layer(D, Wl, pos, np.repeat(pt[None], P, axis=0), kv, x)
    # every cached K/V the chunk may see, in logical order (the chunk's own slots written by the call)
    n_pos = p0 + P
    K = np.stack([O.bf16_to_f32(kv[pt[j // 16], 0, :, j % 16]) for j in range(n_pos)], 1)  # [Hkv][pos][dh]
    V = np.stack([O.bf16_to_f32(kv[pt[j // 16], 1, :, j % 16]) for j in range(n_pos)], 1)
    Kq = torch.from_numpy(np.repeat(K, Hq // Hkv, axis=0).astype(np.float64))
    Vq = torch.from_numpy(np.repeat(V, Hq // Hkv, axis=0).astype(np.float64))
    wq = O.bf16_to_f32(Wl.arrs[1]).astype(np.float64)
    for i in range(P):
        q = rope64((wq @ aux["n"][i].astype(np.float64)).reshape(Hq, dh), pos[i])
        mask = torch.zeros(1, n_pos, dtype=torch.bool)
        mask[0, :pos[i] + 1] = True   # causal: the cache below the chunk and the chunk up to token i
        ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], Kq, Vq, attn_mask=mask)[:, 0, :]
        got = aux["attn"][i].reshape(Hq, dh)
        assert np.allclose(got, ref.numpy(), rtol=1e-5, atol=1e-6), f"chunk token {i}"
    # the chunk's last token differs from what it would see without its predecessors in the cache
    assert not np.allclose(aux["attn"][P - 1], aux["attn"][0])
