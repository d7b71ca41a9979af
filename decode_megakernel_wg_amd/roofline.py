"""Algorithmic bytes of one decode step and the HBM speed-of-light.

The pages define the bound as the bytes a decode step must stream from HBM, the
active weights plus the KV cache read, divided by the HBM bandwidth
(agenticcommons.xyz "Cohere North Mini Code megakernel serving engine", section
為什麼 decode 慢; aimodeling.com "Cohere megakernel engine: one CUDA file, 1.58x
vLLM on H100", section "Decode is a bandwidth game").  Counted per step: every
layer's attention and router weights and norm gain, each expert the step's
tokens select counted once per layer, the LM head and final gain, the embedding
rows of the distinct input tokens, and K and V of every position each sequence
attends to (its prior positions plus the new one).  The new K/V writes and the
logits writes are not counted.
"""
from __future__ import annotations

MI355X_HBM_BYTES_PER_S = 8.0e12


def step_bytes(shape, ctx_lens, unique_experts_per_layer, n_unique_tokens):
    """Algorithmic HBM bytes of one step.  ctx_lens: prior positions per sequence;
    unique_experts_per_layer: iterable of U_l (distinct experts used in layer l)."""
    s = shape
    per_layer_fixed = s.layer_attn_bytes() + s.router_bytes() + 2 * s.d_model
    w = sum(per_layer_fixed + u * s.expert_bytes() for u in unique_experts_per_layer)
    w += 2 * s.vocab * s.d_model + 2 * s.d_model + 2 * s.d_model * n_unique_tokens
    kv = sum((int(c) + 1) * s.kv_bytes_per_pos_layer() * s.n_layers for c in ctx_lens)
    return w + kv


def weight_bytes(shape, unique_experts_per_layer, n_unique_tokens):
    return step_bytes(shape, [], unique_experts_per_layer, n_unique_tokens)


def sol_tokens_per_s(bytes_per_step, tokens_per_step=1, bandwidth=MI355X_HBM_BYTES_PER_S):
    return tokens_per_step * bandwidth / bytes_per_step
