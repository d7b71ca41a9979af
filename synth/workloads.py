"""Synthetic workloads: model shapes, seeds and input recipes (no method arithmetic).

Shapes follow the tiny and the full-size synthetic parallel-transformer MoE
decoders; the full-size one is an invented shape of about 30B total / 3.3B
active parameters, standing in for the model the pages describe (30B total,
3.3B active per token, BF16; agenticcommons.xyz "Cohere North Mini Code
megakernel serving engine", section 為什麼 decode 慢).  Trained weights and the
pages' serving benchmarks are not used; every input here is seeded noise.

Recipe (seeds): weights N(0, 0.02) seed 0; KV prefixes N(0, 1) seed 1; start
tokens seed 2; context lengths seed 3; page shuffle seed 4; skew permutation
seed 5; arrivals seed 6; output lengths seed 7.  RMSNorm gains are 1.0, or, for shapes with
gain_sigma > 0 (parity cases that exercise the gains), BF16(1 + z) with z ~ N(0, gain_sigma) drawn per
layer and for the final norm (seed 0).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

from . import synth

SEED_W, SEED_KV, SEED_TOK, SEED_LEN, SEED_PAGES, SEED_PERM, SEED_ARRIVE, SEED_OUTLEN = range(8)
W_SIGMA = 0.02
KV_SIGMA = 1.0
PAGE = 16


@dataclass(frozen=True)
class Shape:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    d_head: int
    n_experts: int
    top_k: int
    d_ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    page_size: int = PAGE
    gain_sigma: float = 0.0  # RMSNorm gains: 1.0 when 0, else BF16(1 + N(0, gain_sigma)) per layer and final norm

    @property
    def qkv_rows(self):
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.d_head

    def layer_attn_bytes(self):
        d, dh = self.d_model, self.d_head
        return 2 * (self.qkv_rows * d + d * self.n_q_heads * dh)

    def router_bytes(self):
        return 2 * self.n_experts * self.d_model

    def expert_bytes(self):
        return 2 * 3 * self.d_ffn * self.d_model

    def kv_bytes_per_pos_layer(self):
        return 2 * 2 * self.n_kv_heads * self.d_head

    def with_layers(self, n):
        from dataclasses import replace

        return replace(self, n_layers=n)


TINY = Shape(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, d_head=64, n_experts=8, top_k=2, d_ffn=512, vocab=4096)
FULL = Shape(n_layers=48, d_model=2048, n_q_heads=32, n_kv_heads=4, d_head=128, n_experts=128, top_k=8, d_ffn=768, vocab=262144)
# One GPU's share of FULL under 2-way tensor parallelism (half the query and KV heads, half of every expert's
# d_ffn, half the vocabulary; d_model, layers, experts and top-k unchanged): the kernel a GPU would run between
# the per-layer exchanges.  Its synthetic weights come from the same generator (same distributions), drawn for
# this shape.
TP2 = Shape(n_layers=48, d_model=2048, n_q_heads=16, n_kv_heads=2, d_head=128, n_experts=128, top_k=8, d_ffn=384, vocab=131072)
GAIN_SIGMA = 0.1


@dataclass
class Workload:
    name: str
    shape: Shape
    ctx: list            # prior positions per sequence at step 0
    steps: int
    shuffle_pages: bool = False
    router_bias: np.ndarray | None = None
    extra_pages: int = 0  # spare pages in the pool
    tokens: list = field(default_factory=list)

    @property
    def B(self):
        return len(self.ctx)


def start_tokens(shape: Shape, B: int):
    return [synth.token(SEED_TOK, b, shape.vocab) for b in range(B)]


def make(name: str, steps: int | None = None) -> Workload:
    """The named workloads: tiny, tiny_ragged, tiny_long, b1_8k, b8_ragged_uniform, b8_ragged_skewed, long_64k, long_128k, long_256k,
    tp2_b1_8k (b1_8k on one GPU's share of the model under 2-way tensor parallelism); a name ending in "_gains"
    is the same workload with non-unit RMSNorm gains."""
    if name.endswith("_gains"):
        w = make(name[:-len("_gains")], steps)
        w.name = name
        w.shape = replace(w.shape, gain_sigma=GAIN_SIGMA)
        return w
    if name == "tiny":
        w = Workload(name, TINY, [128], 16 if steps is None else steps, extra_pages=2)
    elif name == "tiny_long":  # enough positions for the planner's merge tasks (43 splits of 384 per KV group)
        w = Workload(name, TINY, [16384], 4 if steps is None else steps, extra_pages=2)
    elif name == "tiny_ragged":
        w = Workload(name, TINY, [int(v) for v in synth.loguniform_ints(SEED_LEN, 0, 8, 16, 512)], 16 if steps is None else steps,
                     shuffle_pages=True, extra_pages=3)
    elif name == "b1_8k":
        w = Workload(name, FULL, [8192], 128 if steps is None else steps)
    elif name == "tp2_b1_8k":
        w = Workload(name, TP2, [8192], 128 if steps is None else steps)
    elif name in ("b8_ragged_uniform", "b8_ragged_skewed"):
        ctx = [int(v) for v in synth.loguniform_ints(SEED_LEN, 0, 8, 1024, 32768)]
        bias = synth.skew_bias(SEED_PERM, FULL.n_experts, 1.5) if name.endswith("skewed") else None
        w = Workload(name, FULL, ctx, 128 if steps is None else steps, shuffle_pages=True, router_bias=bias)
    elif name.startswith("long_"):
        n = {"long_64k": 65536, "long_128k": 131072, "long_256k": 262144}[name]
        w = Workload(name, FULL, [n], 32 if steps is None else steps)
    else:
        raise KeyError(name)
    w.tokens = start_tokens(w.shape, w.B)
    return w


def page_tables(w: Workload):
    """Per-sequence page lists with room for ctx + steps + 1 positions; identity or seeded-shuffled pool."""
    need = [-(-(c + w.steps + 1) // PAGE) for c in w.ctx]
    n_pages = sum(need) + w.extra_pages
    pool = synth.permutation(SEED_PAGES, 0, n_pages) if w.shuffle_pages else np.arange(n_pages, dtype=np.int32)
    max_pages = max(need)
    pt = np.full((w.B, max_pages), -1, np.int32)
    o = 0
    for b, n in enumerate(need):
        pt[b, :n] = pool[o:o + n]
        o += n
    return pt, n_pages


# ---- host-side weights (for the oracle) -------------------------------------------------

def host_matrix(kind: int, layer: int, rows: int, cols: int, index0: int = 0) -> np.ndarray:
    return synth.fill_bf16_host(rows * cols, SEED_W, synth.weight_stream(kind, layer), index0, W_SIGMA).reshape(rows, cols)


def host_expert(shape: Shape, layer: int, e: int):
    F, d = shape.d_ffn, shape.d_model
    wg = host_matrix(synth.WGATE, layer, F, d, e * F * d)
    wu = host_matrix(synth.WUP, layer, F, d, e * F * d)
    wd = host_matrix(synth.WDOWN, layer, d, F, e * d * F)
    return wg, wu, wd


ONE_BF16 = np.uint16(0x3F80)


def host_norm(shape: Shape, layer: int) -> np.ndarray:
    """RMSNorm gain of layer `layer` (layer == n_layers: the final norm) as BF16 bit patterns: 1.0, or
    BF16(1 + z) with z the generator's BF16 N(0, gain_sigma) value, the sum taken in fp32 and rounded to
    nearest even."""
    d = shape.d_model
    if not shape.gain_sigma:
        return np.full(d, ONE_BF16, np.uint16)
    z = synth.fill_bf16_host(d, SEED_W, synth.weight_stream(synth.NORM, layer), 0, shape.gain_sigma)
    g = (z.astype(np.uint32) << 16).view(np.float32) + np.float32(1.0)
    u = g.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def host_layer(shape: Shape, layer: int):
    """Dense (non-expert) weights of one layer as uint16 arrays."""
    d, dh = shape.d_model, shape.d_head
    return dict(
        attn_norm=host_norm(shape, layer),
        wq=host_matrix(synth.WQ, layer, shape.n_q_heads * dh, d),
        wk=host_matrix(synth.WK, layer, shape.n_kv_heads * dh, d),
        wv=host_matrix(synth.WV, layer, shape.n_kv_heads * dh, d),
        wo=host_matrix(synth.WO, layer, d, shape.n_q_heads * dh),
        w_router=host_matrix(synth.WROUTER, layer, shape.n_experts, d),
    )


def host_embed(shape: Shape):
    return host_matrix(synth.EMBED, 0, shape.vocab, shape.d_model)


def host_embed_rows(shape: Shape, tokens):
    return np.stack([host_matrix(synth.EMBED, 0, 1, shape.d_model, int(t) * shape.d_model)[0] for t in tokens])


def host_lm_head(shape: Shape):
    return host_matrix(synth.LM_HEAD, 0, shape.vocab, shape.d_model)


def host_kv(w: Workload, pt: np.ndarray, n_pages: int, layer0: int = 0, n_layers: int | None = None):
    s = w.shape
    nl = s.n_layers if n_layers is None else n_layers
    kv = np.zeros((nl, n_pages, 2, s.n_kv_heads, PAGE, s.d_head), np.uint16)
    for b, c in enumerate(w.ctx):
        synth.fill_kv_host(kv, layer0, s.n_kv_heads, s.d_head, PAGE, pt[b], b, 0, c, SEED_KV, KV_SIGMA)
    return kv


# ---- device-side model (for the GPU path) ------------------------------------------------

class DeviceModel:
    """Synthetic weights materialised in HBM as BF16 torch tensors, one block per tensor kind:
    wq [L][Hq*dh][d], wk/wv [L][Hkv*dh][d], wo [L][d][Hq*dh], w_router [L][E][d],
    w_gate/w_up [L][E][F][d], w_down [L][E][d][F], attn_norm [L][d], embed/lm_head [V][d], final_norm [d].
    Values equal host_matrix(...) element for element."""

    def __init__(self, shape: Shape, device="cuda"):
        import torch

        s = shape
        self.shape = s
        L, d, dh, E, F, V = s.n_layers, s.d_model, s.d_head, s.n_experts, s.d_ffn, s.vocab
        bf = torch.bfloat16
        mk = lambda *sz: torch.empty(*sz, dtype=bf, device=device)  # noqa: E731
        self.embed = mk(V, d)
        self.lm_head = mk(V, d)
        self.final_norm = torch.ones(d, dtype=bf, device=device)
        self.attn_norm = torch.ones(L, d, dtype=bf, device=device)
        if s.gain_sigma:
            def up(a):
                return torch.from_numpy(a.view(np.int16)).to(device).view(bf)

            self.final_norm.copy_(up(host_norm(s, L)))
            for l in range(L):
                self.attn_norm[l].copy_(up(host_norm(s, l)))
        self.wq = mk(L, s.n_q_heads * dh, d)
        self.wk = mk(L, s.n_kv_heads * dh, d)
        self.wv = mk(L, s.n_kv_heads * dh, d)
        self.wo = mk(L, d, s.n_q_heads * dh)
        self.w_router = mk(L, E, d)
        self.w_gate = mk(L, E, F, d)
        self.w_up = mk(L, E, F, d)
        self.w_down = mk(L, E, d, F)
        synth.fill_bf16_dev(self.embed, SEED_W, synth.weight_stream(synth.EMBED, 0), 0, W_SIGMA)
        synth.fill_bf16_dev(self.lm_head, SEED_W, synth.weight_stream(synth.LM_HEAD, 0), 0, W_SIGMA)
        for l in range(L):
            for t, kind in ((self.wq, synth.WQ), (self.wk, synth.WK), (self.wv, synth.WV), (self.wo, synth.WO),
                            (self.w_router, synth.WROUTER), (self.w_gate, synth.WGATE), (self.w_up, synth.WUP),
                            (self.w_down, synth.WDOWN)):
                synth.fill_bf16_dev(t[l], SEED_W, synth.weight_stream(kind, l), 0, W_SIGMA)

    def nbytes(self):
        return sum(t.numel() * 2 for t in (self.embed, self.lm_head, self.final_norm, self.attn_norm, self.wq, self.wk, self.wv,
                                           self.wo, self.w_router, self.w_gate, self.w_up, self.w_down))


class DeviceKV:
    """Paged KV cache in HBM: BF16 [L][n_pages][2][Hkv][16][dh], with the workload's page tables and prefixes."""

    def __init__(self, w: Workload, device="cuda", pt=None, n_pages=None):
        import torch

        s = w.shape
        if pt is None:
            pt, n_pages = page_tables(w)
        self.pt_host = pt
        self.n_pages = n_pages
        self.kv = torch.zeros(s.n_layers, n_pages, 2, s.n_kv_heads, PAGE, s.d_head, dtype=torch.bfloat16, device=device)
        self.pt = torch.from_numpy(pt).to(device)
        bad = torch.zeros(1, dtype=torch.int32, device=device)
        for b, c in enumerate(w.ctx):
            synth.fill_kv_dev(self.kv, s.n_layers, 0, n_pages, s.n_kv_heads, s.d_head, PAGE, self.pt[b], b, 0, c, SEED_KV, KV_SIGMA,
                              bad=bad)
        if int(bad.item()) != 0:
            raise RuntimeError("KV fill hit an invalid page")
