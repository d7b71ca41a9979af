"""Drives the CPU oracle over the same synthetic workload the GPU runs, teacher-forced with the GPU's tokens.

Routing near-ties: where the oracle's own top-k differs from the GPU's but the GPU's selection is a top-k
of logits within DELTA_ROUTE of the oracle's (tie_ok: every chosen expert within DELTA_ROUTE of the
oracle's k-th logit, and the chosen order descending up to DELTA_ROUTE), both selections are correct;
the oracle then adopts the GPU's selection for that (layer, token) and counts it ("follow mode").
Anywhere else a routing difference is a failure.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import oracle as O
from synth import workloads as W

DELTA_ROUTE = 1e-3


def dims(shape):
    return O.Dims(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.d_head, shape.n_experts, shape.top_k,
                  shape.d_ffn, shape.vocab, 16, shape.rms_eps, shape.rope_base)


def kth_gap(logits, k):
    s = np.sort(logits.astype(np.float64))[::-1]
    return s[k - 1] - s[k] if k < len(s) else np.inf


def tie_ok(logits, sel, k, delta=DELTA_ROUTE):
    """Whether selection sel (k distinct experts, in rank order) is the top-k of some logits within delta of
    `logits`: each chosen logit at least the k-th largest minus delta, and the chosen order descending up to
    delta (selections of the same logits then differ only in near-ties of membership or of rank)."""
    lg = np.asarray(logits, np.float64)
    g = np.asarray(sel, np.int64)
    if len(set(g.tolist())) != k:
        return False
    kth = np.sort(lg)[::-1][k - 1]
    return bool(np.all(lg[g] >= kth - delta) and np.all(lg[g[1:]] <= lg[g[:-1]] + delta))


class OracleRun:
    """Oracle state (KV cache, per-layer weights) for a workload.  For small models every weight is kept
    in memory; for large ones `layer_source(l)` generates a layer's dense weights on demand and experts
    are generated when selected."""

    def __init__(self, w: W.Workload, pt, n_pages, keep_all=None, lazy_kv=False, keep_kv_layers=()):
        """lazy_kv: generate each layer's cache when the layer runs and drop it afterwards (KV values are keyed
        by logical coordinates, so they do not depend on when they are generated); only the layers listed in
        keep_kv_layers are kept (self.kept[l]), with the step's K/V writes.  For one-step runs of long contexts."""
        self.w = w
        s = self.shape = w.shape
        self.D = dims(s)
        self.pt = pt
        self.n_pages = n_pages
        self.lazy_kv = lazy_kv
        self.keep_kv_layers = set(keep_kv_layers)
        self.kept = {}
        self.kv = None if lazy_kv else W.host_kv(w, pt, n_pages)
        small = s.n_layers * (s.layer_attn_bytes() + s.n_experts * s.expert_bytes()) < 2e9
        self.keep_all = small if keep_all is None else keep_all
        self.final_norm = W.host_norm(s, s.n_layers)
        self.lm_head = W.host_lm_head(s)
        self._layers = {}
        self._experts = {}
        self.bias = w.router_bias
        self.near_ties = 0
        self.route_checked = 0

    def layer_weights(self, l, experts):
        s = self.shape
        if l not in self._layers:
            hl = W.host_layer(s, l)
            if not self.keep_all:
                self._layers.clear()
                self._experts.clear()
            self._layers[l] = hl
        hl = self._layers[l]
        ex = {}
        for e in experts:
            key = (l, int(e))
            if key not in self._experts:
                self._experts[key] = W.host_expert(s, l, int(e))
            ex[int(e)] = self._experts[key]
        return O.LayerWeights(hl["attn_norm"], hl["wq"], hl["wk"], hl["wv"], hl["wo"], hl["w_router"], ex, s.n_experts, self.bias)

    def step(self, tokens, pos, gpu_sel=None):
        """One oracle decode step for tokens at positions pos (prior lengths).  gpu_sel: [L][B][k] GPU selections
        (for the near-tie rule).  Returns logits [B][V], next [B], sel [L][B][k], n [L][B][d]."""
        x, sels, ns = self.layers(tokens, pos, self.shape.n_layers, gpu_sel)
        logits, nxt = O.head(self.D, x, self.final_norm, self.lm_head)
        return logits, nxt, np.stack(sels), np.stack(ns)

    def layers(self, tokens, pos, n_layers, gpu_sel=None):
        """The first n_layers layers of a step: residual stream after them, per-layer selections and
        normalised inputs."""
        s = self.shape
        B = len(tokens)
        x = O.embed(self.D, W.host_embed_rows(s, tokens), np.arange(B, dtype=np.int32))
        sels, ns = [], []
        for l in range(n_layers):
            # own routing first (on this layer's normalised input)
            hl = self.layer_weights(l, [])
            n = np.stack([O.rmsnorm(x[b], hl.arrs[0]) for b in range(B)])
            force = np.full((B, s.top_k), -1, np.int32)
            need = set()
            for b in range(B):
                sel, _, lg = O.router(n[b], hl.arrs[5], s.top_k, self.bias)
                self.route_checked += 1
                if gpu_sel is not None and not np.array_equal(np.asarray(gpu_sel[l][b]), sel):
                    if tie_ok(lg, gpu_sel[l][b], s.top_k):
                        force[b] = gpu_sel[l][b]
                        self.near_ties += 1
                        need.update(int(e) for e in gpu_sel[l][b])
                        continue
                    raise AssertionError(f"routing differs at layer {l} token {b}: gpu {list(gpu_sel[l][b])} oracle {list(sel)} "
                                         f"(k-th gap {kth_gap(lg, s.top_k):.3g}, gpu-chosen logits {lg[np.asarray(gpu_sel[l][b])]})")
                need.update(int(e) for e in sel)
            Wl = self.layer_weights(l, sorted(need))
            if self.lazy_kv:
                kvl = W.host_kv(self.w, self.pt, self.n_pages, layer0=l, n_layers=1)[0]
                if l in self.keep_kv_layers:
                    self.kept[l] = kvl
            else:
                kvl = self.kv[l]
            x, aux = O.layer(self.D, Wl, pos, self.pt, kvl, x, sel_force=force if (force >= 0).any() else None)
            del kvl
            sels.append(aux["sel"])
            ns.append(aux["n"])
            if s.n_layers >= 24 and l % 12 == 11:  # progress of long oracle runs
                print(f"[oracle] layer {l + 1}/{s.n_layers}", file=sys.stderr, flush=True)
        return x, sels, ns


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def top2_gap(logits):
    s = np.sort(np.asarray(logits, np.float64))[-2:]
    return s[1] - s[0]
