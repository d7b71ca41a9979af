"""A decode session over the C ABI: synthetic model and KV cache in HBM, step loop on one stream.

Used by the tests, smoke() and bench.py.  PyTorch only allocates device memory and
provides the stream; every step of the decode path runs in the persistent kernel.
The greedy loop keeps everything on the device: step s reads the tokens that step
s-1's argmax wrote (mk_next_tokens) and its lengths from a preset row of
lengths, so the timed loop is one kernel launch per step.
"""
from __future__ import annotations

import numpy as np
import torch

from synth import workloads as W

from . import mk


class Session:
    def __init__(self, w: W.Workload, model: W.DeviceModel | None = None, device="cuda", pt=None, n_pages=None, kv=None,
                 max_steps=None):
        self.w = w
        self.shape = s = w.shape
        self.dev = torch.device(device)
        self.model = model if model is not None else W.DeviceModel(s, device)
        self.kvc = kv if kv is not None else W.DeviceKV(w, device, pt=pt, n_pages=n_pages)
        self.B = w.B
        m = self.model
        weights = dict(embed=m.embed, lm_head=m.lm_head, final_norm=m.final_norm, attn_norm=m.attn_norm, wq=m.wq, wk=m.wk, wv=m.wv,
                       wo=m.wo, w_router=m.w_router, w_gate=m.w_gate, w_up=m.w_up, w_down=m.w_down)
        self.desc = mk.make_desc(s, self.B, self.kvc.pt_host.shape[1], self.kvc.n_pages, w.router_bias)
        self.h = mk.Model(self.desc, weights)
        n = (w.steps if max_steps is None else max_steps) + 1
        ctx = np.array(w.ctx, np.int32)
        self.seq_rows_host = ctx[None, :] + np.arange(n, dtype=np.int32)[:, None]   # lengths at step s
        self.seq_rows = torch.from_numpy(self.seq_rows_host.copy()).to(self.dev)
        self.tokens0 = torch.tensor(w.tokens, dtype=torch.int32, device=self.dev)
        self.logits = torch.empty(self.B, s.vocab, dtype=torch.float32, device=self.dev)
        self.next_ptr = self.h.mk_next_tokens()
        self.s = 0
        self.h.mk_build_tasks(self.seq_rows_host[0])

    def step(self, rebuild=False, stream=None, tokens=None):
        """Enqueue decode step self.s (asynchronous); the first step reads the start tokens, later steps the
        previous step's greedy tokens."""
        if rebuild:
            self.h.mk_build_tasks(self.seq_rows_host[self.s])
        tok = tokens if tokens is not None else (self.tokens0 if self.s == 0 else self.next_ptr)
        self.h.mk_decode_step(tok, self.seq_rows[self.s], self.kvc.pt, self.kvc.kv, self.logits, stream)
        self.s += 1

    def rewind(self, s=0):
        self.s = s

    def next_tokens(self):
        torch.cuda.synchronize(self.dev)
        return mk.read_device(self.next_ptr, 4 * self.B)

    def status(self):
        return self.h.mk_status()
