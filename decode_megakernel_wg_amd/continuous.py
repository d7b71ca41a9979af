"""Continuous batching over the C ABI: the live batch changes from step to step.

Per decode step: the prefixes of newly admitted sequences are written into their pages (untimed: it stands
for the prefill this path does not cover), the live batch's task list is rebuilt on the host
(mk_build_tasks), the step's tokens, lengths and page tables go to the device in one copy, one
mk_decode_step runs, and the greedy tokens come back to the host, where they become the next step's
inputs of the sequences that continue.  The schedule (arrivals, lengths, pages from a LIFO free list) is
synth.continuous's.  PyTorch only allocates memory and provides the stream.
"""
from __future__ import annotations

import ctypes as C
import time

import numpy as np
import torch

from synth import continuous as CB
from synth import synth
from synth import workloads as W

from . import mk


class ContinuousSession:
    def __init__(self, shape: W.Shape, n_steps: int, model: W.DeviceModel | None = None, device="cuda", lo=CB.PREFIX_LO,
                 hi=CB.PREFIX_HI, n_pages=None, router_bias=None, mean_gap=CB.MEAN_GAP):
        self.shape = s = shape
        self.dev = torch.device(device)
        self.steps, self.seqs, self.n_pages, self.max_pages = CB.schedule(n_steps, n_pages, lo, hi, mean_gap=mean_gap)
        self.model = model if model is not None else W.DeviceModel(s, device)
        m = self.model
        self.kv = torch.zeros(s.n_layers, self.n_pages, 2, s.n_kv_heads, W.PAGE, s.d_head, dtype=torch.bfloat16, device=self.dev)
        weights = dict(embed=m.embed, lm_head=m.lm_head, final_norm=m.final_norm, attn_norm=m.attn_norm, wq=m.wq, wk=m.wk, wv=m.wv,
                       wo=m.wo, w_router=m.w_router, w_gate=m.w_gate, w_up=m.w_up, w_down=m.w_down)
        self.desc = mk.make_desc(s, CB.MAX_BATCH, self.max_pages, self.n_pages, router_bias)
        self.h = mk.Model(self.desc, weights)
        self.logits = torch.empty(CB.MAX_BATCH, s.vocab, dtype=torch.float32, device=self.dev)
        self.next_ptr = self.h.mk_next_tokens()
        # one pinned staging block per step: tokens [8], lengths [8], page tables [8][max_pages]
        nw = 2 * CB.MAX_BATCH + CB.MAX_BATCH * self.max_pages
        self.h_in = torch.empty(nw, dtype=torch.int32, pin_memory=True)
        self.d_in = torch.empty(nw, dtype=torch.int32, device=self.dev)
        self._bad = torch.zeros(1, dtype=torch.int32, device=self.dev)
        self.reset()

    def reset(self):
        """Back to step 0 (the prefixes are written again as sequences are admitted)."""
        self.t = 0
        self.last_tok = {}

    def admit(self, st: CB.Step):
        s = self.shape
        for sid in st.admitted:
            q = self.seqs[sid]
            pt = torch.tensor(q.pages, dtype=torch.int32, device=self.dev)
            synth.fill_kv_dev(self.kv, s.n_layers, 0, self.n_pages, s.n_kv_heads, s.d_head, W.PAGE, pt, sid, 0, q.prefix, W.SEED_KV,
                              W.KV_SIGMA, bad=self._bad)

    def tokens_for(self, st: CB.Step):
        return [self.last_tok[sid] if sid in self.last_tok else synth.token(W.SEED_TOK, sid, self.shape.vocab) for sid in st.sids]

    def step(self):
        """Run step self.t.  Returns (sids, tokens fed, positions, next tokens, seconds of the timed part: task
        rebuild + input copy + step + token read-back)."""
        st = self.steps[self.t]
        self.admit(st)
        torch.cuda.synchronize(self.dev)
        B = len(st.sids)
        toks = self.tokens_for(st)
        pt = CB.page_table(st, self.seqs, self.max_pages)
        t0 = time.perf_counter()
        self.h.mk_build_tasks(st.pos)
        hin = self.h_in.numpy()
        hin[:B] = toks
        hin[CB.MAX_BATCH:CB.MAX_BATCH + B] = st.pos
        o = 2 * CB.MAX_BATCH
        hin[o:o + B * self.max_pages] = pt.reshape(-1)
        self.d_in[:o + B * self.max_pages].copy_(self.h_in[:o + B * self.max_pages], non_blocking=True)
        d_tok = self.d_in[:B]
        d_pos = self.d_in[CB.MAX_BATCH:CB.MAX_BATCH + B]
        d_pt = self.d_in[o:o + B * self.max_pages]
        self.h.mk_decode_step(d_tok, d_pos, d_pt, self.kv, self.logits)
        torch.cuda.current_stream(self.dev).synchronize()
        nxt = mk.read_device(self.next_ptr, 4 * B)
        dt = time.perf_counter() - t0
        for b, sid in enumerate(st.sids):
            self.last_tok[sid] = int(nxt[b])
        self.t += 1
        return st.sids, toks, st.pos.copy(), nxt, dt

    def run_pipelined(self, n_steps, kernel_events=False):
        """Enqueue steps self.t .. self.t + n_steps - 1 back to back without waiting for results: the host
        rebuilds step t+1's task list and stages its inputs while the GPU runs step t, and the tokens of
        continuing sequences move device-to-device from the previous step's greedy output.  Admitted
        prefixes are written on the stream between steps and their time is measured separately.  Returns
        (seconds from the first enqueue to the last step's completion, seconds of prefix writes on the GPU,
        seconds of each step's kernel when kernel_events, else None)."""
        stream = torch.cuda.current_stream(self.dev)
        nw = self.h_in.numel()
        if not hasattr(self, "_pipe"):
            self._pipe = dict(h=[torch.empty(nw, dtype=torch.int32, pin_memory=True) for _ in range(2)],
                              d=[torch.empty(nw, dtype=torch.int32, device=self.dev) for _ in range(2)],
                              ev=[torch.cuda.Event() for _ in range(2)])
        P = self._pipe
        fills, kev = [], []
        prev = None
        o = 2 * CB.MAX_BATCH
        tok_bytes = 4
        torch.cuda.synchronize(self.dev)
        t0 = time.perf_counter()
        for i in range(n_steps):
            st = self.steps[self.t]
            if st.admitted:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                self.admit(st)
                e1.record(stream)
                fills.append((e0, e1))
            B = len(st.sids)
            self.h.mk_build_tasks(st.pos)
            k = i % 2
            P["ev"][k].synchronize()  # this staging block's previous copy has been consumed
            hin = P["h"][k].numpy()
            hin[:B] = [synth.token(W.SEED_TOK, sid, self.shape.vocab) for sid in st.sids]  # new sequences' start tokens
            hin[CB.MAX_BATCH:CB.MAX_BATCH + B] = st.pos
            hin[o:o + B * self.max_pages] = CB.page_table(st, self.seqs, self.max_pages).reshape(-1)
            d = P["d"][k]
            d[:o + B * self.max_pages].copy_(P["h"][k][:o + B * self.max_pages], non_blocking=True)
            P["ev"][k].record(stream)
            # continuing sequences: their previous greedy token, copied on the device in runs of consecutive slots
            if prev is not None:
                src = {sid: b for b, sid in enumerate(prev.sids)}
                b = 0
                while b < B:
                    if st.sids[b] not in src:
                        b += 1
                        continue
                    e = b
                    while e + 1 < B and st.sids[e + 1] in src and src[st.sids[e + 1]] == src[st.sids[e]] + 1:
                        e += 1
                    mk._hiprt().hipMemcpyAsync(C.c_void_p(d.data_ptr() + tok_bytes * b),
                                               C.c_void_p(self.next_ptr + tok_bytes * src[st.sids[b]]), tok_bytes * (e - b + 1),
                                               3, C.c_void_p(stream.cuda_stream))  # hipMemcpyDeviceToDevice
                    b = e + 1
            if kernel_events:
                ke = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                ke[0].record(stream)
            self.h.mk_decode_step(d[:B], d[CB.MAX_BATCH:CB.MAX_BATCH + B], d[o:o + B * self.max_pages], self.kv, self.logits, stream)
            if kernel_events:
                ke[1].record(stream)
                kev.append(ke)
            prev = st
            self.t += 1
        torch.cuda.synchronize(self.dev)
        wall = time.perf_counter() - t0
        fill_s = sum(a.elapsed_time(b) for a, b in fills) * 1e-3
        kern = [a.elapsed_time(b) * 1e-3 for a, b in kev] if kernel_events else None
        return wall, fill_s, kern

    def status(self):
        if int(self._bad.item()) != 0:
            raise RuntimeError("KV prefix fill hit an invalid page")
        return self.h.mk_status()
