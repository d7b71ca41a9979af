"""GPU parity of chunked prefill and mixed prefill + decode steps (mk_mixed_step) against the oracle.

A prompt of P tokens is run as steps of up to 8 entries that are consecutive positions of one sequence
(first_of maps each entry to its chunk's first entry); each entry attends causally to the cache below the
chunk and to the chunk's tokens up to itself, and writes its own K/V slot.  The oracle runs the same batch
in order with the entries sharing the sequence's page-table row, which is causal by construction (pinned
in test_oracle_prefill).  After the prompt, the sequence decodes greedily with mk_decode_step.  Same bar as
the decode tests: logits relative L2 <= 1e-2 for every entry of every step, greedy tokens equal unless the
oracle's top-2 gap is below 1e-2, routing identical except at oracle near-ties, integer work bit-exact
(selection, slot table, page walks, counters), the KV cache written equal to the oracle's up to BF16
rounding (gpu_checks.kv_layers_close: from an empty cache the first tokens attend over a few positions, so
one rounding flip of a V element reaches the next layer's input undamped).
"""
import numpy as np
import pytest
import torch

from gpu_checks import check_step, kv_layers_close
from oracle_runner import OracleRun, rel_l2, top2_gap
from synth import synth
from synth import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("cuda")]

LOGIT_TOL = 1e-2
TOKEN_GAP = 1e-2
CHUNK = 8


class Seqs:
    """Sequences with seeded prefixes in one paged KV pool on the device, their page-table rows, a handle, and
    the oracle over the same pool."""

    def __init__(self, shape, prefixes, room, model=None, flags=0):
        from decode_megakernel_wg_amd import mk

        self.shape = s = shape
        need = [-(-(p + room) // 16) for p in prefixes]
        self.n_pages = sum(need) + 2
        perm = synth.permutation(W.SEED_PAGES, 1, self.n_pages)
        self.max_pages = max(need)
        self.rows = np.full((len(prefixes), self.max_pages), -1, np.int32)
        o = 0
        for i, n in enumerate(need):
            self.rows[i, :n] = perm[o:o + n]
            o += n
        self.model = model if model is not None else W.DeviceModel(s)
        m = self.model
        self.kv = torch.zeros(s.n_layers, self.n_pages, 2, s.n_kv_heads, 16, s.d_head, dtype=torch.bfloat16, device="cuda")
        for i, p in enumerate(prefixes):
            synth.fill_kv_dev(self.kv, s.n_layers, 0, self.n_pages, s.n_kv_heads, s.d_head, 16,
                              torch.from_numpy(self.rows[i]).cuda(), i, 0, p, W.SEED_KV, W.KV_SIGMA)
        weights = dict(embed=m.embed, lm_head=m.lm_head, final_norm=m.final_norm, attn_norm=m.attn_norm, wq=m.wq, wk=m.wk, wv=m.wv,
                       wo=m.wo, w_router=m.w_router, w_gate=m.w_gate, w_up=m.w_up, w_down=m.w_down)
        self.desc = mk.make_desc(s, 8, self.max_pages, self.n_pages)
        self.h = mk.Model(self.desc, weights)
        self.h.mk_debug_set(mk.MK_DBG_PAGE_WALK | mk.MK_DBG_COUNT_TASKS | flags)
        self.own_list = bool(flags & mk.MK_DBG_MERGE_TASKS)  # the handle's list differs from mk_plan_tasks'
        self.logits = torch.empty(8, s.vocab, dtype=torch.float32, device="cuda")
        self.orc = OracleRun(W.Workload("prefill", s, list(prefixes), 1), self.rows, self.n_pages)
        self.worst = 0.0
        self.agree = self.total = 0

    def step(self, entries, tokens):
        """One step over entries [(sequence, position)], consecutive entries of one sequence forming a chunk;
        checked against the oracle.  Returns the GPU's greedy tokens."""
        from decode_megakernel_wg_amd import mk

        s = self.shape
        B = len(entries)
        lens = np.array([p for _, p in entries], np.int32)
        first = np.arange(B, dtype=np.int32)
        for b in range(1, B):
            if entries[b - 1][0] == entries[b][0]:
                first[b] = first[b - 1]
        rows = self.rows[[q for q, _ in entries]]
        chunked = (first != np.arange(B)).any()
        tasks = self.h.mk_build_tasks(lens, want_tasks=self.own_list, first_of=first if chunked else None)
        self.last_tasks = tasks
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa: E731
        tok_d, len_d, first_d, rows_d = dev(tokens), dev(lens), dev(first), dev(rows)
        if chunked:
            self.h.mk_mixed_step(tok_d, len_d, first_d, rows_d, self.kv, self.logits)
        else:
            self.h.mk_decode_step(tok_d, len_d, rows_d, self.kv, self.logits)
        self.h.mk_status()
        logits = self.logits[:B].cpu().numpy()
        nxt = mk.read_device(self.h.mk_next_tokens(), 4 * B)
        check_step(self.h, s, self.desc, rows, lens, first_of=first if chunked else None,
                   tasks=tasks if self.own_list else None)
        gsel = self.h.mk_debug_read(mk.MK_DBGK_ROUTE_SEL, (s.n_layers, B, s.top_k), np.int32)
        self.orc.pt = rows
        ol, onx, _, _ = self.orc.step(list(tokens), lens.astype(np.int64), gpu_sel=gsel)
        for b in range(B):
            e = rel_l2(logits[b], ol[b])
            self.worst = max(self.worst, e)
            assert e <= LOGIT_TOL, f"entry {b} {entries[b]}: logits rel L2 {e:.3e}"
            assert nxt[b] == int(np.argmax(logits[b]))
            self.total += 1
            if nxt[b] == onx[b]:
                self.agree += 1
            else:
                assert top2_gap(ol[b]) < TOKEN_GAP, f"entry {b}: token {nxt[b]} vs oracle {onx[b]}"
        return [int(t) for t in nxt]

    def check_kv(self):
        from oracle import oracle as O

        kv_gpu = self.kv.view(torch.int16).cpu().numpy().view(np.uint16)
        kv_layers_close(O.bf16_to_f32(kv_gpu), O.bf16_to_f32(self.orc.kv), "prefill")
        assert (kv_gpu == self.orc.kv).mean() > 0.95

    def finish(self):
        assert self.agree >= 0.99 * self.total
        assert self.orc.near_ties <= max(1, 0.01 * self.orc.route_checked)


def prompt(n, seed0=1000, vocab=4096):
    return [synth.token(W.SEED_TOK, seed0 + i, vocab) for i in range(n)]


@pytest.mark.parametrize("prefix", [0, 40])
def test_prefill_64_then_decode_16(prefix):
    """Tiny model: a 64-token prompt in eight 8-token chunk steps (from an empty cache, or after a 40-position
    prefix that ends mid-page), then 16 greedy decode steps of the same sequence."""
    P, n_dec = 64, 16
    sq = Seqs(W.TINY, [prefix], P + n_dec + 1)
    toks = prompt(P)
    nxt = None
    for c in range(0, P, CHUNK):
        nxt = sq.step([(0, prefix + c + i) for i in range(CHUNK)], toks[c:c + CHUNK])
    tok = nxt[-1]
    for i in range(n_dec):
        tok = sq.step([(0, prefix + P + i)], [tok])[0]
    sq.check_kv()
    sq.finish()
    print(f"prefill 64 + decode 16 after {prefix}: worst logits rel L2 {sq.worst:.2e}")


def test_mixed_prefill_and_decode_batch():
    """Tiny model: one step whose batch holds a 5-token prompt chunk of one sequence and decode tokens of three
    others (ragged contexts), then a step with a 3-token chunk at the front and two chunks of 2 behind it."""
    sq = Seqs(W.TINY, [30, 200, 17, 77], 16)
    toks = prompt(5) + prompt(3, 2000)
    sq.step([(0, 30), (0, 31), (0, 32), (0, 33), (0, 34), (1, 200), (2, 17), (3, 77)], toks)
    sq.step([(1, 201), (1, 202), (1, 203), (0, 35), (0, 36), (3, 78), (3, 79), (2, 18)], prompt(8, 3000))
    sq.check_kv()
    sq.finish()


def test_mixed_full_size():
    """Full-size model (d_head 128, the wave-independent attention): a 4-token prompt chunk of one sequence
    together with decode tokens of four others, then the chunk's sequence decodes one token."""
    sq = Seqs(W.FULL, [1000, 5000, 300, 2000, 9000], 8)
    nxt = sq.step([(0, 1000), (0, 1001), (0, 1002), (0, 1003), (1, 5000), (2, 300), (3, 2000), (4, 9000)],
                  prompt(8, 4000, W.FULL.vocab))
    sq.step([(0, 1004)], [nxt[3]])
    sq.finish()
    print(f"mixed full size: worst logits rel L2 {sq.worst:.2e}")


def test_mixed_prefill_merge_tasks():
    """Tiny model: an 8-token prompt chunk after a 2000-position prefix, with the splits of every entry merged by
    merge tasks (MK_DBG_MERGE_TASKS: a chunk's entries share a layer's split budget, so a chunk alone never
    reaches the planner's 33 splits), then two decode steps of the same sequence."""
    from decode_megakernel_wg_amd import mk

    sq = Seqs(W.TINY, [2000], 16, flags=mk.MK_DBG_MERGE_TASKS)
    nxt = sq.step([(0, 2000 + i) for i in range(CHUNK)], prompt(CHUNK, 5000))
    assert (sq.last_tasks[:, 0] == 8).sum() == W.TINY.n_layers * W.TINY.n_kv_heads * CHUNK * 2
    tok = nxt[-1]
    for i in range(2):
        tok = sq.step([(0, 2000 + CHUNK + i)], [tok])[0]
    sq.check_kv()
    sq.finish()
    print(f"prefill with merge tasks: worst logits rel L2 {sq.worst:.2e}")
