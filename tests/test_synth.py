"""Pins of the seeded input generator (shared by the oracle's tests and the GPU harness)."""
import math

import numpy as np
import pytest
from scipy.special import ndtr

from synth import synth, workloads as W


def bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_splitmix64_published_sequence():
    # First outputs of SplitMix64 from state 0 (Steele, Lea & Flood 2014; the reference splitmix64.c sequence).
    assert [int(v) for v in synth.splitmix64(0, 3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


@pytest.mark.parametrize("sigma", [0.02, 1.0])
def test_table_is_the_rounded_normal_cdf(sigma):
    t = synth.Table.get(sigma)
    thr = t.thr.astype(np.float64) / 2.0 ** 63
    assert np.all(np.diff(t.thr.astype(np.float64)) >= 0)
    assert t.thr[-1] == np.uint64(1 << 63)
    # independent check with scipy's normal CDF: P(|X| < midpoint(v_k, v_k+1))
    k = np.arange(t.n - 1)
    mid = 0.5 * (bf16_value(k) + bf16_value(k + 1))
    ref = 2.0 * ndtr(mid / sigma) - 1.0
    assert np.max(np.abs(thr[:-1] - ref)) < 1e-12
    # guide table: first index whose threshold exceeds the bucket start
    j = np.arange(0, 1 << 16, 997)
    lo = j.astype(np.float64) * 2.0 ** 47
    for jj, l in zip(j, lo):
        g = int(t.guide[jj])
        assert float(t.thr[g]) > l and (g == 0 or float(t.thr[g - 1]) <= l)


def test_sample_moments_and_histogram():
    a = synth.fill_bf16_host(4_000_000, 0, 12345, 0, 0.02)
    f = bf16_value(a)
    assert abs(f.mean()) < 3 * 0.02 / math.sqrt(len(f))
    assert abs(f.std() / 0.02 - 1) < 2e-3
    # chi-square of the BF16 magnitudes against the exact mass of their rounding intervals (scipy's normal CDF)
    mag = (a & 0x7FFF).astype(np.int64)
    cuts = np.quantile(mag, np.linspace(0, 1, 21)[1:-1]).astype(np.int64)
    counts = np.bincount(np.searchsorted(cuts, mag, side="left"), minlength=20)
    edges = np.concatenate([[-1], cuts, [0x7F7F]])
    upper = lambda k: 0.5 * (bf16_value(k) + bf16_value(k + 1)) if k >= 0 else 0.0  # noqa: E731
    probs = np.array([2 * (ndtr(upper(hi) / 0.02) - ndtr(upper(lo) / 0.02)) for lo, hi in zip(edges[:-1], edges[1:])])
    expect = probs * len(a)
    chi2 = ((counts - expect) ** 2 / expect).sum()
    assert chi2 < 60, chi2


def test_streams_and_indices_are_independent_of_chunking():
    a = synth.fill_bf16_host(1000, 0, synth.weight_stream(synth.WQ, 3), 0)
    b = synth.fill_bf16_host(500, 0, synth.weight_stream(synth.WQ, 3), 500)
    assert np.array_equal(a[500:], b)
    c = synth.fill_bf16_host(1000, 0, synth.weight_stream(synth.WQ, 4), 0)
    assert not np.array_equal(a, c)


def test_kv_values_do_not_depend_on_page_placement():
    s = W.TINY
    n_pages = 12
    ident = np.arange(n_pages, dtype=np.int32)
    shuf = synth.permutation(7, 0, n_pages)
    kv1 = np.zeros((2, n_pages, 2, s.n_kv_heads, 16, s.d_head), np.uint16)
    kv2 = np.zeros_like(kv1)
    synth.fill_kv_host(kv1, 0, s.n_kv_heads, s.d_head, 16, ident, 0, 0, 150, 1)
    synth.fill_kv_host(kv2, 0, s.n_kv_heads, s.d_head, 16, shuf, 0, 0, 150, 1)
    for pos in (0, 15, 16, 149):
        p1, p2 = ident[pos // 16], shuf[pos // 16]
        assert np.array_equal(kv1[:, p1, :, :, pos % 16], kv2[:, p2, :, :, pos % 16])
    # values follow the logical key
    idx = (((1 * synth.KV_POS_SPAN + 37) * 2 + 1) * s.n_kv_heads + 1) * s.d_head
    ref = synth.fill_bf16_host(s.d_head, 1, 0, idx, 1.0)
    assert np.array_equal(kv1[1, ident[37 // 16], 1, 1, 37 % 16], ref)


def test_out_of_range_pages_are_rejected():
    kv = np.zeros((1, 4, 2, 2, 16, 64), np.uint16)
    with pytest.raises(ValueError):
        synth.fill_kv_host(kv, 0, 2, 64, 16, np.array([0, 9], np.int32), 0, 0, 20, 1)


def test_loguniform_and_permutation():
    v = synth.loguniform_ints(3, 0, 20000, 1024, 32768)
    assert v.min() >= 1024 and v.max() <= 32768
    assert abs(v.mean() / ((32768 - 1024) / math.log(32)) - 1) < 0.03
    p = synth.permutation(4, 0, 1000)
    assert sorted(p.tolist()) == list(range(1000))


def test_skew_bias_reading():
    E = 128
    b = synth.skew_bias(5, E, 1.5)
    perm = synth.permutation(5, 0, E)
    for r in (1, 2, 10, 128):
        assert b[perm[r - 1]] == np.float32(-1.5 * math.log(r))
    assert b.max() == 0.0


def test_workload_page_tables():
    w = W.make("tiny_ragged")
    pt, n_pages = W.page_tables(w)
    used = pt[pt >= 0]
    assert len(np.unique(used)) == len(used) and used.max() < n_pages
    for b, c in enumerate(w.ctx):
        assert (pt[b] >= 0).sum() * 16 >= c + w.steps + 1
