"""GPU parity of fp8kv_paged_prefill: prefill / chunked-prefill rows against the oracle's
prefill (each row a causal decode over its prefix), over head geometries, both cache
dtypes, windows, degenerate chunks, per-head scales, and at long context on sampled rows."""
import numpy as np
import pytest

import synthetic as syn
from gpu_util import (E4M3, BF16, assert_close, dev_caches, gpu_prefill, gpu_write,
                      oracle_prefill, oracle_write, say)

pytestmark = pytest.mark.gpu

LENS, CHUNKS = [37, 300, 1027, 16, 5, 40], [37, 64, 200, 1, 5, 0]


def _mk(Hq, Hkv, D, lens, chunks, cid, cache=syn.E4M3, window=0):
    w = syn.make_workload(f"pf-{Hq}-{Hkv}-{D}-{cache}-w{window}", cid, num_q_heads=Hq,
                          num_kv_heads=Hkv, head_dim=D, context_lens=lens, outlier_frac=0.01,
                          layers=(("l0", window, cache),))
    return w, syn.prefill_queries(w, chunks, cid)


MAX_FULL_PAIRS = 3000   # beyond this many (row, head) pairs the oracle runs on a sample


def _sample_pairs(w, pq, seed):
    """Every row for the first and the last query head (all tiles, all tails), and every
    head for the first, the last and three random rows of each sequence."""
    rng = np.random.default_rng(seed)
    Hq = w.num_q_heads
    pairs = {(r, hq) for r in range(pq.num_tokens) for hq in (0, Hq - 1)}
    for b in range(w.num_seqs):
        a, e = int(pq.query_start_loc[b]), int(pq.query_start_loc[b + 1])
        if e > a:
            for r in {a, e - 1, *rng.integers(a, e, 3).tolist()}:
                pairs |= {(r, hq) for hq in range(Hq)}
    return np.array(sorted(pairs), np.int32)


def _check(w, pq, out_f32=False, heads=None, pairs=None, context_lens=None, max_query_len=None):
    layer = w.layers[0]
    if pairs is None and pq.num_tokens * w.num_q_heads > MAX_FULL_PAIRS:
        pairs = _sample_pairs(w, pq, 170)
    cdt = E4M3 if layer.cache_dtype == syn.E4M3 else BF16
    kc, vc = dev_caches(w, cdt)
    gpu_write(w, layer, kc, vc, heads=heads)
    okc, ovc = oracle_write(w, layer, heads=heads)
    got = gpu_prefill(w, layer, kc, vc, pq, out_f32=out_f32, heads=heads,
                      context_lens=context_lens, max_query_len=max_query_len)
    ref = oracle_prefill(w, layer, okc, ovc, pq, pairs=pairs, heads=heads,
                         context_lens=context_lens)
    if pairs is not None:
        got = got[pairs[:, 0], pairs[:, 1]]
    tol = dict(atol=2e-4, rtol=2e-3) if out_f32 else {}
    assert_close(got, ref, what=w.name, **tol)
    return got, ref


SHAPES = [(4, 1, 64), (32, 8, 128), (64, 8, 128), (12, 2, 128), (64, 8, 64), (8, 1, 256),
          (16, 1, 256)]


@pytest.mark.parametrize("cache", [syn.E4M3, syn.BF16])
@pytest.mark.parametrize("Hq,Hkv,D", SHAPES)
def test_prefill_matches_oracle(Hq, Hkv, D, cache):
    w, pq = _mk(Hq, Hkv, D, LENS, CHUNKS, cid=150 + Hq + D, cache=cache)
    say(f"prefill {w.name}")
    _check(w, pq)


def test_prefill_f32_output():
    w, pq = _mk(32, 8, 128, [700, 2049, 90], [700, 333, 17], cid=160)
    say(f"prefill f32 {w.name}")
    _check(w, pq, out_f32=True)


@pytest.mark.parametrize("window", [1, 17, 128, 512])
def test_prefill_windows(window):
    w, pq = _mk(64, 8, 64, [1, 20, 200, 1100], [1, 20, 150, 300], cid=161, window=window)
    say(f"prefill window={window}")
    _check(w, pq)


def test_prefill_degenerate_chunks():
    """Chunks longer than the context (rows before position 0 are zero), a larger
    max_query_len than needed, and sequences without rows."""
    w, pq = _mk(32, 8, 128, [20, 5, 64, 3], [0, 12, 64, 0], cid=162)
    say("prefill degenerate chunks")
    got, ref = _check(w, pq, max_query_len=100)
    assert not got[:7].any()              # sequence 1: 12 rows over 5 positions


def test_prefill_per_head_scales():
    w, pq = _mk(32, 8, 128, [37, 600, 1027], [37, 100, 64], cid=163)
    w, scales = syn.with_head_magnitudes(w, 163)
    say(f"prefill per-head {w.name}")
    _check(w, pq, heads=scales[0])


def test_prefill_long_context_sampled():
    """A 256-token chunk at the end of a 131072-token context (the 8B attention shape):
    sampled rows of every query head against the oracle, f32 output."""
    w = syn.llama8b_long(131072, "amax")
    pq = syn.prefill_queries(w, [256], 164)
    rng = np.random.default_rng(164)
    rows = np.unique(np.concatenate([[0, 255], rng.integers(0, 256, 6)]))
    pairs = np.array([(r, hq) for r in rows for hq in (0, 5, 17, 31)], np.int32)
    say(f"prefill long {w.name}")
    _check(w, pq, out_f32=True, pairs=pairs)


def test_full_prefill_8b_sampled():
    """Whole-prompt prefill of 8192 tokens (the 8B shape) in one call: sampled rows."""
    w = syn.llama8b_long(8192, "amax")
    pq = syn.prefill_queries(w, [8192], 165)
    rng = np.random.default_rng(165)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 127, 8191], rng.integers(0, 8192, 10)]))
    pairs = np.array([(r, hq) for r in rows for hq in (0, 3, 4, 31)], np.int32)
    say(f"prefill full {w.name}")
    _check(w, pq, pairs=pairs)
