"""GPU parity of the Hadamard-rotation entry points: the rotated cache write is bit-exact
against the oracle's rotated write (rotation in f32 in the same butterfly order, then the
same quantiser), and the rotated decode (query rotation, decode, output rotated back)
matches the oracle's rotated decode within the decode tolerance; the fused rotated step writes
the step token's bytes exactly as the rotated write does and decodes within that tolerance."""
import numpy as np
import pytest
import torch

import fp8_kv_cache_reshape_amd as F
import oracle
import synthetic as syn
from gpu_util import (BF16, DEV, E4M3, DeviceInputs, assert_close, dev_caches, host_caches,
                      new_counters, say, step_rows_by_seq, to_host_bits, u16_dev)

pytestmark = pytest.mark.gpu


def _mk(Hq, Hkv, D, lens, cid, cache=syn.E4M3, window=0):
    w = syn.make_workload(f"rot-{Hq}-{Hkv}-{D}-{cache}-w{window}", cid, num_q_heads=Hq,
                          num_kv_heads=Hkv, head_dim=D, context_lens=lens, outlier_frac=0.01,
                          layers=(("l0", window, cache),))
    L = w.layers[0]
    # scales calibrated on the rotated rows (amax / 448), as a caller would
    rk = oracle.hadamard_f32(syn.bf16_bits_to_f32(L.k))
    rv = oracle.hadamard_f32(syn.bf16_bits_to_f32(L.v))
    ks = float(np.float32(np.abs(rk).max()) / np.float32(448.0)) if cache == syn.E4M3 else 1.0
    vs = float(np.float32(np.abs(rv).max()) / np.float32(448.0)) if cache == syn.E4M3 else 1.0
    return w, L, ks, vs


def _write_both(w, L, ks, vs):
    cdt = E4M3 if L.cache_dtype == syn.E4M3 else BF16
    kc, vc = dev_caches(w, cdt)
    slots = torch.from_numpy(w.slot_mapping).to(DEV)
    F.fp8kv_cache_write_rotated(u16_dev(L.k), u16_dev(L.v), kc, vc, cdt, slots, w.num_tokens,
                                w.num_kv_heads, w.head_dim, 16, w.num_blocks, ks, vs)
    torch.cuda.synchronize()
    okc, ovc = host_caches(w, cdt)
    oracle.cache_write_rotated(L.k, L.v, okc, ovc, cdt, w.slot_mapping, w.num_kv_heads, w.head_dim,
                               16, w.num_blocks, ks, vs)
    return cdt, kc, vc, okc, ovc


@pytest.mark.parametrize("cache", [syn.E4M3, syn.BF16])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_rotated_write_bit_exact(D, cache):
    w, L, ks, vs = _mk(2 * 4, 4, D, [37, 300, 1027, 16], cid=180 + D, cache=cache)
    say(f"cache_write_rotated {w.name}")
    cdt, kc, vc, okc, ovc = _write_both(w, L, ks, vs)
    assert np.array_equal(to_host_bits(kc), okc), "key cache bytes differ"
    assert np.array_equal(to_host_bits(vc), ovc), "value cache bytes differ"


def _decode(w, L, ks, vs, kc, vc, cdt, out_f32=False, num_splits=0):
    dev = DeviceInputs(w)
    B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    win = L.sliding_window
    nbytes = F.fp8kv_paged_decode_rotated_workspace_size(B, Hq, Hkv, D, 16, w.max_context_len, win,
                                                        num_splits)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    out = torch.empty(B * Hq * D, dtype=torch.float32 if out_f32 else torch.bfloat16, device=DEV)
    F.fp8kv_paged_decode_rotated(out, F.FP8KV_F32 if out_f32 else F.FP8KV_BF16, dev.q, kc, vc, cdt,
                                 dev.bt, w.max_blocks_per_seq, dev.cl, w.max_context_len, B, Hq, Hkv,
                                 D, 16, w.num_blocks, ks, vs, win, num_splits, ws, nbytes)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64).reshape(B, Hq, D)


def _check_decode(w, L, ks, vs, out_f32=False, num_splits=0):
    cdt, kc, vc, okc, ovc = _write_both(w, L, ks, vs)
    got = _decode(w, L, ks, vs, kc, vc, cdt, out_f32=out_f32, num_splits=num_splits)
    ref = oracle.paged_decode_rotated(w.q, okc, ovc, cdt, w.block_tables, w.context_lens,
                                      w.num_q_heads, w.num_kv_heads, w.head_dim, 16, ks, vs,
                                      L.sliding_window)
    tol = dict(atol=2e-4, rtol=2e-3) if out_f32 else {}
    assert_close(got, ref, what=w.name, **tol)


SHAPES = [(4, 1, 64), (32, 8, 128), (64, 8, 128), (64, 8, 64), (16, 1, 256)]


@pytest.mark.parametrize("cache", [syn.E4M3, syn.BF16])
@pytest.mark.parametrize("Hq,Hkv,D", SHAPES)
def test_rotated_decode_matches_oracle(Hq, Hkv, D, cache):
    w, L, ks, vs = _mk(Hq, Hkv, D, [1, 16, 17, 300, 1027, 0], cid=190 + Hq + D, cache=cache)
    say(f"paged_decode_rotated {w.name}")
    _check_decode(w, L, ks, vs)


@pytest.mark.parametrize("num_splits", [1, 5, 129])
def test_rotated_decode_split_counts(num_splits):
    w, L, ks, vs = _mk(32, 8, 128, [5, 700, 2049, 16], cid=200)
    say(f"paged_decode_rotated splits={num_splits}")
    _check_decode(w, L, ks, vs, out_f32=True, num_splits=num_splits)


@pytest.mark.parametrize("window", [17, 512])
def test_rotated_decode_windows(window):
    w, L, ks, vs = _mk(64, 8, 64, [1, 20, 200, 1100], cid=201, window=window)
    say(f"paged_decode_rotated window={window}")
    _check_decode(w, L, ks, vs)


# ---- the fused rotated step: write the step token rotated + decode + rotate back

def _step(w, L, ks, vs, kc, vc, cdt, out_f32=False, num_splits=0, counters=None):
    dev = DeviceInputs(w)
    B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    win = L.sliding_window
    if counters is None:
        counters = new_counters(B, Hkv)
    nbytes = F.fp8kv_paged_decode_rotated_workspace_size(B, Hq, Hkv, D, 16, w.max_context_len, win,
                                                        num_splits)
    # NaN bytes: every partial and rotated row the step reads must be its own
    ws = torch.full((max(nbytes, 256),), 0xFF, dtype=torch.uint8, device=DEV)
    kn, vn = step_rows_by_seq(w, L)
    kd, vd = u16_dev(kn), u16_dev(vn)
    out = torch.empty(B * Hq * D, dtype=torch.float32 if out_f32 else torch.bfloat16, device=DEV)
    F.fp8kv_decode_step_rotated(out, F.FP8KV_F32 if out_f32 else F.FP8KV_BF16, dev.q, kd, vd, kc, vc,
                                cdt, dev.bt, w.max_blocks_per_seq, dev.cl, w.max_context_len, B, Hq,
                                Hkv, D, 16, w.num_blocks, ks, vs, win, num_splits, counters,
                                counters.numel(), ws, ws.numel())
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64).reshape(B, Hq, D), counters


def _check_step(w, L, ks, vs, out_f32=False, num_splits=0):
    """Context rows written by the rotated cache write, the step token by the rotated step:
    the cache bytes equal the oracle's rotated write of every row, the output matches the
    oracle's rotated decode over that cache, and the counters are back at zero."""
    cdt = E4M3 if L.cache_dtype == syn.E4M3 else BF16
    kc, vc = dev_caches(w, cdt)
    rows = w.prefix_token_rows()
    slots = torch.from_numpy(np.ascontiguousarray(w.slot_mapping[rows])).to(DEV)
    kp, vp = u16_dev(L.k[rows]), u16_dev(L.v[rows])
    F.fp8kv_cache_write_rotated(kp, vp, kc, vc, cdt, slots, len(rows), w.num_kv_heads, w.head_dim,
                                16, w.num_blocks, ks, vs)
    got, cnt = _step(w, L, ks, vs, kc, vc, cdt, out_f32=out_f32, num_splits=num_splits)
    okc, ovc = host_caches(w, cdt)
    oracle.cache_write_rotated(L.k, L.v, okc, ovc, cdt, w.slot_mapping, w.num_kv_heads, w.head_dim,
                               16, w.num_blocks, ks, vs)
    assert np.array_equal(to_host_bits(kc), okc), "key cache bytes differ after the rotated step"
    assert np.array_equal(to_host_bits(vc), ovc), "value cache bytes differ after the rotated step"
    ref = oracle.paged_decode_rotated(w.q, okc, ovc, cdt, w.block_tables, w.context_lens,
                                      w.num_q_heads, w.num_kv_heads, w.head_dim, 16, ks, vs,
                                      L.sliding_window)
    tol = dict(atol=2e-4, rtol=2e-3) if out_f32 else {}
    assert_close(got, ref, what=w.name, **tol)
    assert not cnt.cpu().numpy().any(), "counters were not returned to zero"
    return got


@pytest.mark.parametrize("cache", [syn.E4M3, syn.BF16])
@pytest.mark.parametrize("Hq,Hkv,D", SHAPES + [(8, 1, 256)])
def test_rotated_step_matches_oracle(Hq, Hkv, D, cache):
    w, L, ks, vs = _mk(Hq, Hkv, D, [1, 16, 17, 300, 1027, 0], cid=210 + Hq + D, cache=cache)
    say(f"decode_step_rotated {w.name}")
    _check_step(w, L, ks, vs)


# 1: the kernel writes final rows itself; 64: in-kernel merge over two batches; 129: more
# partials than the in-kernel merge takes, so the merge kernel and the rotate-back launch run
@pytest.mark.parametrize("num_splits", [0, 1, 5, 64, 129])
def test_rotated_step_split_counts(num_splits):
    w, L, ks, vs = _mk(32, 8, 128, [5, 700, 2049, 16], cid=220)
    say(f"decode_step_rotated splits={num_splits}")
    _check_step(w, L, ks, vs, out_f32=True, num_splits=num_splits)


@pytest.mark.parametrize("num_splits", [1, 3, 16, 17])
def test_rotated_step_d256_group8(num_splits):
    w, L, ks, vs = _mk(8, 1, 256, [5, 700, 4100, 16, 1500], cid=221)
    say(f"decode_step_rotated d256 g8 splits={num_splits}")
    _check_step(w, L, ks, vs, out_f32=True, num_splits=num_splits)


@pytest.mark.parametrize("window", [1, 17, 512])
def test_rotated_step_windows(window):
    w, L, ks, vs = _mk(64, 8, 64, [1, 20, 200, 1100], cid=222, window=window)
    say(f"decode_step_rotated window={window}")
    _check_step(w, L, ks, vs)


def test_rotated_step_fixed_splits_reproducible():
    """A fixed split count: two steps over the same cache give the same output, bit for bit."""
    w, L, ks, vs = _mk(32, 8, 128, [3000, 900, 40], cid=223)
    say("decode_step_rotated reproducibility")
    a = _check_step(w, L, ks, vs, out_f32=True, num_splits=7)
    b = _check_step(w, L, ks, vs, out_f32=True, num_splits=7)
    assert np.array_equal(a, b)


# ---- per-kv-head scales on the rotated path

def _head_scales(w, L):
    """Per-kv-head amax / 448 scales of the rotated rows (float32 [Hkv] each)."""
    rk = oracle.hadamard_f32(syn.bf16_bits_to_f32(L.k)).reshape(w.num_tokens, w.num_kv_heads, -1)
    rv = oracle.hadamard_f32(syn.bf16_bits_to_f32(L.v)).reshape(w.num_tokens, w.num_kv_heads, -1)
    ks = (np.abs(rk).max(axis=(0, 2)).astype(np.float32) / np.float32(448.0)).astype(np.float32)
    vs = (np.abs(rv).max(axis=(0, 2)).astype(np.float32) / np.float32(448.0)).astype(np.float32)
    return ks, vs


def _mk_ph(Hq, Hkv, D, lens, cid, window=0):
    # outliers on some heads only, so the per-head scales differ widely
    w = syn.make_workload(f"rotph-{Hq}-{Hkv}-{D}-w{window}", cid, num_q_heads=Hq, num_kv_heads=Hkv,
                          head_dim=D, context_lens=lens, outlier_frac=0.02,
                          layers=(("l0", window, syn.E4M3),))
    L = w.layers[0]
    ks, vs = _head_scales(w, L)
    return w, L, ks, vs


def _write_ph_both(w, L, ks, vs, rows=None):
    kc, vc = dev_caches(w, E4M3)
    rows = np.arange(w.num_tokens) if rows is None else rows
    slots = torch.from_numpy(np.ascontiguousarray(w.slot_mapping[rows])).to(DEV)
    kd, vd = u16_dev(L.k[rows]), u16_dev(L.v[rows])
    ksd, vsd = torch.from_numpy(ks).to(DEV), torch.from_numpy(vs).to(DEV)
    F.fp8kv_cache_write_rotated_per_head(kd, vd, kc, vc, E4M3, slots, len(rows), w.num_kv_heads,
                                         w.head_dim, 16, w.num_blocks, ksd, vsd)
    torch.cuda.synchronize()
    okc, ovc = host_caches(w, E4M3)
    oracle.cache_write_rotated_per_head(L.k, L.v, okc, ovc, E4M3, w.slot_mapping, w.num_kv_heads,
                                        w.head_dim, 16, w.num_blocks, ks, vs)
    return kc, vc, okc, ovc, ksd, vsd


@pytest.mark.parametrize("D", [64, 128, 256])
def test_rotated_per_head_write_bit_exact(D):
    w, L, ks, vs = _mk_ph(4 * 4, 4, D, [37, 300, 1027, 16], cid=230 + D)
    assert len(set(ks.tolist())) > 1
    say(f"cache_write_rotated_per_head {w.name} k_scales={ks.tolist()}")
    kc, vc, okc, ovc, _, _ = _write_ph_both(w, L, ks, vs)
    assert np.array_equal(to_host_bits(kc), okc), "key cache bytes differ"
    assert np.array_equal(to_host_bits(vc), ovc), "value cache bytes differ"


def _ref_ph(w, L, ks, vs, okc, ovc):
    return oracle.paged_decode_rotated_per_head(w.q, okc, ovc, E4M3, w.block_tables, w.context_lens,
                                                w.num_q_heads, w.num_kv_heads, w.head_dim, 16, ks, vs,
                                                L.sliding_window)


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (64, 8, 64), (16, 2, 256)])
def test_rotated_per_head_decode_matches_oracle(Hq, Hkv, D):
    w, L, ks, vs = _mk_ph(Hq, Hkv, D, [1, 17, 300, 1027, 0], cid=240 + D)
    say(f"paged_decode_rotated_per_head {w.name}")
    kc, vc, okc, ovc, ksd, vsd = _write_ph_both(w, L, ks, vs)
    dev = DeviceInputs(w)
    B = w.num_seqs
    nbytes = F.fp8kv_paged_decode_rotated_workspace_size(B, Hq, Hkv, D, 16, w.max_context_len, 0, 0)
    ws = torch.full((max(nbytes, 256),), 0xFF, dtype=torch.uint8, device=DEV)
    out = torch.empty(B * Hq * D, dtype=torch.bfloat16, device=DEV)
    F.fp8kv_paged_decode_rotated_per_head(out, F.FP8KV_BF16, dev.q, kc, vc, E4M3, dev.bt,
                                          w.max_blocks_per_seq, dev.cl, w.max_context_len, B, Hq, Hkv,
                                          D, 16, w.num_blocks, ksd, vsd, 0, 0, ws, ws.numel())
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64).reshape(B, Hq, D)
    assert_close(got, _ref_ph(w, L, ks, vs, okc, ovc), what=w.name)


@pytest.mark.parametrize("num_splits", [0, 1, 129])
def test_rotated_per_head_step_matches_oracle(num_splits):
    w, L, ks, vs = _mk_ph(32, 8, 128, [5, 700, 2049, 16], cid=250)
    say(f"decode_step_rotated_per_head splits={num_splits}")
    kc, vc, _, _, ksd, vsd = _write_ph_both(w, L, ks, vs, rows=w.prefix_token_rows())
    dev = DeviceInputs(w)
    B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    cnt = new_counters(B, Hkv)
    nbytes = F.fp8kv_paged_decode_rotated_workspace_size(B, Hq, Hkv, D, 16, w.max_context_len, 0,
                                                        num_splits)
    ws = torch.full((max(nbytes, 256),), 0xFF, dtype=torch.uint8, device=DEV)
    kn, vn = step_rows_by_seq(w, L)
    kd, vd = u16_dev(kn), u16_dev(vn)
    out = torch.empty(B * Hq * D, dtype=torch.float32, device=DEV)
    F.fp8kv_decode_step_rotated_per_head(out, F.FP8KV_F32, dev.q, kd, vd, kc, vc, E4M3, dev.bt,
                                         w.max_blocks_per_seq, dev.cl, w.max_context_len, B, Hq, Hkv,
                                         D, 16, w.num_blocks, ksd, vsd, 0, num_splits, cnt,
                                         cnt.numel(), ws, ws.numel())
    torch.cuda.synchronize()
    okc, ovc = host_caches(w, E4M3)
    oracle.cache_write_rotated_per_head(L.k, L.v, okc, ovc, E4M3, w.slot_mapping, w.num_kv_heads,
                                        w.head_dim, 16, w.num_blocks, ks, vs)
    assert np.array_equal(to_host_bits(kc), okc), "key cache bytes differ after the step"
    assert np.array_equal(to_host_bits(vc), ovc), "value cache bytes differ after the step"
    got = out.cpu().numpy().astype(np.float64).reshape(B, Hq, D)
    assert_close(got, _ref_ph(w, L, ks, vs, okc, ovc), atol=2e-4, rtol=2e-3, what=w.name)
    assert not cnt.cpu().numpy().any(), "counters were not returned to zero"


# ---- prefill over a rotated cache

PF_LENS, PF_CHUNKS = [37, 300, 1027, 16, 5, 40], [37, 64, 200, 1, 5, 0]


def _prefill_rot(w, L, ks, vs, kc, vc, cdt, pq, out_f32=False, num_query_tokens=None):
    dev = DeviceInputs(w)
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    T = pq.num_tokens if num_query_tokens is None else num_query_tokens
    nbytes = F.fp8kv_paged_prefill_rotated_workspace_size(T, Hq, D)
    ws = torch.full((max(nbytes, 256),), 0xFF, dtype=torch.uint8, device=DEV)
    out = torch.full((max(pq.num_tokens, 1) * Hq * D,), float("nan"),
                     dtype=torch.float32 if out_f32 else torch.bfloat16, device=DEV)
    q = u16_dev(pq.q)
    qsl = torch.from_numpy(np.ascontiguousarray(pq.query_start_loc)).to(DEV)
    F.fp8kv_paged_prefill_rotated(out, F.FP8KV_F32 if out_f32 else F.FP8KV_BF16, q, qsl, kc, vc, cdt,
                                  dev.bt, w.max_blocks_per_seq, dev.cl, w.max_context_len,
                                  w.num_seqs, pq.max_query_len, T, Hq, Hkv, D, 16, w.num_blocks, ks,
                                  vs, L.sliding_window, ws, ws.numel())
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)[: pq.num_tokens * Hq * D].reshape(
        pq.num_tokens, Hq, D)


def _pf_pairs(w, pq, seed=280):
    """Every row for the first and the last query head (all tiles and tails), and every
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


def _check_prefill_rot(w, L, ks, vs, pq, out_f32=False):
    cdt, kc, vc, okc, ovc = _write_both(w, L, ks, vs)
    got = _prefill_rot(w, L, ks, vs, kc, vc, cdt, pq, out_f32=out_f32)
    pairs = _pf_pairs(w, pq)
    ref = oracle.paged_prefill_rotated_pairs(pairs, pq.q, pq.query_start_loc, okc, ovc, cdt,
                                             w.block_tables, w.context_lens, w.num_q_heads,
                                             w.num_kv_heads, w.head_dim, 16, ks, vs, L.sliding_window)
    tol = dict(atol=2e-4, rtol=2e-3) if out_f32 else {}
    assert_close(got[pairs[:, 0], pairs[:, 1]], ref, what=f"{w.name} rotated prefill", **tol)
    assert np.all(np.isfinite(got)), "non-finite rows"
    return got, ref


@pytest.mark.parametrize("cache", [syn.E4M3, syn.BF16])
@pytest.mark.parametrize("Hq,Hkv,D", [(4, 1, 64), (32, 8, 128), (64, 8, 64), (12, 2, 128)])
def test_rotated_prefill_matches_oracle(Hq, Hkv, D, cache):
    w, L, ks, vs = _mk(Hq, Hkv, D, PF_LENS, cid=260 + Hq + D, cache=cache)
    pq = syn.prefill_queries(w, PF_CHUNKS, 260 + Hq + D)
    say(f"paged_prefill_rotated {w.name}")
    _check_prefill_rot(w, L, ks, vs, pq)


def test_rotated_prefill_f32_output():
    w, L, ks, vs = _mk(32, 8, 128, [700, 2049, 90], cid=270)
    pq = syn.prefill_queries(w, [200, 333, 17], 270)
    say(f"paged_prefill_rotated f32 {w.name}")
    _check_prefill_rot(w, L, ks, vs, pq, out_f32=True)


@pytest.mark.parametrize("window", [17, 512])
def test_rotated_prefill_windows(window):
    w, L, ks, vs = _mk(64, 8, 64, [1, 20, 200, 1100], cid=271, window=window)
    pq = syn.prefill_queries(w, [1, 20, 150, 300], 271)
    say(f"paged_prefill_rotated window={window}")
    _check_prefill_rot(w, L, ks, vs, pq)


def test_rotated_prefill_rows_past_num_query_tokens_are_untouched():
    """num_query_tokens below query_start_loc[B]: the rows before it match the oracle, the
    rows past it keep their NaN fill (neither read nor written)."""
    w, L, ks, vs = _mk(32, 8, 128, [300, 500], cid=272)
    pq = syn.prefill_queries(w, [100, 60], 272)
    cdt, kc, vc, okc, ovc = _write_both(w, L, ks, vs)
    got = _prefill_rot(w, L, ks, vs, kc, vc, cdt, pq, num_query_tokens=130)
    pairs = np.array([(r, hq) for r in (0, 59, 99, 100, 129) for hq in range(w.num_q_heads)], np.int32)
    ref = oracle.paged_prefill_rotated_pairs(pairs, pq.q, pq.query_start_loc, okc, ovc, cdt,
                                             w.block_tables, w.context_lens, w.num_q_heads,
                                             w.num_kv_heads, w.head_dim, 16, ks, vs)
    assert_close(got[pairs[:, 0], pairs[:, 1]], ref, what="rows before num_query_tokens")
    assert np.all(np.isfinite(got[:130]))
    assert np.all(np.isnan(got[130:]))
