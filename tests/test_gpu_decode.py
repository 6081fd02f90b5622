"""GPU parity of fp8kv_paged_decode against the fp64 oracle on small, ragged inputs that span
several blocks, splits and a partial tail block, for every supported head_dim, several group
ratios, both cache dtypes, windows and split counts; with the separate merge kernel and with
a counter buffer (the partials merged inside the decode kernel)."""
import numpy as np
import pytest
import torch

import fp8_kv_cache_reshape_amd as F
import oracle
import synthetic as syn
from gpu_util import (BF16, E4M3, DeviceInputs, assert_close, dev_caches, gpu_decode, gpu_write,
                      new_counters, oracle_decode, oracle_write, say)

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 64, 65, 300, 1027]


def _mk(Hq, Hkv, D, lens=LENS, cache=syn.E4M3, window=0, cid=40, std=1.0, outliers=0.01,
        scale="amax"):
    return syn.make_workload(f"small-{Hq}-{Hkv}-{D}-{cache}-w{window}", cid, num_q_heads=Hq,
                             num_kv_heads=Hkv, head_dim=D, context_lens=lens, std=std,
                             outlier_frac=outliers, scale_mode=scale,
                             layers=(("l0", window, cache),))


def _run(w, out_f32=False, num_splits=0, window=None, split_api=False, fused=False):
    layer = w.layers[0]
    cdt = E4M3 if layer.cache_dtype == syn.E4M3 else BF16
    kc, vc = dev_caches(w, cdt)
    gpu_write(w, layer, kc, vc)
    okc, ovc = oracle_write(w, layer)
    cnt = new_counters(w.num_seqs, w.num_kv_heads) if fused else None
    got = gpu_decode(w, layer, kc, vc, out_f32=out_f32, num_splits=num_splits, window=window,
                     split_api=split_api, counters=cnt)
    ref = oracle_decode(w, layer, okc, ovc, window=window)
    if fused:
        assert not cnt.cpu().numpy().any(), "counters were not returned to zero"
    return got, ref


SHAPES = [(4, 1, 64), (2, 2, 64), (32, 8, 128), (64, 8, 128), (12, 2, 128), (16, 1, 128),
          (64, 8, 64), (8, 1, 256), (16, 1, 256)]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("cache", [syn.E4M3, syn.BF16])
@pytest.mark.parametrize("Hq,Hkv,D", SHAPES)
def test_decode_matches_oracle(Hq, Hkv, D, cache, fused):
    w = _mk(Hq, Hkv, D, cache=cache)
    say(f"decode {w.name} fused={fused}")
    got, ref = _run(w, fused=fused)
    assert_close(got, ref, what=w.name)


# with counters: 64 splits merge in the kernel in two batches per lane; 129 are more than it
# merges, so the merge kernel follows the decode
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 64, 129])
def test_split_counts(num_splits, fused):
    w = _mk(32, 8, 128, lens=[5, 700, 2049, 16], cid=41)
    say(f"decode splits={num_splits} fused={fused}")
    got, ref = _run(w, num_splits=num_splits, fused=fused, out_f32=True)
    assert_close(got, ref, atol=2e-4, rtol=2e-3, what=f"splits={num_splits}")


def test_in_kernel_merge_equals_merge_kernel():
    """The same split partials merged by the last workgroup (counters given, fixed split
    count: no run-time claims) and by the merge kernel: both sum the same fp32 partials, so
    they differ by fp32 rounding only (at most 64 plain fp32 terms against a compensated sum:
    2 * 64 * 2^-24 * max|V|); two runs of the in-kernel merge are bit-identical."""
    w = _mk(64, 8, 128, lens=[4000, 333, 2500], cid=49)
    say("decode in-kernel merge vs merge kernel")
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc)
    cnt = new_counters(w.num_seqs, w.num_kv_heads)
    a = gpu_decode(w, layer, kc, vc, out_f32=True, num_splits=9)
    b = gpu_decode(w, layer, kc, vc, out_f32=True, num_splits=9, counters=cnt)
    c = gpu_decode(w, layer, kc, vc, out_f32=True, num_splits=9, counters=cnt)
    assert np.array_equal(b, c)
    assert not cnt.cpu().numpy().any()
    vmax = float(np.nanmax(np.abs(oracle.e4m3_decode(oracle_write(w, layer)[1])))) * layer.v_scale
    assert np.abs(a - b).max() <= 2 * 64 * 2.0 ** -24 * vmax


@pytest.mark.parametrize("window", [1, 2, 15, 16, 17, 128, 129, 512, 5000])
@pytest.mark.parametrize("cache", [syn.E4M3, syn.BF16])
def test_sliding_windows(window, cache):
    w = _mk(64, 8, 64, lens=[1, 20, 200, 1100], cid=42, cache=cache, window=window)
    say(f"decode window={window} {cache}")
    got, ref = _run(w)
    assert_close(got, ref, what=f"window={window}")


def test_f32_output_is_tighter():
    w = _mk(32, 8, 128, lens=[3000, 77], cid=43)
    say("decode f32 out")
    got, ref = _run(w, out_f32=True)
    assert_close(got, ref, atol=2e-4, rtol=2e-3, what="f32 out")


def test_uncalibrated_scale_one():
    w = _mk(32, 8, 128, lens=[900, 31], cid=44, scale="uncal")
    say("decode uncalibrated scale")
    got, ref = _run(w)
    assert_close(got, ref, what="uncal")


def test_partial_then_merge_equals_one_call():
    w = _mk(64, 8, 128, lens=[2000, 100], cid=45)
    say("decode partial+merge")
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc)
    a = gpu_decode(w, layer, kc, vc, out_f32=True, num_splits=5)
    b = gpu_decode(w, layer, kc, vc, out_f32=True, num_splits=5, split_api=True)
    assert np.array_equal(a, b)
    c = gpu_decode(w, layer, kc, vc, out_f32=True, num_splits=1, split_api=True)
    d = gpu_decode(w, layer, kc, vc, out_f32=True, num_splits=1)
    assert np.abs(c - d).max() < 1e-6


def test_deterministic_and_placement_invariant():
    w = _mk(32, 8, 128, lens=[1500, 33, 260], cid=46)
    say("decode determinism / block placement")
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc)
    a = gpu_decode(w, layer, kc, vc, out_f32=True)
    b = gpu_decode(w, layer, kc, vc, out_f32=True)
    assert np.array_equal(a, b)
    # move every physical block and rewrite the block table: the result is bit-identical
    rng = np.random.default_rng(0)
    newpos = rng.permutation(w.num_blocks)
    tile = w.num_kv_heads * w.block_size * w.head_dim
    kc2, vc2 = torch.empty_like(kc), torch.empty_like(vc)
    idx = torch.from_numpy(newpos).to(kc.device)
    kc2.view(w.num_blocks, tile)[idx] = kc.view(w.num_blocks, tile)
    vc2.view(w.num_blocks, tile)[idx] = vc.view(w.num_blocks, tile)
    w2 = syn.Workload(**{**w.__dict__, "block_tables": newpos[w.block_tables].astype(np.int32)})
    c = gpu_decode(w2, layer, kc2, vc2, out_f32=True)
    assert np.array_equal(a, c)


def test_empty_and_single_token_contexts():
    w = _mk(8, 2, 128, lens=[0, 1, 0, 2], cid=47)
    say("decode empty / single token")
    got, ref = _run(w)
    assert np.array_equal(got[0], np.zeros_like(got[0])) and np.array_equal(got[2], np.zeros_like(got[2]))
    assert_close(got, ref, what="empty/single")


def test_context_longer_than_hint_is_clamped():
    """context_lens above max_context_len are read as max_context_len (no out-of-range walk)."""
    w = _mk(32, 8, 128, lens=[600, 400], cid=48)
    say("decode clamp to max_context_len")
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc)
    okc, ovc = oracle_write(w, layer)
    got = gpu_decode(w, layer, kc, vc, max_context_len=500)
    ref = oracle_decode(w, layer, okc, ovc, context_lens=np.minimum(w.context_lens, 500))
    assert_close(got, ref, what="clamped")
