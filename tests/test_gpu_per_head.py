"""GPU parity of the per-attention-head scale entry points (one K and one V scale per kv
head, page "FP8 KV Cache Quantization: Capacity Gains and Accuracy Risk", "Scales and
calibration"): the per-head write is bit-exact against the oracle's per-head write, and the
per-head decode and decode step match the oracle's per-head decode, over the launch shapes
that take different merge routes (one pass, in-kernel merge of one or two quads per lane,
the merge kernel)."""
import numpy as np
import pytest
import torch

import fp8_kv_cache_reshape_amd as F
import synthetic as syn
from gpu_util import (BF16, E4M3, DEV, assert_close, dev_caches, gpu_decode, gpu_decode_step,
                      gpu_write, oracle_decode, oracle_write, say, to_host_bits, u16_dev)

pytestmark = pytest.mark.gpu

LENS = [1, 16, 17, 300, 1027, 0]


def _mk(Hq, Hkv, D, lens, cid, window=0, cache=syn.E4M3, kind="calibrated"):
    """A workload and its per-head scales: "calibrated" gives the kv heads magnitudes 2^-3 ..
    2^3 apart with per-head amax/448 scales; "spread" keeps the data and draws scales over
    [0.05, 8] (codes that saturate, and subnormal codes)."""
    w = syn.make_workload(f"ph-{Hq}-{Hkv}-{D}-{kind}-w{window}", cid, num_q_heads=Hq,
                          num_kv_heads=Hkv, head_dim=D, context_lens=lens, outlier_frac=0.01,
                          layers=(("l0", window, cache),))
    if kind == "calibrated":
        w, scales = syn.with_head_magnitudes(w, cid)
        return w, scales[0]
    if kind == "pow2":
        # powers of two from 2^-9 to 2^4 (the multiply-by-reciprocal path), with one head
        # whose value scale is not (that head divides): both paths in one launch
        ks = np.float32(2.0) ** (np.arange(Hkv) % 14 - 9).astype(np.float32)
        vs = np.float32(2.0) ** (4 - np.arange(Hkv) % 14).astype(np.float32)
        if Hkv > 1:
            vs[-1] = np.float32(0.0371)
        return w, (ks, vs)
    return w, (syn.spread_head_scales(Hkv, cid), syn.spread_head_scales(Hkv, cid + 500))


@pytest.mark.parametrize("kind", ["calibrated", "spread", "pow2"])
@pytest.mark.parametrize("Hkv,D", [(1, 64), (2, 128), (8, 128), (4, 256)])
def test_write_per_head_bit_exact(Hkv, D, kind):
    w, heads = _mk(2 * Hkv, Hkv, D, LENS, cid=80 + D + Hkv, kind=kind)
    say(f"cache_write_per_head {w.name}")
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc, heads=heads)
    okc, ovc = oracle_write(w, layer, heads=heads)
    assert np.array_equal(to_host_bits(kc), okc), "key cache bytes differ"
    assert np.array_equal(to_host_bits(vc), ovc), "value cache bytes differ"


def test_write_per_head_bf16_ignores_scales():
    w, _ = _mk(8, 2, 128, LENS, cid=90, cache=syn.BF16)
    say(f"cache_write_per_head bf16 {w.name}")
    layer = w.layers[0]
    kc, vc = dev_caches(w, BF16)
    slots = torch.from_numpy(w.slot_mapping).to(DEV)
    F.fp8kv_cache_write_per_head(u16_dev(layer.k), u16_dev(layer.v), kc, vc, BF16, slots,
                                 w.num_tokens, w.num_kv_heads, w.head_dim, w.block_size,
                                 w.num_blocks, None, None)
    torch.cuda.synchronize()
    okc, ovc = oracle_write(w, layer)
    assert np.array_equal(to_host_bits(kc), okc) and np.array_equal(to_host_bits(vc), ovc)


def _check_decode(w, heads, num_splits=0, out_f32=False):
    layer = w.layers[0]
    okc, ovc = oracle_write(w, layer, heads=heads)
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc, heads=heads)
    got = gpu_decode(w, layer, kc, vc, out_f32=out_f32, num_splits=num_splits, heads=heads)
    ref = oracle_decode(w, layer, okc, ovc, heads=heads)
    if out_f32:
        assert_close(got, ref, atol=2e-4, rtol=2e-3, what=w.name)
    else:
        assert_close(got, ref, what=w.name)


SHAPES = [(4, 1, 64), (32, 8, 128), (64, 8, 128), (12, 2, 128), (64, 8, 64), (16, 1, 256)]


@pytest.mark.parametrize("kind", ["calibrated", "spread"])
@pytest.mark.parametrize("Hq,Hkv,D", SHAPES)
def test_decode_per_head_matches_oracle(Hq, Hkv, D, kind):
    w, heads = _mk(Hq, Hkv, D, LENS, cid=100 + Hq + D, kind=kind)
    say(f"paged_decode_per_head {w.name}")
    _check_decode(w, heads)


@pytest.mark.parametrize("num_splits", [1, 5, 129])
def test_decode_per_head_split_counts(num_splits):
    w, heads = _mk(32, 8, 128, [5, 700, 2049, 16], cid=110)
    say(f"paged_decode_per_head splits={num_splits}")
    _check_decode(w, heads, num_splits=num_splits, out_f32=True)


@pytest.mark.parametrize("window", [17, 512])
def test_decode_per_head_windows(window):
    w, heads = _mk(64, 8, 64, [1, 20, 200, 1100], cid=111, window=window)
    say(f"paged_decode_per_head window={window}")
    _check_decode(w, heads)


def _check_step(w, heads, num_splits=0, out_f32=False):
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc, rows=w.prefix_token_rows(), heads=heads)
    got, ws = gpu_decode_step(w, layer, kc, vc, out_f32=out_f32, num_splits=num_splits, heads=heads)
    okc, ovc = oracle_write(w, layer, heads=heads)
    assert np.array_equal(to_host_bits(kc), okc), "key cache bytes differ after the step"
    assert np.array_equal(to_host_bits(vc), ovc), "value cache bytes differ after the step"
    ref = oracle_decode(w, layer, okc, ovc, heads=heads)
    if out_f32:
        assert_close(got, ref, atol=2e-4, rtol=2e-3, what=w.name)
    else:
        assert_close(got, ref, what=w.name)
    assert not ws.cpu().numpy().any(), "counters were not returned to zero"


# (4,1,64) and (32,8,128): one channel quad per lane in the in-kernel merge; (64,8,128):
# two; (16,1,256): more than the in-kernel merge takes, so the merge kernel follows
@pytest.mark.parametrize("Hq,Hkv,D", [(4, 1, 64), (32, 8, 128), (64, 8, 128), (16, 1, 256)])
@pytest.mark.parametrize("num_splits", [0, 1, 129])
def test_step_per_head_matches_oracle(Hq, Hkv, D, num_splits):
    w, heads = _mk(Hq, Hkv, D, [1, 16, 17, 300, 2049, 0], cid=120 + Hq + D)
    say(f"decode_step_per_head {w.name} splits={num_splits}")
    _check_step(w, heads, num_splits=num_splits, out_f32=num_splits == 129)


def test_equal_head_scales_match_per_tensor():
    """Per-head arrays holding one value give the per-tensor result: the same cache bytes,
    and outputs that differ only by the rounding of the score scale (log2(e)/sqrt(d) is
    rounded to float before the key scale multiplies it, instead of after)."""
    w, _ = _mk(32, 8, 128, [4000, 333, 17], cid=130)
    layer = w.layers[0]
    heads = (np.full(8, layer.k_scale, np.float32), np.full(8, layer.v_scale, np.float32))
    say(f"per-head equal scales vs per-tensor {w.name}")
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc)
    kc2, vc2 = dev_caches(w, E4M3)
    gpu_write(w, layer, kc2, vc2, heads=heads)
    assert torch.equal(kc, kc2) and torch.equal(vc, vc2)
    a = gpu_decode(w, layer, kc, vc, out_f32=True)
    b = gpu_decode(w, layer, kc, vc, out_f32=True, heads=heads)
    # the score scale differs by at most one float rounding (2^-24 relative); base-2 scores
    # here are below 64 in magnitude, so every weight moves by less than 64 * 2^-23 relative
    assert np.abs(a - b).max() <= 1e-5 * max(1.0, np.abs(a).max())


def test_step_per_head_headline_128k():
    """One sequence of 128K tokens, 32 query heads on 8 kv heads of different magnitudes."""
    w = syn.llama8b_long(131072, "amax")
    w, scales = syn.with_head_magnitudes(w, 140)
    say(f"decode_step_per_head {w.name}")
    _check_step(w, scales[0])


@pytest.mark.parametrize("num_splits", [1, 3, 64])
def test_split_passes_per_head_equal_one_call(num_splits):
    """fp8kv_paged_decode_partial_per_head + fp8kv_paged_decode_merge_per_head run the same
    kernels as fp8kv_paged_decode_per_head without a counter buffer: the same bits, and the
    oracle's per-head decode within the f32 tolerance (the passes a context-parallel decode
    would run on each device and after the gather)."""
    w, heads = _mk(32, 8, 128, [2000, 100, 4099], cid=150)
    say(f"per-head split passes splits={num_splits}")
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc, heads=heads)
    a = gpu_decode(w, layer, kc, vc, out_f32=True, num_splits=num_splits, heads=heads)
    b = gpu_decode(w, layer, kc, vc, out_f32=True, num_splits=num_splits, heads=heads, split_api=True)
    assert np.array_equal(a, b)
    okc, ovc = oracle_write(w, layer, heads=heads)
    assert_close(b, oracle_decode(w, layer, okc, ovc, heads=heads), atol=2e-4, rtol=2e-3,
                 what="per-head split passes")
