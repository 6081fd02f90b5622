"""GPU parity of the fused fp8kv_decode_step (write the step token + decode, one launch):
the cache bytes equal the oracle's after the step, the output matches the oracle, and the
workspace's arrival counters return to zero so the next step can reuse it."""
import numpy as np
import pytest
import torch

import fp8_kv_cache_reshape_amd as F
import oracle
import synthetic as syn
from gpu_util import (BF16, E4M3, DeviceInputs, assert_close, dev_caches, gpu_decode,
                      gpu_decode_step, gpu_write, oracle_decode, oracle_write, say, to_host_bits)

pytestmark = pytest.mark.gpu


def _mk(Hq, Hkv, D, lens, cache=syn.E4M3, window=0, cid=60, scale="amax"):
    return syn.make_workload(f"step-{Hq}-{Hkv}-{D}-{cache}-w{window}", cid, num_q_heads=Hq,
                             num_kv_heads=Hkv, head_dim=D, context_lens=lens, outlier_frac=0.01,
                             scale_mode=scale, layers=(("l0", window, cache),))


def _check_step(w, num_splits=0, out_f32=False):
    layer = w.layers[0]
    cdt = E4M3 if layer.cache_dtype == syn.E4M3 else BF16
    kc, vc = dev_caches(w, cdt)
    gpu_write(w, layer, kc, vc, rows=w.prefix_token_rows())      # the context before the step
    got, ws = gpu_decode_step(w, layer, kc, vc, out_f32=out_f32, num_splits=num_splits)
    okc, ovc = oracle_write(w, layer)                                # context + step token
    assert np.array_equal(to_host_bits(kc), okc), "key cache bytes differ after the step"
    assert np.array_equal(to_host_bits(vc), ovc), "value cache bytes differ after the step"
    ref = oracle_decode(w, layer, okc, ovc)
    if out_f32:
        assert_close(got, ref, atol=2e-4, rtol=2e-3, what=w.name)
    else:
        assert_close(got, ref, what=w.name)
    counters = ws[:w.num_seqs * w.num_kv_heads * 4].cpu().numpy()
    assert not counters.any(), "arrival counters were not returned to zero"
    return got, ref


SHAPES = [(4, 1, 64), (32, 8, 128), (64, 8, 128), (12, 2, 128), (64, 8, 64), (8, 1, 256), (16, 1, 256)]


@pytest.mark.parametrize("cache", [syn.E4M3, syn.BF16])
@pytest.mark.parametrize("Hq,Hkv,D", SHAPES)
def test_step_matches_oracle(Hq, Hkv, D, cache):
    w = _mk(Hq, Hkv, D, [1, 16, 17, 300, 1027, 0], cache=cache)
    say(f"decode_step {w.name}")
    _check_step(w)


# 64 asks for 43 splits of 3 blocks (two merge batches per thread); 129 gives one block per
# split, more partials than the in-kernel merge takes, so the step queues the merge kernel
@pytest.mark.parametrize("num_splits", [1, 2, 5, 64, 129])
def test_step_split_counts(num_splits):
    w = _mk(32, 8, 128, [5, 700, 2049, 16], cid=61)
    say(f"decode_step splits={num_splits}")
    _check_step(w, num_splits=num_splits, out_f32=True)


# head_dim 256, group 8: up to 16 splits merge inside the kernel in one round trip (four
# passes over the channel quads per lane); 17 splits queue the merge kernel
@pytest.mark.parametrize("num_splits", [1, 3, 16, 17])
@pytest.mark.parametrize("window", [0, 512])
def test_step_d256_group8_merge(num_splits, window):
    w = _mk(8, 1, 256, [5, 700, 4100, 16, 1500], cid=65, window=window)
    say(f"decode_step d256 g8 splits={num_splits} window={window}")
    _check_step(w, num_splits=num_splits, out_f32=True)


@pytest.mark.parametrize("window", [1, 17, 128, 512])
def test_step_windows(window):
    w = _mk(64, 8, 64, [1, 20, 200, 1100], cid=62, window=window)
    say(f"decode_step window={window}")
    _check_step(w)


def test_consecutive_steps_reuse_one_workspace():
    """Three decode steps in a row (context grows by one token each) with one workspace."""
    full = _mk(32, 8, 128, [900, 2500, 37], cid=63)
    layer = full.layers[0]
    kc, vc = dev_caches(full, E4M3)
    B, Hq, Hkv, D = full.num_seqs, full.num_q_heads, full.num_kv_heads, full.head_dim
    ws = torch.zeros(F.fp8kv_decode_step_workspace_size(B, Hq, Hkv, D, 16, full.max_context_len, 0, 0),
                     dtype=torch.uint8, device="cuda")
    first = True
    for k in (2, 1, 0):
        lens = np.maximum(full.context_lens - k, 0).astype(np.int32)
        w = syn.Workload(**{**full.__dict__, "context_lens": lens})
        say(f"decode_step consecutive lens={lens.tolist()}")
        if first:        # the context before the first step
            first = False
            rows = np.concatenate([np.arange(full.seq_offsets[b], full.seq_offsets[b] + max(int(L) - 1, 0))
                                   for b, L in enumerate(lens)])
            gpu_write(full, layer, kc, vc, rows=rows)
        got, ws = gpu_decode_step(w, layer, kc, vc, workspace=ws)
        # the oracle writes exactly the tokens [0, L_b) of every sequence
        rows = np.concatenate([np.arange(full.seq_offsets[b], full.seq_offsets[b] + int(L)) for b, L in enumerate(lens)])
        ws_sub = syn.Workload(**{**full.__dict__, "context_lens": lens, "slot_mapping": full.slot_mapping[rows],
                                 "layers": [syn.Layer(k=layer.k[rows], v=layer.v[rows], cache_dtype=layer.cache_dtype,
                                                      k_scale=layer.k_scale, v_scale=layer.v_scale)]})
        okc, ovc = oracle_write(ws_sub, ws_sub.layers[0])
        written = okc != 0x7F
        assert np.array_equal(to_host_bits(kc)[written], okc[written])
        ref = oracle_decode(w, layer, okc, ovc)
        assert_close(got, ref, what=f"step lens={lens.tolist()}")
        assert not ws[:B * Hkv * 4].cpu().numpy().any(), "arrival counters were not returned to zero"


def test_step_agrees_with_two_calls():
    w = _mk(64, 8, 128, [4000, 333], cid=64)
    say("decode_step vs write + decode")
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc)
    two = gpu_decode(w, layer, kc, vc, out_f32=True)
    kc2, vc2 = dev_caches(w, E4M3)
    gpu_write(w, layer, kc2, vc2, rows=w.prefix_token_rows())
    one, _ = gpu_decode_step(w, layer, kc2, vc2, out_f32=True)
    assert torch.equal(kc, kc2) and torch.equal(vc, vc2)
    # Both merge the same fp32 partials: sum_s w_s x_s / Lambda with sum_s w_s |x_s| <=
    # max|V| * Lambda.  The in-kernel merge sums at most 64 terms in plain fp32, the merge
    # kernel compensates, so they differ by at most about 2 * 64 * 2^-24 * max|V|.
    vmax = float(np.nanmax(np.abs(oracle.e4m3_decode(to_host_bits(vc))))) * layer.v_scale   # NaN: unwritten
    assert np.abs(one - two).max() <= 2 * 64 * 2.0 ** -24 * vmax


def test_step_headline_128k():
    w = syn.llama8b_long(131072, "amax")
    say(f"decode_step {w.name}")
    _check_step(w)


@pytest.mark.parametrize("L,window", [(528, 0), (529, 0), (4000, 512), (4000, 513)])
def test_step_at_single_split_threshold(L, window):
    """The planner keeps one split up to 33 blocks per (sequence, kv head) and splits beyond:
    both sides of that threshold (context and window) against the oracle."""
    w = _mk(32, 8, 128, [L, L - 7, 16], cid=66, window=window)
    ns = F.fp8kv_paged_decode_num_splits(w.num_seqs, w.num_kv_heads, w.head_dim, 16,
                                         w.max_context_len, window, 0)
    assert (ns == 1) == ((L <= 528) if window == 0 else (window <= 512))
    say(f"decode_step threshold L={L} window={window} splits={ns}")
    _check_step(w, out_f32=True)
