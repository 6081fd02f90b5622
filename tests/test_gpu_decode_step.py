"""GPU parity of the fused fp8kv_decode_step (write the step token + decode, one launch):
the cache bytes equal the oracle's after the step, the output matches the oracle, and every
counter returns to zero so the next step can reuse the buffer, whatever its batch.  Also the
reproducibility contract: bit-identical outputs with a fixed split count, and run-to-run
differences within fp32 rounding with the automatic plan's run-time step claims."""
import numpy as np
import pytest
import torch

import fp8_kv_cache_reshape_amd as F
import oracle
import synthetic as syn
from gpu_util import (BF16, E4M3, DeviceInputs, assert_close, dev_caches, gpu_decode,
                      gpu_decode_step, gpu_write, new_counters, oracle_decode, oracle_write, say,
                      to_host_bits)

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
    assert not ws.cpu().numpy().any(), "counters were not returned to zero"
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


def test_consecutive_steps_reuse_one_counter_buffer():
    """Three decode steps in a row (context grows by one token each) with one counter buffer
    and one workspace."""
    full = _mk(32, 8, 128, [900, 2500, 37], cid=63)
    layer = full.layers[0]
    kc, vc = dev_caches(full, E4M3)
    B, Hq, Hkv, D = full.num_seqs, full.num_q_heads, full.num_kv_heads, full.head_dim
    cnt = new_counters(B, Hkv)
    wsb = F.fp8kv_paged_decode_workspace_size(B, Hq, Hkv, D, 16, full.max_context_len, 0, 0)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
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
        got, _ = gpu_decode_step(w, layer, kc, vc, counters=cnt, workspace=ws)
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
        assert not cnt.cpu().numpy().any(), "counters were not returned to zero"


def _batch(full, seqs):
    """The sub-workload of sequences `seqs` of `full` (its own block tables, the same cache)."""
    idx = np.asarray(seqs)
    return syn.Workload(**{**full.__dict__, "num_seqs": len(idx), "q": full.q[idx],
                           "block_tables": np.ascontiguousarray(full.block_tables[idx]),
                           "context_lens": np.ascontiguousarray(full.context_lens[idx]),
                           "seq_offsets": full.seq_offsets[idx]})


def test_counter_buffer_serves_growing_batches():
    """One counter buffer sized for 5 sequences and one partials workspace serve a batch of 2,
    then of 5, then of 3 (a serving loop whose batch changes every step).  The second call's
    new counter records were never touched, and the workspace held the first call's partials:
    every output must match the oracle and every counter must be zero after every call."""
    full = _mk(32, 8, 128, [3000, 700, 2049, 1500, 4100], cid=67)
    layer = full.layers[0]
    kc, vc = dev_caches(full, E4M3)
    gpu_write(full, layer, kc, vc, rows=full.prefix_token_rows())
    okc, ovc = oracle_write(full, layer)
    cnt = new_counters(5, full.num_kv_heads)
    wsb = F.fp8kv_paged_decode_workspace_size(5, 32, 8, 128, 16, full.max_context_len, 0, 0)
    ws = torch.full((wsb,), 0xFF, dtype=torch.uint8, device="cuda")
    for seqs, splits in (([0, 1], 0), ([0, 1, 2, 3, 4], 0), ([4, 2, 3], 7), ([1, 3, 0, 2, 4], 0)):
        w = _batch(full, seqs)
        say(f"decode_step growing batch seqs={seqs} splits={splits}")
        got, _ = gpu_decode_step(w, layer, kc, vc, num_splits=splits, counters=cnt, workspace=ws)
        assert_close(got, oracle_decode(w, layer, okc, ovc), what=f"batch {seqs}")
        assert not cnt.cpu().numpy().any(), f"counters not zero after batch {seqs}"
    # every step token was written where the oracle writes it
    assert np.array_equal(to_host_bits(kc), okc) and np.array_equal(to_host_bits(vc), ovc)


def _repeat_step(w, num_splits, runs=3, out_f32=True):
    """The same fused step `runs` times on the same inputs (the step token rewritten with the
    same bytes each time): the outputs of every run."""
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc, rows=w.prefix_token_rows())
    dev = DeviceInputs(w)
    cnt = new_counters(w.num_seqs, w.num_kv_heads)
    outs = []
    for r in range(runs):
        got, _ = gpu_decode_step(w, layer, kc, vc, out_f32=out_f32, num_splits=num_splits, dev=dev,
                                 counters=cnt)
        outs.append(got)
    return outs, kc, vc


@pytest.mark.parametrize("which", ["headline", "b8"])
def test_fixed_split_count_is_bit_reproducible(which):
    """With num_splits > 0 no step is claimed at run time: every run gives the same bits."""
    w = syn.llama8b_long(131072, "amax") if which == "headline" else \
        _mk(32, 8, 128, [16384, 24576, 20000, 17777, 16385, 23000, 19999, 24000], cid=68)
    ns = 32 if which == "headline" else 4
    say(f"decode_step reproducibility {w.name} splits={ns}")
    outs, _, _ = _repeat_step(w, ns)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), "fixed split count: outputs differ between runs"


def test_automatic_plan_differs_only_by_fp32_rounding():
    """With num_splits = 0 the last steps are claimed at run time, so which workgroup sums
    which 64-token step -- and the fp32 order of the sums -- changes between runs.  Each run
    is within E of the exact weighted average of the decoded values, relative to max|V|:
    p enters P.V as a bf16 pair whose representation error is at most 2^-18 p (which
    rounding a term gets depends on the reference maximum of the workgroup that took it),
    the matrix-core accumulator adds at most 256 terms in fp32 between compensated flushes,
    and the merge adds at most 64 terms in fp32.  So E = 2^-18 + (256 + 64) * 2^-24, and two
    runs differ by at most 2E * max|V|."""
    w = syn.llama8b_long(131072, "amax")
    say(f"decode_step automatic plan run-to-run {w.name}")
    outs, _, vc = _repeat_step(w, 0)
    layer = w.layers[0]
    vmax = float(np.nanmax(np.abs(oracle.e4m3_decode(to_host_bits(vc))))) * layer.v_scale
    bound = 2 * (2.0 ** -18 + (256 + 64) * 2.0 ** -24) * vmax
    worst = max(float(np.abs(o - outs[0]).max()) for o in outs[1:])
    say(f"automatic plan: worst run-to-run difference {worst:.3g} (bound {bound:.3g})")
    assert worst <= bound
