"""The optional device error word (fp8kv_set_error_word): every kernel that guards a
device-resident index reports the inputs it had to skip, clamp or read as empty, and the
word stays zero on valid inputs.  Every bad input here is one the kernels already guard
(nothing is read or written out of bounds); the outputs are checked where the header defines
them."""
import numpy as np
import pytest
import torch

import fp8_kv_cache_reshape_amd as F
import synthetic as syn
from gpu_util import (DEV, E4M3, DeviceInputs, assert_close, dev_caches, gpu_decode, gpu_decode_step,
                      gpu_prefill, gpu_write, new_counters, oracle_decode, oracle_write, say,
                      to_host_bits)

pytestmark = pytest.mark.gpu

BLOCK_ID, SLOT, CTX, QLEN = (F.FP8KV_DEVERR_BLOCK_ID, F.FP8KV_DEVERR_SLOT,
                             F.FP8KV_DEVERR_CONTEXT_LEN, F.FP8KV_DEVERR_QUERY_LEN)


@pytest.fixture
def word():
    """A zeroed device word installed as this thread's error word for the test."""
    wd = torch.zeros(64, dtype=torch.int32, device=DEV)
    F.fp8kv_set_error_word(wd)
    try:
        yield wd
    finally:
        F.fp8kv_set_error_word(None)


def _read(wd) -> int:
    torch.cuda.synchronize()
    v = int(wd[0].item()) & 0xFFFFFFFF
    assert not wd[1:].cpu().numpy().any(), "the library wrote past the error word"
    return v


def _mk(lens, window=0, cid=300, Hq=32, Hkv=8, D=128):
    return syn.make_workload(f"err-{Hq}-{Hkv}-{D}-w{window}", cid, num_q_heads=Hq, num_kv_heads=Hkv,
                             head_dim=D, context_lens=lens, layers=(("l0", window, syn.E4M3),))


def test_valid_inputs_leave_the_word_zero(word):
    w = _mk([5, 700, 2049, 16, 0])
    layer = w.layers[0]
    say("error word: valid write, decode (both merges), step, prefill, rotated path")
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc, rows=w.prefix_token_rows())
    gpu_decode_step(w, layer, kc, vc)
    gpu_decode_step(w, layer, kc, vc, num_splits=3)
    gpu_decode(w, layer, kc, vc)
    gpu_decode(w, layer, kc, vc, counters=new_counters(w.num_seqs, w.num_kv_heads))
    gpu_decode(w, layer, kc, vc, num_splits=4, split_api=True)
    gpu_decode(w, layer, kc, vc, window=17)
    pq = syn.prefill_queries(w, [3, 64, 200, 16, 0], 171)
    gpu_prefill(w, layer, kc, vc, pq)
    gpu_prefill(w, layer, kc, vc, pq, window=40)
    assert _read(word) == 0


def test_slots_past_the_cache(word):
    say("error word: slots past the cache")
    Hkv, D, NB = 2, 64, 3
    k = torch.ones(4 * Hkv * D, dtype=torch.bfloat16, device=DEV)
    kc = torch.full((NB * Hkv * 16 * D,), 0x5A, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0x5A)
    neg = torch.tensor([-1, -100, -1, -7], dtype=torch.int64, device=DEV)
    F.fp8kv_cache_write(k, k, kc, vc, E4M3, neg, 4, Hkv, D, 16, NB, 1.0, 1.0)
    assert _read(word) == 0, "negative slots are padding, not errors"
    bad = torch.tensor([-1, 5, NB * 16, NB * 16 + 5], dtype=torch.int64, device=DEV)
    F.fp8kv_cache_write(k, k, kc, vc, E4M3, bad, 4, Hkv, D, 16, NB, 1.0, 1.0)
    assert _read(word) == SLOT
    # the valid slot 5 was written, nothing else
    assert int((kc != 0x5A).sum()) == Hkv * D and int((vc != 0x5A).sum()) == Hkv * D
    word.zero_()
    F.fp8kv_cache_write_rotated(k, k, kc, vc, E4M3, bad, 4, Hkv, D, 16, NB, 1.0, 1.0)
    assert _read(word) == SLOT


@pytest.mark.parametrize("fused", [False, True])
def test_bad_block_id_in_the_window(word, fused):
    """A table entry past num_blocks inside a sequence's window is read as an empty block and
    reported; the same entry outside the window (not attended) is not."""
    w = _mk([700, 300], window=0)
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc)
    okc, ovc = oracle_write(w, layer)
    bt = w.block_tables.copy()
    bt[0, 3] = w.num_blocks + 7              # block 3 of sequence 0: positions 48..63
    wb = syn.Workload(**{**w.__dict__, "block_tables": bt})
    cnt = new_counters(w.num_seqs, w.num_kv_heads) if fused else None
    say(f"error word: bad block id, fused={fused}")
    got = gpu_decode(wb, layer, kc, vc, num_splits=3, counters=cnt)
    assert np.all(np.isfinite(got))
    # sequence 1 is untouched by the bad entry
    assert_close(got[1:], oracle_decode(w, layer, okc, ovc)[1:], what="other sequence")
    assert _read(word) == BLOCK_ID
    word.zero_()
    # a 512-position window of sequence 0 (positions 188..699) no longer covers block 3
    gpu_decode(wb, layer, kc, vc, window=512, counters=cnt)
    assert _read(word) == 0


def test_step_with_a_bad_block_for_its_token(word):
    w = _mk([700, 300, 17])
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc, rows=w.prefix_token_rows())
    before_k, before_v = to_host_bits(kc), to_host_bits(vc)
    bt = w.block_tables.copy()
    bt[2, 1] = -3                           # sequence 2's token (position 16) sits in block 1
    wb = syn.Workload(**{**w.__dict__, "block_tables": bt})
    say("error word: step token with a bad block id")
    got, _ = gpu_decode_step(wb, layer, kc, vc)
    assert np.all(np.isfinite(got))
    assert _read(word) == BLOCK_ID
    # sequences 0 and 1 wrote their tokens; sequence 2 wrote nothing
    okc, ovc = oracle_write(w, layer)
    kk = to_host_bits(kc)
    changed = np.nonzero(kk != before_k)[0]
    assert changed.size > 0 and np.array_equal(kk[changed], okc[changed])
    tile = w.num_kv_heads * 16 * w.head_dim
    blocks = set((changed // tile).tolist())
    assert blocks <= {int(w.block_tables[0, 699 // 16]), int(w.block_tables[1, 299 // 16])}


@pytest.mark.parametrize("lens_dev", [[900, 300], [-5, 300]])
def test_context_length_clamped(word, lens_dev):
    w = _mk([600, 300])
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc)
    dev = DeviceInputs(w, context_lens=np.array(lens_dev, np.int32))
    say(f"error word: context lengths {lens_dev} with max_context_len 600")
    got = gpu_decode(w, layer, kc, vc, dev=dev, max_context_len=600)
    assert np.all(np.isfinite(got))
    assert _read(word) == CTX


def test_prefill_reports(word):
    w = _mk([300, 120])
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc)
    pq = syn.prefill_queries(w, [40, 20], 172)
    say("error word: prefill chunk longer than max_query_len")
    gpu_prefill(w, layer, kc, vc, pq, max_query_len=32)
    assert _read(word) == QLEN
    word.zero_()
    say("error word: prefill context above the hint")
    gpu_prefill(w, layer, kc, vc, pq, max_context_len=200)
    assert _read(word) == CTX
    word.zero_()
    bt = w.block_tables.copy()
    bt[1, 2] = w.num_blocks                 # block 2 of sequence 1: positions 32..47, attended
    wb = syn.Workload(**{**w.__dict__, "block_tables": bt})
    say("error word: prefill bad block id")
    out = gpu_prefill(wb, layer, kc, vc, pq)
    assert np.all(np.isfinite(out))
    assert _read(word) == BLOCK_ID
