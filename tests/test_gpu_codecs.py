"""GPU parity of the E5M2 and INT8 cache codecs: writes (bulk, slot patterns, every bf16
input) bit-exact against the oracle's codec write, and the decode, the fused step and the
prefill over such caches within the decode tolerance of the oracle's attention."""
import numpy as np
import pytest
import torch

import fp8_kv_cache_reshape_amd as F
import oracle
import synthetic as syn
from gpu_util import (DEV, DeviceInputs, assert_close, new_counters, say, step_rows_by_seq, to_host_bits,
                      u16_dev)

pytestmark = pytest.mark.gpu

CODECS = {"e5m2": (F.FP8KV_E5M2, oracle.CACHE_E5M2, 57344.0),
          "int8": (F.FP8KV_INT8, oracle.CACHE_INT8, 127.0)}


def _scales(L, top):
    """Calibrated scales for the codec: amax / its largest code (from the workload's
    amax/448 scales)."""
    return (float(np.float32(L.k_scale) * np.float32(448.0) / np.float32(top)),
            float(np.float32(L.v_scale) * np.float32(448.0) / np.float32(top)))


def _mk(Hq, Hkv, D, lens, cid, window=0):
    return syn.make_workload(f"codec-{Hq}-{Hkv}-{D}-w{window}", cid, num_q_heads=Hq,
                             num_kv_heads=Hkv, head_dim=D, context_lens=lens, outlier_frac=0.01,
                             layers=(("l0", window, syn.E4M3),))


def _gpu_write(w, L, codec, ks, vs, rows=None):
    n = w.num_blocks * w.num_kv_heads * 16 * w.head_dim
    kc = torch.full((n,), 0x55, dtype=torch.uint8, device=DEV)
    vc = torch.full((n,), 0x55, dtype=torch.uint8, device=DEV)
    rows = np.arange(w.num_tokens) if rows is None else rows
    slots = torch.from_numpy(np.ascontiguousarray(w.slot_mapping[rows])).to(DEV)
    F.fp8kv_cache_write(u16_dev(L.k[rows]), u16_dev(L.v[rows]), kc, vc, codec, slots, len(rows),
                        w.num_kv_heads, w.head_dim, 16, w.num_blocks, ks, vs)
    torch.cuda.synchronize()
    return kc, vc


def _oracle_write(w, L, ocodec, ks, vs):
    n = w.num_blocks * w.num_kv_heads * 16 * w.head_dim
    kc, vc = np.full(n, 0x55, np.uint8), np.full(n, 0x55, np.uint8)
    oracle.cache_write_codec(L.k, L.v, kc, vc, ocodec, w.slot_mapping, w.num_kv_heads, w.head_dim,
                             16, w.num_blocks, ks, vs)
    return kc, vc


@pytest.mark.parametrize("name", sorted(CODECS))
# 0.125, 2^-7, 2^-126, 2^20 and 2^127 (a subnormal reciprocal) are powers of two: the
# multiply-by-reciprocal path; 0.0371 and 250 divide
@pytest.mark.parametrize("scale", [1.0, 0.0371, 250.0, 0.125, 2.0 ** -7, 2.0 ** -126, 2.0 ** 20,
                                   2.0 ** 127])
def test_codec_write_every_bf16_input(name, scale):
    """Every bf16 bit pattern once as a key and once as a value element, scattered to random
    slots (the per-token store path) and, in a second write, to in-order slots (the
    transposed path)."""
    codec, ocodec, _ = CODECS[name]
    Hkv, D = 2, 128
    T = 65536 // (Hkv * D)
    keys = np.arange(65536, dtype=np.uint16).reshape(T, Hkv, D)
    vals = keys[::-1].reshape(T, Hkv, D).copy()
    rng = np.random.default_rng(7)
    NB = T // 16 + 7
    for order in ("scattered", "in_order"):
        slots = (rng.permutation(NB * 16)[:T] if order == "scattered" else np.arange(T) + 32).astype(np.int64)
        w = syn.Workload(name="every-bf16", num_seqs=0, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D,
                         block_size=16, num_blocks=NB, context_lens=np.zeros(0, np.int32),
                         block_tables=np.zeros((0, 1), np.int32), seq_offsets=np.zeros(1, np.int64),
                         slot_mapping=slots, q=np.zeros((0, Hkv, D), np.uint16), layers=[])
        L = syn.Layer(k=keys, v=vals, cache_dtype="e4m3", k_scale=scale, v_scale=scale)
        say(f"codec write {name} scale={scale} {order}")
        kc, vc = _gpu_write(w, L, codec, scale, scale)
        okc, ovc = _oracle_write(w, L, ocodec, scale, scale)
        assert np.array_equal(to_host_bits(kc), okc), "key bytes differ"
        assert np.array_equal(to_host_bits(vc), ovc), "value bytes differ"


def _decode_gpu(w, L, codec, kc, vc, ks, vs, num_splits=0):
    dev = DeviceInputs(w)
    B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    nb = F.fp8kv_paged_decode_workspace_size(B, Hq, Hkv, D, 16, w.max_context_len, L.sliding_window,
                                             num_splits)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
    out = torch.empty(B * Hq * D, dtype=torch.bfloat16, device=DEV)
    F.fp8kv_paged_decode(out, F.FP8KV_BF16, dev.q, kc, vc, codec, dev.bt, w.max_blocks_per_seq, dev.cl,
                         w.max_context_len, B, Hq, Hkv, D, 16, w.num_blocks, ks, vs, L.sliding_window,
                         num_splits, None, 0, ws, nb)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64).reshape(B, Hq, D)


@pytest.mark.parametrize("name", sorted(CODECS))
@pytest.mark.parametrize("Hq,Hkv,D", [(4, 1, 64), (32, 8, 128), (64, 8, 64), (16, 1, 256)])
def test_codec_decode_matches_oracle(name, Hq, Hkv, D):
    codec, ocodec, top = CODECS[name]
    w = _mk(Hq, Hkv, D, [1, 16, 17, 300, 1027, 0], cid=210 + Hq + D)
    L = w.layers[0]
    ks, vs = _scales(L, top)
    say(f"codec decode {name} {w.name}")
    kc, vc = _gpu_write(w, L, codec, ks, vs)
    okc, ovc = _oracle_write(w, L, ocodec, ks, vs)
    assert np.array_equal(to_host_bits(kc), okc) and np.array_equal(to_host_bits(vc), ovc)
    for splits in (0, 1, 129):
        got = _decode_gpu(w, L, codec, kc, vc, ks, vs, splits)
        ref = oracle.paged_decode(w.q, okc, ovc, ocodec, w.block_tables, w.context_lens, Hq, Hkv, D,
                                  16, ks, vs)
        assert_close(got, ref, what=f"{name} {w.name} splits={splits}")


@pytest.mark.parametrize("name", sorted(CODECS))
def test_codec_decode_step_matches_oracle(name):
    codec, ocodec, top = CODECS[name]
    w = _mk(32, 8, 128, [1, 16, 17, 300, 2049], cid=220)
    L = w.layers[0]
    ks, vs = _scales(L, top)
    say(f"codec step {name}")
    kc, vc = _gpu_write(w, L, codec, ks, vs, rows=w.prefix_token_rows())
    dev = DeviceInputs(w)
    B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    nb = F.fp8kv_paged_decode_workspace_size(B, Hq, Hkv, D, 16, w.max_context_len, 0, 0)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
    cnt = new_counters(B, Hkv)
    kn, vn = step_rows_by_seq(w, L)
    out = torch.empty(B * Hq * D, dtype=torch.bfloat16, device=DEV)
    F.fp8kv_decode_step(out, F.FP8KV_BF16, dev.q, u16_dev(kn), u16_dev(vn), kc, vc, codec, dev.bt,
                        w.max_blocks_per_seq, dev.cl, w.max_context_len, B, Hq, Hkv, D, 16,
                        w.num_blocks, ks, vs, 0, 0, cnt, cnt.numel(), ws, nb)
    torch.cuda.synchronize()
    okc, ovc = _oracle_write(w, L, ocodec, ks, vs)
    assert np.array_equal(to_host_bits(kc), okc) and np.array_equal(to_host_bits(vc), ovc)
    got = out.float().cpu().numpy().astype(np.float64).reshape(B, Hq, D)
    ref = oracle.paged_decode(w.q, okc, ovc, ocodec, w.block_tables, w.context_lens, Hq, Hkv, D, 16,
                              ks, vs)
    assert_close(got, ref, what=f"{name} step")


@pytest.mark.parametrize("name", sorted(CODECS))
def test_codec_prefill_matches_oracle(name):
    codec, ocodec, top = CODECS[name]
    w = _mk(32, 8, 128, [37, 300, 1027, 16], cid=230)
    L = w.layers[0]
    ks, vs = _scales(L, top)
    pq = syn.prefill_queries(w, [37, 64, 200, 1], 230)
    say(f"codec prefill {name}")
    kc, vc = _gpu_write(w, L, codec, ks, vs)
    dev = DeviceInputs(w)
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    out = torch.empty(pq.num_tokens * Hq * D, dtype=torch.bfloat16, device=DEV)
    F.fp8kv_paged_prefill(out, F.FP8KV_BF16, u16_dev(pq.q),
                          torch.from_numpy(pq.query_start_loc).to(DEV), kc, vc, codec, dev.bt,
                          w.max_blocks_per_seq, dev.cl, w.max_context_len, w.num_seqs, pq.max_query_len,
                          Hq, Hkv, D, 16, w.num_blocks, ks, vs, 0)
    torch.cuda.synchronize()
    okc, ovc = _oracle_write(w, L, ocodec, ks, vs)
    got = out.float().cpu().numpy().astype(np.float64).reshape(pq.num_tokens, Hq, D)
    # every row for heads 0 and Hq-1, every head for the first and last rows of each chunk
    rows = sorted({int(x) for b in range(w.num_seqs) for x in
                   (pq.query_start_loc[b], pq.query_start_loc[b + 1] - 1)
                   if pq.query_start_loc[b + 1] > pq.query_start_loc[b]})
    pairs = np.array(sorted({(r, h) for r in range(pq.num_tokens) for h in (0, Hq - 1)} |
                            {(r, h) for r in rows for h in range(Hq)}), np.int32)
    ref = oracle.paged_prefill_pairs(pairs, pq.q, pq.query_start_loc, okc, ovc, ocodec,
                                     w.block_tables, w.context_lens, Hq, Hkv, D, 16, ks, vs)
    assert_close(got[pairs[:, 0], pairs[:, 1]], ref, what=f"{name} prefill")
