"""Pins for the oracle's per-attention-head scale path ([CAP "Scales and calibration"]: one
K scale and one V scale per kv head).  The per-tensor oracle is pinned on its own (codec
and attention suites); these tests pin the per-head functions to it: a per-head write or
decode must equal the per-tensor one made, head by head, with that head's scales."""
import numpy as np

import oracle
import synthetic as syn

E4M3 = oracle.CACHE_E4M3


def _wl(Hq=8, Hkv=4, D=64, lens=(37, 100, 16), cid=71):
    return syn.make_workload(f"ph-{Hq}-{Hkv}-{D}", cid, num_q_heads=Hq, num_kv_heads=Hkv,
                             head_dim=D, context_lens=list(lens), outlier_frac=0.02)


def _empty(w):
    n = w.num_blocks * w.num_kv_heads * w.block_size * w.head_dim
    return np.zeros(n, np.uint8), np.zeros(n, np.uint8)


def _write_ph(w, ks, vs):
    kc, vc = _empty(w)
    L = w.layers[0]
    oracle.cache_write_per_head(L.k, L.v, kc, vc, E4M3, w.slot_mapping, w.num_kv_heads,
                                w.head_dim, w.block_size, w.num_blocks, ks, vs)
    return kc, vc


def _write_pt(w, k_scale, v_scale):
    kc, vc = _empty(w)
    L = w.layers[0]
    oracle.cache_write(L.k, L.v, kc, vc, E4M3, w.slot_mapping, w.num_kv_heads, w.head_dim,
                       w.block_size, w.num_blocks, k_scale, v_scale)
    return kc, vc


def _tiles(c, w):
    return c.reshape(w.num_blocks, w.num_kv_heads, -1)


def test_equal_head_scales_reduce_to_per_tensor():
    w = _wl()
    s_k, s_v = np.float32(0.0371), np.float32(1.93)
    ks = np.full(w.num_kv_heads, s_k, np.float32)
    vs = np.full(w.num_kv_heads, s_v, np.float32)
    kc, vc = _write_ph(w, ks, vs)
    pk, pv = _write_pt(w, float(s_k), float(s_v))
    assert np.array_equal(kc, pk) and np.array_equal(vc, pv)
    pairs = np.array([(b, hq) for b in range(w.num_seqs) for hq in range(w.num_q_heads)], np.int32)
    a = oracle.paged_decode_pairs_per_head(pairs, w.q, kc, vc, E4M3, w.block_tables, w.context_lens,
                                           w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                           ks, vs)
    b = oracle.paged_decode_pairs(pairs, w.q, pk, pv, E4M3, w.block_tables, w.context_lens,
                                  w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                  float(s_k), float(s_v))
    assert np.array_equal(a, b)


def test_write_is_per_tensor_write_head_by_head():
    w = _wl(cid=72)
    ks = syn.spread_head_scales(w.num_kv_heads, 72)
    vs = syn.spread_head_scales(w.num_kv_heads, 73)
    assert len(set(ks.tolist())) == w.num_kv_heads           # distinct, so a wrong head shows
    kc, vc = _write_ph(w, ks, vs)
    for h in range(w.num_kv_heads):
        pk, pv = _write_pt(w, float(ks[h]), float(vs[h]))
        assert np.array_equal(_tiles(kc, w)[:, h], _tiles(pk, w)[:, h]), f"key head {h}"
        assert np.array_equal(_tiles(vc, w)[:, h], _tiles(pv, w)[:, h]), f"value head {h}"


def test_decode_uses_the_scales_of_each_query_heads_kv_head():
    w = _wl(Hq=12, Hkv=3, D=64, lens=(200, 33), cid=74)
    ks = syn.spread_head_scales(w.num_kv_heads, 74)
    vs = syn.spread_head_scales(w.num_kv_heads, 75)
    kc, vc = _write_ph(w, ks, vs)
    g = w.num_q_heads // w.num_kv_heads
    pairs = np.array([(b, hq) for b in range(w.num_seqs) for hq in range(w.num_q_heads)], np.int32)
    got = oracle.paged_decode_pairs_per_head(pairs, w.q, kc, vc, E4M3, w.block_tables,
                                             w.context_lens, w.num_q_heads, w.num_kv_heads,
                                             w.head_dim, w.block_size, ks, vs)
    for i, (b, hq) in enumerate(pairs):
        h = hq // g
        ref = oracle.paged_decode_pairs(np.array([[b, hq]], np.int32), w.q, kc, vc, E4M3,
                                        w.block_tables, w.context_lens, w.num_q_heads,
                                        w.num_kv_heads, w.head_dim, w.block_size,
                                        float(ks[h]), float(vs[h]))[0]
        assert np.array_equal(got[i], ref), (b, hq)


def test_per_head_amax_scales_bound_each_head():
    """Calibrated per-head scales put every head's largest element at or below 448 after
    division, and some element of every head at 448 (amax / (amax / 448))."""
    w = _wl(cid=76)
    k = w.layers[0].k
    sc = syn.per_head_amax_scales(k)
    x = syn.bf16_bits_to_f32(k).astype(np.float64)
    for h in range(w.num_kv_heads):
        y = np.abs(x[:, h, :]) / np.float64(sc[h])
        assert y.max() <= 448.0 * (1 + 2 ** -20) and y.max() >= 448.0 * (1 - 2 ** -20)
