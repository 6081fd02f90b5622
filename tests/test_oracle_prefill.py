"""Pins for the oracle's prefill / chunked-prefill attention.  Its definition: the query
row at position p attends causally to the cached positions [lo, p] -- a decode over a
context of length p + 1 -- so the pins tie it to the decode oracle (pinned on its own),
to causality and chunking invariants, and to an independent matrix-form evaluation."""
import numpy as np

import oracle
import synthetic as syn

E4M3, BF16 = oracle.CACHE_E4M3, oracle.CACHE_BF16


def _setup(lens=(40, 100, 17), chunks=(5, 33, 17), Hq=8, Hkv=2, D=64, cid=81, cache=E4M3):
    w = syn.make_workload(f"pf-{Hq}-{Hkv}-{D}", cid, num_q_heads=Hq, num_kv_heads=Hkv,
                          head_dim=D, context_lens=list(lens), outlier_frac=0.02,
                          layers=(("l0", 0, syn.E4M3 if cache == E4M3 else syn.BF16),))
    L = w.layers[0]
    n = w.num_blocks * w.num_kv_heads * w.block_size * w.head_dim
    dt = np.uint8 if cache == E4M3 else np.uint16
    kc, vc = np.zeros(n, dt), np.zeros(n, dt)
    oracle.cache_write(L.k, L.v, kc, vc, cache, w.slot_mapping, Hkv, D, 16, w.num_blocks,
                       L.k_scale, L.v_scale)
    pq = syn.prefill_queries(w, list(chunks), cid)
    return w, L, kc, vc, pq


def _prefill(w, L, kc, vc, pq, cache=E4M3, window=0, lens=None):
    return oracle.paged_prefill(pq.q, pq.query_start_loc, kc, vc, cache, w.block_tables,
                                w.context_lens if lens is None else lens, w.num_q_heads,
                                w.num_kv_heads, w.head_dim, 16, L.k_scale, L.v_scale, window)


def _positions(w, pq):
    pos = np.empty(pq.num_tokens, np.int64)
    for b in range(w.num_seqs):
        a, e = pq.query_start_loc[b], pq.query_start_loc[b + 1]
        pos[a:e] = int(w.context_lens[b]) - (e - a) + np.arange(e - a)
    return pos


def _as_decode(w, L, kc, vc, pq, window=0):
    """Each row recomputed as a decode: its query as the sequence's query, the context cut
    to the row's position + 1."""
    pos = _positions(w, pq)
    out = np.empty((pq.num_tokens, w.num_q_heads, w.head_dim))
    for b in range(w.num_seqs):
        for r in range(pq.query_start_loc[b], pq.query_start_loc[b + 1]):
            q = w.q.copy()
            q[b] = pq.q[r]
            cl = w.context_lens.copy()
            cl[b] = pos[r] + 1
            pairs = np.array([(b, hq) for hq in range(w.num_q_heads)], np.int32)
            out[r] = oracle.paged_decode_pairs(pairs, q, kc, vc, E4M3, w.block_tables, cl,
                                               w.num_q_heads, w.num_kv_heads, w.head_dim, 16,
                                               L.k_scale, L.v_scale, window)
    return out


def test_each_row_is_a_decode_over_its_prefix():
    w, L, kc, vc, pq = _setup()
    np.testing.assert_array_equal(_prefill(w, L, kc, vc, pq), _as_decode(w, L, kc, vc, pq))


def test_window_rows_are_windowed_decodes():
    w, L, kc, vc, pq = _setup(cid=82)
    for window in (1, 7, 16, 60):
        np.testing.assert_array_equal(_prefill(w, L, kc, vc, pq, window=window),
                                      _as_decode(w, L, kc, vc, pq, window=window))


def test_future_positions_are_never_read():
    """Poisoning every position after a row's own leaves that row unchanged; changing the
    row's own position changes it."""
    w, L, kc, vc, pq = _setup(lens=(50,), chunks=(20,), cid=83)
    base = _prefill(w, L, kc, vc, pq)
    pos = _positions(w, pq)
    r = 7                                             # position 37 of 50
    kc2, vc2 = kc.copy(), vc.copy()
    n = w.num_blocks * w.num_kv_heads * 16 * w.head_dim
    later = np.arange(pos[r] + 1, 50)
    # rewrite the later slots with other values through the oracle's own write
    noise = syn.f32_to_bf16_bits(np.full((later.size, w.num_kv_heads, w.head_dim), 3.0, np.float32))
    oracle.cache_write(noise, noise, kc2, vc2, E4M3, w.slot_mapping[later], w.num_kv_heads,
                       w.head_dim, 16, w.num_blocks, L.k_scale, L.v_scale)
    assert not np.array_equal(kc, kc2) and kc2.size == n
    after = _prefill(w, L, kc2, vc2, pq)
    np.testing.assert_array_equal(after[: r + 1], base[: r + 1])
    assert np.abs(after[r + 1:] - base[r + 1:]).max() > 1e-3
    own = np.array([pos[r]])
    kc3, vc3 = kc.copy(), vc.copy()
    oracle.cache_write(noise[:1], noise[:1], kc3, vc3, E4M3, w.slot_mapping[own], w.num_kv_heads,
                       w.head_dim, 16, w.num_blocks, L.k_scale, L.v_scale)
    assert np.abs(_prefill(w, L, kc3, vc3, pq)[r] - base[r]).max() > 1e-3


def test_chunked_prefill_equals_one_chunk():
    """A chunk of n rows equals two calls: the first n1 rows against the context without
    the last n - n1 tokens, then the rest against the whole context."""
    w, L, kc, vc, pq = _setup(lens=(70, 45), chunks=(30, 45), cid=84)
    whole = _prefill(w, L, kc, vc, pq)
    n1 = np.array([12, 20], np.int32)
    qsl1 = np.array([0, 12, 32], np.int32)
    first_rows = np.concatenate([np.arange(0, 12), np.arange(30, 50)])
    second_rows = np.concatenate([np.arange(12, 30), np.arange(50, 75)])
    first = oracle.paged_prefill(pq.q[first_rows], qsl1, kc, vc, E4M3, w.block_tables,
                                 w.context_lens - (pq.chunk_lens - n1), w.num_q_heads,
                                 w.num_kv_heads, w.head_dim, 16, L.k_scale, L.v_scale)
    qsl2 = np.array([0, 18, 43], np.int32)
    second = oracle.paged_prefill(pq.q[second_rows], qsl2, kc, vc, E4M3, w.block_tables,
                                  w.context_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, 16,
                                  L.k_scale, L.v_scale)
    np.testing.assert_array_equal(first, whole[first_rows])
    np.testing.assert_array_equal(second, whole[second_rows])


def test_matrix_form_over_unpaged_rows():
    """bf16 cache (stored values are the inputs): causal masked softmax(Q K^T / sqrt(d)) V
    evaluated as whole matrices in numpy over the unpaged K/V rows of each sequence."""
    w, L, kc, vc, pq = _setup(lens=(23, 40), chunks=(23, 9), Hq=6, Hkv=3, D=64, cid=85,
                              cache=BF16)
    got = _prefill(w, L, kc, vc, pq, cache=BF16)
    g = w.num_q_heads // w.num_kv_heads
    for b in range(w.num_seqs):
        Lb = int(w.context_lens[b])
        rows = slice(w.seq_offsets[b], w.seq_offsets[b] + Lb)
        K = syn.bf16_bits_to_f32(L.k[rows]).astype(np.float64)        # [Lb][Hkv][D]
        V = syn.bf16_bits_to_f32(L.v[rows]).astype(np.float64)
        a, e = pq.query_start_loc[b], pq.query_start_loc[b + 1]
        Q = syn.bf16_bits_to_f32(pq.q[a:e]).astype(np.float64)        # [n][Hq][D]
        qpos = Lb - (e - a) + np.arange(e - a)
        allowed = np.arange(Lb)[None, :] <= qpos[:, None]             # [n][Lb]
        for hq in range(w.num_q_heads):
            S = Q[:, hq, :] @ K[:, hq // g, :].T / np.sqrt(w.head_dim)
            S = np.where(allowed, S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            np.testing.assert_allclose(got[a:e, hq], P @ V[:, hq // g, :], rtol=1e-12, atol=1e-12)


def test_degenerate_rows():
    """A sequence with no chunk contributes no rows; a row placed before position 0 (a
    chunk longer than the context) attends to nothing and is zero; a single-token chunk is
    the decode of the whole context."""
    w, L, kc, vc, pq = _setup(lens=(20, 30, 12), chunks=(0, 1, 12), cid=86)
    out = _prefill(w, L, kc, vc, pq)
    assert out.shape[0] == 13
    pairs = np.array([(1, hq) for hq in range(w.num_q_heads)], np.int32)
    q = w.q.copy()
    q[1] = pq.q[0]
    dec = oracle.paged_decode_pairs(pairs, q, kc, vc, E4M3, w.block_tables, w.context_lens,
                                    w.num_q_heads, w.num_kv_heads, w.head_dim, 16, L.k_scale,
                                    L.v_scale)
    np.testing.assert_array_equal(out[0], dec)
    lens = w.context_lens.copy()
    lens[2] = 5                                      # 12 rows, positions -7 .. 4
    short = _prefill(w, L, kc, vc, pq, lens=lens)
    assert not short[1:8].any() and np.abs(short[8:]).max() > 0
