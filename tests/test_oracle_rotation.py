"""Pins for the oracle's Hadamard rotation path (K and V rotated before caching, attention
in the rotated space, output rotated back).  Each pin fixes the oracle by something other
than itself: the Sylvester closed form, orthonormality, exact f32 arithmetic on inputs
whose sums are exact, the unrotated (pinned) oracle, and the outlier-spreading effect."""
import numpy as np

import oracle
import synthetic as syn

E4M3, BF16 = oracle.CACHE_E4M3, oracle.CACHE_BF16


def _sylvester(d):
    i = np.arange(d)
    pop = np.array([[bin(a & b).count("1") for b in i] for a in i])
    return np.where(pop % 2 == 0, 1.0, -1.0) / np.sqrt(d)


def test_rotation_is_the_normalised_sylvester_matrix():
    for d in (2, 4, 8, 64, 128, 256):
        np.testing.assert_allclose(oracle.hadamard_f64(np.eye(d)), _sylvester(d), rtol=0, atol=1e-15)


def test_rotation_is_its_own_inverse_and_keeps_dot_products():
    rng = np.random.default_rng(3)
    for d in (64, 128, 256):
        x = rng.standard_normal((5, d))
        y = rng.standard_normal((5, d))
        np.testing.assert_allclose(oracle.hadamard_f64(oracle.hadamard_f64(x)), x, atol=1e-13)
        np.testing.assert_allclose((oracle.hadamard_f64(x) * oracle.hadamard_f64(y)).sum(1),
                                   (x * y).sum(1), rtol=1e-12, atol=1e-12)


def test_f32_rotation_within_its_rounding_bound():
    """Each butterfly stage rounds once (relative 2^-24), then the scale rounds: the f32
    result is within (log2 d + 1) * 2^-24 * (sum |x|)/sqrt(d) of the exact product, and
    exact on integer inputs whose partial sums fit in f32 at d = 64 and 256 (scale a power
    of two)."""
    rng = np.random.default_rng(4)
    for d in (64, 128, 256):
        x = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(rng.standard_normal((20, d)).astype(np.float32)))
        got = oracle.hadamard_f32(x).astype(np.float64)
        exact = x.astype(np.float64) @ _sylvester(d).T
        bound = (np.log2(d) + 2) * 2.0 ** -24 * np.abs(x).sum(1, keepdims=True) / np.sqrt(d)
        assert np.all(np.abs(got - exact) <= bound)
    for d in (64, 256):
        z = rng.integers(-50, 51, (10, d)).astype(np.float32)
        np.testing.assert_array_equal(oracle.hadamard_f32(z).astype(np.float64),
                                      z.astype(np.float64) @ _sylvester(d).T)


def _exact_workload(cache, cid=91):
    """d = 64 rows x = H r with r in {-1, 0, 1}: x is a multiple of 1/8 below 8 in
    magnitude (exact in bf16), and the f32 rotation of x gives r back exactly."""
    D, Hkv, Hq = 64, 2, 8
    w = syn.make_workload(f"rot-exact-{cache}", cid, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                          context_lens=[37, 90], layers=(("l0", 0, cache),))
    rng = np.random.default_rng(cid)
    H = _sylvester(D)
    r_k = rng.integers(-1, 2, (w.num_tokens, Hkv, D)).astype(np.float64)
    r_v = rng.integers(-1, 2, (w.num_tokens, Hkv, D)).astype(np.float64)
    xk, xv = r_k @ H.T, r_v @ H.T                     # H is symmetric
    to_bits = lambda a: syn.f32_to_bf16_bits(a.astype(np.float32))
    assert np.array_equal(syn.bf16_bits_to_f32(to_bits(xk)), xk.astype(np.float32))
    return w, to_bits(xk), to_bits(xv), to_bits(r_k), to_bits(r_v)


def _caches(w, cdt):
    n = w.num_blocks * w.num_kv_heads * 16 * w.head_dim
    dt = np.uint8 if cdt == E4M3 else np.uint16
    return np.zeros(n, dt), np.zeros(n, dt)


def test_rotated_write_is_the_plain_write_of_the_rotated_rows():
    for cdt, cache in ((E4M3, syn.E4M3), (BF16, syn.BF16)):
        w, xk, xv, rk, rv = _exact_workload(cache)
        a_k, a_v = _caches(w, cdt)
        oracle.cache_write_rotated(xk, xv, a_k, a_v, cdt, w.slot_mapping, w.num_kv_heads, w.head_dim,
                                   16, w.num_blocks, 0.0123, 0.0071)
        b_k, b_v = _caches(w, cdt)
        oracle.cache_write(rk, rv, b_k, b_v, cdt, w.slot_mapping, w.num_kv_heads, w.head_dim, 16,
                           w.num_blocks, 0.0123, 0.0071)
        assert np.array_equal(a_k, b_k) and np.array_equal(a_v, b_v)


def test_rotated_decode_equals_plain_decode_when_the_rotation_is_exact():
    """bf16 cache: the rotated cache holds r = H x exactly, so attention in the rotated
    space, rotated back, is the plain attention over x (up to fp64 rounding)."""
    w, xk, xv, rk, rv = _exact_workload(syn.BF16, cid=92)
    rot_k, rot_v = _caches(w, BF16)
    oracle.cache_write_rotated(xk, xv, rot_k, rot_v, BF16, w.slot_mapping, w.num_kv_heads,
                               w.head_dim, 16, w.num_blocks, 1.0, 1.0)
    pl_k, pl_v = _caches(w, BF16)
    oracle.cache_write(xk, xv, pl_k, pl_v, BF16, w.slot_mapping, w.num_kv_heads, w.head_dim, 16,
                       w.num_blocks, 1.0, 1.0)
    for window in (0, 10):
        got = oracle.paged_decode_rotated(w.q, rot_k, rot_v, BF16, w.block_tables, w.context_lens,
                                          w.num_q_heads, w.num_kv_heads, w.head_dim, 16, 1.0, 1.0,
                                          window)
        ref = oracle.paged_decode(w.q, pl_k, pl_v, BF16, w.block_tables, w.context_lens,
                                  w.num_q_heads, w.num_kv_heads, w.head_dim, 16, 1.0, 1.0, window)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_rotation_spreads_outliers_and_lowers_the_fp8_error():
    """The effect the rotation is for: with 1 % of key channels scaled x8 (per-tensor amax
    scales), fp8 attention through the rotated cache is closer to the exact bf16 attention
    than through the plain cache, on every seed tried."""
    for cid in (93, 94, 95):
        w = syn.make_workload(f"rot-outliers-{cid}", cid, num_q_heads=8, num_kv_heads=2,
                              head_dim=128, context_lens=[300, 700], outlier_frac=0.01,
                              outlier_mult=8.0)
        L = w.layers[0]
        ref_k, ref_v = _caches(w, BF16)
        oracle.cache_write(L.k, L.v, ref_k, ref_v, BF16, w.slot_mapping, 2, 128, 16, w.num_blocks,
                           1.0, 1.0)
        ref = oracle.paged_decode(w.q, ref_k, ref_v, BF16, w.block_tables, w.context_lens, 8, 2,
                                  128, 16, 1.0, 1.0)
        pk, pv = _caches(w, E4M3)
        oracle.cache_write(L.k, L.v, pk, pv, E4M3, w.slot_mapping, 2, 128, 16, w.num_blocks,
                           L.k_scale, L.v_scale)
        plain = oracle.paged_decode(w.q, pk, pv, E4M3, w.block_tables, w.context_lens, 8, 2, 128, 16,
                                    L.k_scale, L.v_scale)
        # calibrated scales of the rotated rows
        rk = oracle.hadamard_f32(syn.bf16_bits_to_f32(L.k))
        rv = oracle.hadamard_f32(syn.bf16_bits_to_f32(L.v))
        ks = float(np.float32(np.abs(rk).max()) / np.float32(448.0))
        vs = float(np.float32(np.abs(rv).max()) / np.float32(448.0))
        qk, qv = _caches(w, E4M3)
        oracle.cache_write_rotated(L.k, L.v, qk, qv, E4M3, w.slot_mapping, 2, 128, 16, w.num_blocks,
                                   ks, vs)
        pairs = np.array([(b, hq) for b in range(2) for hq in range(8)], np.int32)
        rot = oracle.paged_decode_rotated_pairs(pairs, w.q, qk, qv, E4M3, w.block_tables,
                                                w.context_lens, 8, 2, 128, 16, ks, vs).reshape(2, 8, 128)
        e_plain = np.abs(plain - ref).max()
        e_rot = np.abs(rot - ref).max()
        assert e_rot < e_plain, (cid, e_rot, e_plain)


# ---- per-kv-head scales on the rotated path

def test_rotated_per_head_write_is_the_per_tensor_rotated_write_head_by_head():
    w = syn.make_workload("rot-ph-write", 96, num_q_heads=12, num_kv_heads=3, head_dim=128,
                          context_lens=[70, 300], outlier_frac=0.01)
    L = w.layers[0]
    ks = syn.spread_head_scales(w.num_kv_heads, 96)
    vs = syn.spread_head_scales(w.num_kv_heads, 97)
    assert len(set(ks.tolist())) == w.num_kv_heads        # distinct, so a wrong head shows
    kc, vc = _caches(w, E4M3)
    oracle.cache_write_rotated_per_head(L.k, L.v, kc, vc, E4M3, w.slot_mapping, w.num_kv_heads,
                                        w.head_dim, 16, w.num_blocks, ks, vs)
    tiles = lambda c: c.reshape(w.num_blocks, w.num_kv_heads, -1)
    for h in range(w.num_kv_heads):
        pk, pv = _caches(w, E4M3)
        oracle.cache_write_rotated(L.k, L.v, pk, pv, E4M3, w.slot_mapping, w.num_kv_heads, w.head_dim,
                                   16, w.num_blocks, float(ks[h]), float(vs[h]))
        assert np.array_equal(tiles(kc)[:, h], tiles(pk)[:, h]), f"key head {h}"
        assert np.array_equal(tiles(vc)[:, h], tiles(pv)[:, h]), f"value head {h}"


def test_rotated_per_head_decode_equals_plain_decode_when_the_codes_are_exact():
    """Rows x = H r (r in {-1, 0, 1}) rotate back to r exactly in f32; with power-of-two
    scales that differ per kv head, r / s is an exact e4m3 code, so the rotated fp8 cache
    dequantises to r with each head's own scales, and attention in the rotated space, rotated
    back, is the plain attention over x held in a bf16 cache.  A scale taken from the wrong
    head, or a scale applied twice, moves the result off it."""
    w, xk, xv, rk, rv = _exact_workload(syn.E4M3, cid=98)
    ks = np.array([0.25, 0.5], np.float32)
    vs = np.array([0.125, 1.0], np.float32)
    rot_k, rot_v = _caches(w, E4M3)
    oracle.cache_write_rotated_per_head(xk, xv, rot_k, rot_v, E4M3, w.slot_mapping,
                                        w.num_kv_heads, w.head_dim, 16, w.num_blocks, ks, vs)
    pl_k, pl_v = _caches(w, BF16)
    oracle.cache_write(xk, xv, pl_k, pl_v, BF16, w.slot_mapping, w.num_kv_heads, w.head_dim, 16,
                       w.num_blocks, 1.0, 1.0)
    for window in (0, 10):
        got = oracle.paged_decode_rotated_per_head(w.q, rot_k, rot_v, E4M3, w.block_tables,
                                                   w.context_lens, w.num_q_heads, w.num_kv_heads,
                                                   w.head_dim, 16, ks, vs, window)
        ref = oracle.paged_decode(w.q, pl_k, pl_v, BF16, w.block_tables, w.context_lens,
                                  w.num_q_heads, w.num_kv_heads, w.head_dim, 16, 1.0, 1.0, window)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)
    # the same cache read with the heads' scales swapped is measurably different
    ref0 = oracle.paged_decode(w.q, pl_k, pl_v, BF16, w.block_tables, w.context_lens,
                               w.num_q_heads, w.num_kv_heads, w.head_dim, 16, 1.0, 1.0, 0)
    bad = oracle.paged_decode_rotated_per_head(w.q, rot_k, rot_v, E4M3, w.block_tables,
                                               w.context_lens, w.num_q_heads, w.num_kv_heads,
                                               w.head_dim, 16, ks[::-1].copy(), vs[::-1].copy(), 0)
    assert np.abs(bad - ref0).max() > 1e-3


# ---- prefill over a rotated cache

def test_rotated_prefill_equals_plain_prefill_when_the_rotation_is_exact():
    """bf16 cache holding r = H x exactly: every chunk row's rotated prefill, rotated back,
    is the plain prefill over x (up to fp64 rounding), with and without a window."""
    w, xk, xv, rk, rv = _exact_workload(syn.BF16, cid=99)
    rot_k, rot_v = _caches(w, BF16)
    oracle.cache_write_rotated(xk, xv, rot_k, rot_v, BF16, w.slot_mapping, w.num_kv_heads,
                               w.head_dim, 16, w.num_blocks, 1.0, 1.0)
    pl_k, pl_v = _caches(w, BF16)
    oracle.cache_write(xk, xv, pl_k, pl_v, BF16, w.slot_mapping, w.num_kv_heads, w.head_dim, 16,
                       w.num_blocks, 1.0, 1.0)
    pq = syn.prefill_queries(w, [9, 40], 99)
    for window in (0, 10):
        args = (w.block_tables, w.context_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, 16,
                1.0, 1.0, window)
        got = oracle.paged_prefill_rotated(pq.q, pq.query_start_loc, rot_k, rot_v, BF16, *args)
        ref = oracle.paged_prefill(pq.q, pq.query_start_loc, pl_k, pl_v, BF16, *args)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_rotated_prefill_last_row_is_the_rotated_decode():
    """A chunk's last row sits at the context's last position, so its rotated prefill is
    the rotated decode of that token, bit for bit (the same fp64 steps)."""
    w = syn.make_workload("rot-pf-dec", 100, num_q_heads=8, num_kv_heads=2, head_dim=128,
                          context_lens=[70, 300], outlier_frac=0.01)
    L = w.layers[0]
    kc, vc = _caches(w, E4M3)
    oracle.cache_write_rotated(L.k, L.v, kc, vc, E4M3, w.slot_mapping, 2, 128, 16, w.num_blocks,
                               0.02, 0.03)
    pq = syn.prefill_queries(w, [5, 12], 100)
    q = w.q.copy()
    last = pq.query_start_loc[1:] - 1
    q[0], q[1] = pq.q[last[0]], pq.q[last[1]]
    for window in (0, 33):
        pf = oracle.paged_prefill_rotated_pairs(
            np.array([(r, hq) for r in last for hq in range(8)], np.int32), pq.q,
            pq.query_start_loc, kc, vc, E4M3, w.block_tables, w.context_lens, 8, 2, 128, 16, 0.02,
            0.03, window)
        dec = oracle.paged_decode_rotated(q, kc, vc, E4M3, w.block_tables, w.context_lens, 8, 2, 128,
                                          16, 0.02, 0.03, window)
        assert np.array_equal(pf, dec.reshape(-1, 128))
