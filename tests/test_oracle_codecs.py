"""Pins for the oracle's E5M2 and INT8 codecs and the cache paths that use them: torch's
float8_e5m2 decoder and rounding, brute-force nearest-value search, numpy's rint and
clip, and the pinned E4M3 path on values every codec holds exactly."""
import numpy as np
import torch

import oracle
import synthetic as syn

E4M3, E5M2, INT8 = oracle.CACHE_E4M3, oracle.CACHE_E5M2, oracle.CACHE_INT8


def _all_bf16_f32():
    return syn.bf16_bits_to_f32(np.arange(65536, dtype=np.uint16))


np.seterr(invalid="ignore", over="ignore")   # NaN and inf inputs are part of the sweeps


def test_e5m2_decode_matches_torch_on_every_code():
    c = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(c).view(torch.float8_e5m2).double().numpy()
    np.testing.assert_array_equal(oracle.e5m2_decode(c), ref)


def test_e5m2_format_facts():
    d = oracle.e5m2_decode(np.arange(256, dtype=np.uint8))
    assert np.nanmax(d[np.isfinite(d)]) == 57344.0                 # largest finite
    assert d[1] == 2.0 ** -16 and d[4] == 2.0 ** -14               # smallest subnormal / normal
    assert np.isinf(d[0x7C]) and np.isnan(d[0x7D]) and np.isnan(d[0x7F])
    assert np.signbit(d[0x80]) and d[0x80] == 0.0


def test_e5m2_encode_matches_torch_rounding_in_range():
    y = _all_bf16_f32().astype(np.float64)
    y = np.concatenate([y, y * 3.0 / 7.0, y * 1.0001])
    ok = np.isfinite(y) & (np.abs(y) <= 57344.0)
    ref = torch.from_numpy(y[ok].astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e5m2_encode(y[ok]), ref)


def test_e5m2_encode_is_the_nearest_code_by_brute_force():
    """Every bf16 value at several scales: the code is the nearest finite value (ties to the
    even code), saturating at 57344."""
    mags = oracle.e5m2_decode(np.arange(0x7C, dtype=np.uint8))   # +0 .. 57344, increasing
    for scale in (1.0, 0.37, 1e-3, 250.0):
        y = (_all_bf16_f32() / np.float32(scale)).astype(np.float64)
        y = y[np.isfinite(y)]
        a = np.minimum(np.abs(y), 57344.0)
        idx = np.searchsorted(mags, a)                            # mags[idx-1] < a <= mags[idx]
        hi = np.minimum(idx, len(mags) - 1)
        lo = np.maximum(hi - 1, 0)
        dlo, dhi = a - mags[lo], mags[hi] - a
        pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(hi % 2 == 0, hi, lo)))
        pick = np.where(a == mags[hi], hi, pick)
        want = pick.astype(np.uint8) | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
        np.testing.assert_array_equal(oracle.e5m2_encode(y), want)


def test_e5m2_special_values():
    enc = lambda v: int(oracle.e5m2_encode(np.array([v]))[0])
    assert enc(np.inf) == 0x7B and enc(-np.inf) == 0xFB and enc(1e9) == 0x7B
    assert enc(61439.0) == 0x7B and enc(57344.0) == 0x7B
    assert enc(np.nan) == 0x7F and enc(-np.nan) == 0xFF
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(2.0 ** -17) == 0x00 and enc(3 * 2.0 ** -17) == 0x02   # ties to even


def test_int8_encode_is_rint_and_clip():
    y = np.concatenate([_all_bf16_f32().astype(np.float64), np.arange(-300, 300.5, 0.25)])
    y = y[np.isfinite(y)]
    want = np.clip(np.rint(y), -127, 127).astype(np.int8).view(np.uint8)
    np.testing.assert_array_equal(oracle.int8_encode(y), want)
    assert oracle.int8_encode(np.array([np.nan]))[0] == 0
    assert oracle.int8_encode(np.array([np.inf, -np.inf])).view(np.int8).tolist() == [127, -127]
    np.testing.assert_array_equal(oracle.int8_decode(np.arange(256, dtype=np.uint8)),
                                  np.arange(256, dtype=np.uint8).view(np.int8).astype(np.float64))


def test_int8_hand_ties_and_clamp():
    """Hand values: halves round to the even integer (2.5 -> 2, 3.5 -> 4, -3.5 -> -4,
    -2.5 -> -2, 0.5 -> 0, -0.5 -> 0), just off a half rounds to nearest, 126.5 -> 126 and
    127.5 -> 127 (the even neighbour 128 clamps to 127), -127.5 and below clamp to -127
    (never -128)."""
    cases = {2.5: 2, 3.5: 4, -3.5: -4, -2.5: -2, 0.5: 0, -0.5: 0, 1.5: 2, -1.5: -2,
             2.5000001: 3, 2.4999999: 2, 126.5: 126, 127.5: 127, 128.0: 127, -127.5: -127,
             -128.0: -127, -1e30: -127, 0.0: 0, -0.0: 0}
    got = oracle.int8_encode(np.array(list(cases), dtype=np.float64)).view(np.int8).tolist()
    assert got == list(cases.values())


def _small_integer_workload(cid):
    """Elements in {0, +-1, +-2, +-3, +-4}: with scale 1 every codec stores them exactly."""
    w = syn.make_workload(f"codec-{cid}", cid, num_q_heads=8, num_kv_heads=2, head_dim=64,
                          context_lens=[37, 120])
    rng = np.random.default_rng(cid)
    k = syn.f32_to_bf16_bits(rng.integers(-4, 5, (w.num_tokens, 2, 64)).astype(np.float32))
    v = syn.f32_to_bf16_bits(rng.integers(-4, 5, (w.num_tokens, 2, 64)).astype(np.float32))
    return w, k, v


def test_codec_caches_decode_like_e4m3_on_exact_values():
    """Same slots and layout, same dequantised values: decode attention over an E5M2 or
    INT8 cache equals the pinned E4M3 path when all three hold the values exactly, and the
    E4M3 bytes of the codec write equal oracle.cache_write's."""
    w, k, v = _small_integer_workload(96)
    n = w.num_blocks * 2 * 16 * 64
    caches = {}
    for codec in (E4M3, E5M2, INT8):
        kc, vc = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
        oracle.cache_write_codec(k, v, kc, vc, codec, w.slot_mapping, 2, 64, 16, w.num_blocks, 1.0, 1.0)
        caches[codec] = (kc, vc)
    ek, ev = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    oracle.cache_write(k, v, ek, ev, E4M3, w.slot_mapping, 2, 64, 16, w.num_blocks, 1.0, 1.0)
    assert np.array_equal(caches[E4M3][0], ek) and np.array_equal(caches[E4M3][1], ev)
    outs = {c: oracle.paged_decode(w.q, *caches[c], c, w.block_tables, w.context_lens, 8, 2, 64,
                                   16, 1.0, 1.0) for c in caches}
    np.testing.assert_array_equal(outs[E5M2], outs[E4M3])
    np.testing.assert_array_equal(outs[INT8], outs[E4M3])


def test_codec_write_bytes_are_the_codec_of_each_element():
    """Every byte of a codec write is the codec's encoder applied to its element's f32
    quotient, at the element's position in the documented tile layout (the layout the
    E4M3 pins fix; the test above shows the codec write uses the E4M3 write's slots)."""
    w = syn.make_workload("codec-pos", 97, num_q_heads=4, num_kv_heads=2, head_dim=64,
                          context_lens=[20, 9])
    L = w.layers[0]
    n = w.num_blocks * 2 * 16 * 64
    for codec, enc in ((E5M2, oracle.e5m2_encode), (INT8, oracle.int8_encode)):
        for scale in (0.05, 1.0):
            kc, vc = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
            oracle.cache_write_codec(L.k, L.v, kc, vc, codec, w.slot_mapping, 2, 64, 16,
                                     w.num_blocks, scale, scale)
            for cache, rows in ((kc, L.k), (vc, L.v)):
                want = np.zeros(n, np.uint8)
                q = (syn.bf16_bits_to_f32(rows) / np.float32(scale)).astype(np.float64)
                codes = enc(q)
                pos = _positions(w, cache is vc)
                want[pos] = codes.reshape(-1)
                assert np.array_equal(cache, want)


def _positions(w, is_value):
    """Byte position of every (token, head, channel) element in the documented layout."""
    T, Hkv, D = w.num_tokens, 2, 64
    t, h, i = np.meshgrid(np.arange(T), np.arange(Hkv), np.arange(D), indexing="ij")
    slot = w.slot_mapping[t]
    blk, off = slot // 16, slot % 16
    tile = (blk * Hkv + h) * 16 * D
    if is_value:
        return (tile + i * 16 + off).reshape(-1)
    # key tile: (slot quad, chunk, slot in quad, channel quarter), 16-byte chunks; D = 64
    q = D // 4
    g, wv = i // q, i % q
    return (tile + (((off // 4) * (q // 16) + wv // 16) * 4 + off % 4) * 64 + g * 16 + wv % 16).reshape(-1)
