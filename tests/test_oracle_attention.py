"""Pins for the oracle's paged decode attention and cache write (CPU only).

The pages print no attention input/output example, so the oracle is pinned by
closed forms and invariants that a dropped term, a wrong sign, a wrong index or
a transposed operand would break: single-row and two-row closed forms, uniform
weights, windows, exact power-of-two scaling, independence of block placement,
GQA head grouping, a hand case, and a 60-digit decimal evaluation of tiny cases.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import synthetic as syn

E4M3, BF16 = 0, 1


def _dec(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def key_tile_offset(t, i, D, eb):
    """Element offset inside a key tile (16 slots x D channels): 16-byte chunks ordered
    (slot quad, chunk, slot within quad, channel quarter), as the library header states."""
    q = D // 4
    g = i // q
    w = (i % q) * eb
    K = min(16, q * eb)
    C = q * eb // K
    byte = (((t // 4) * C + w // K) * 4 + t % 4) * (4 * K) + g * K + w % K
    return byte // eb


def test_key_tile_layout_is_a_bijection_and_token_major_at_d64():
    for D in (8, 16, 64, 128, 256):
        for eb in (1, 2):
            t = np.arange(16)[:, None]
            i = np.arange(D)[None, :]
            off = key_tile_offset(t, i, D, eb)
            assert sorted(off.reshape(-1).tolist()) == list(range(16 * D))
    t = np.arange(16)[:, None]
    i = np.arange(64)[None, :]
    assert np.array_equal(key_tile_offset(t, i, 64, 1), t * 64 + i)
    # a 16-byte chunk holds consecutive channels of one slot
    off = key_tile_offset(np.full(16, 5), np.arange(32, 48), 128, 1)
    assert np.array_equal(np.diff(off), np.ones(15))


class Paged:
    """A tiny hand-built paged cache: sequences laid out with an explicit block table."""

    def __init__(self, oracle_mod, lens, Hq, Hkv, D, bs=16, seed=0, cache_dtype=E4M3,
                 k_scale=0.05, v_scale=0.03, slack=3, std=1.0):
        self.o = oracle_mod
        rng = np.random.default_rng(seed)
        self.lens = np.array(lens, dtype=np.int32)
        self.Hq, self.Hkv, self.D, self.bs = Hq, Hkv, D, bs
        self.cache_dtype, self.k_scale, self.v_scale = cache_dtype, k_scale, v_scale
        nb = [(L + bs - 1) // bs for L in lens]
        self.NB = sum(nb) + slack
        perm = rng.permutation(self.NB).astype(np.int32)
        self.bt = np.full((len(lens), max(1, max(nb))), perm[-1], dtype=np.int32)
        cur = 0
        for b, n in enumerate(nb):
            self.bt[b, :n] = perm[cur:cur + n]
            cur += n
        T = int(sum(lens))
        self.k = syn.f32_to_bf16_bits((rng.standard_normal((T, Hkv, D)) * std).astype(np.float32))
        self.v = syn.f32_to_bf16_bits((rng.standard_normal((T, Hkv, D)) * std).astype(np.float32))
        self.q = syn.f32_to_bf16_bits(rng.standard_normal((len(lens), Hq, D)).astype(np.float32))
        self.offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        self.slots = np.concatenate([
            self.bt[b, np.arange(L) // bs].astype(np.int64) * bs + np.arange(L) % bs
            for b, L in enumerate(lens)]) if T else np.zeros(0, np.int64)
        self.write()

    def write(self):
        dt = np.uint8 if self.cache_dtype == E4M3 else np.uint16
        poison = 0x7F if self.cache_dtype == E4M3 else 0x7FC0
        n = self.NB * self.Hkv * self.bs * self.D
        self.kc = np.full(n, poison, dtype=dt)
        self.vc = np.full(n, poison, dtype=dt)
        self.o.cache_write(self.k, self.v, self.kc, self.vc, self.cache_dtype, self.slots,
                           self.Hkv, self.D, self.bs, self.NB, self.k_scale, self.v_scale)

    def decode(self, window=0, k_scale=None, v_scale=None):
        return self.o.paged_decode(self.q, self.kc, self.vc, self.cache_dtype, self.bt, self.lens,
                                   self.Hq, self.Hkv, self.D, self.bs,
                                   self.k_scale if k_scale is None else k_scale,
                                   self.v_scale if v_scale is None else v_scale, window)

    def rows(self, b, h):
        """Dequantised logical K, V rows of (seq b, kv head h), gathered by the test itself."""
        L = int(self.lens[b])
        j = np.arange(L)
        blk = self.bt[b, j // self.bs].astype(np.int64)
        off = j % self.bs
        i = np.arange(self.D)
        kidx = blk[:, None] * self.Hkv * self.bs * self.D + h * self.bs * self.D + \
            key_tile_offset(off[:, None], i[None, :], self.D, 1 if self.cache_dtype == E4M3 else 2)
        vidx = ((blk[:, None] * self.Hkv + h) * self.D + i[None, :]) * self.bs + off[:, None]
        if self.cache_dtype == E4M3:
            return _dec(self.kc[kidx]) * self.k_scale, _dec(self.vc[vidx]) * self.v_scale
        return (syn.bf16_bits_to_f32(self.kc[kidx]).astype(np.float64),
                syn.bf16_bits_to_f32(self.vc[vidx]).astype(np.float64))

    def qf(self, b, hq):
        return syn.bf16_bits_to_f32(self.q[b, hq]).astype(np.float64)


def test_hand_case_d2(oracle_mod):
    """q=(1,0), K=I, V=I, scale 1: weights are logistic(+-1/sqrt2)."""
    out = oracle_mod.attention_rows(np.array([1.0, 0.0]), np.eye(2), np.eye(2))
    a = 1.0 / (1.0 + math.exp(-1.0 / math.sqrt(2.0)))
    assert abs(out[0] - a) < 1e-15 and abs(out[1] - (1 - a)) < 1e-15
    assert abs(out[0] - 0.66976155) < 1e-8


def test_single_row_returns_value(oracle_mod):
    rng = np.random.default_rng(1)
    q, K, V = rng.standard_normal(8), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    assert np.array_equal(oracle_mod.attention_rows(q, K, V), V[0])


def test_two_row_closed_form(oracle_mod):
    rng = np.random.default_rng(2)
    for _ in range(50):
        D = int(rng.integers(1, 9))
        q, K, V = rng.standard_normal(D) * 3, rng.standard_normal((2, D)), rng.standard_normal((2, D))
        delta = (q @ K[0] - q @ K[1]) / math.sqrt(D)
        w0 = 1.0 / (1.0 + math.exp(-delta))
        want = w0 * V[0] + (1.0 - w0) * V[1]
        assert np.allclose(oracle_mod.attention_rows(q, K, V), want, rtol=0, atol=1e-14)


def test_zero_query_gives_mean_of_values(oracle_mod):
    rng = np.random.default_rng(3)
    K, V = rng.standard_normal((37, 16)), rng.standard_normal((37, 16))
    out = oracle_mod.attention_rows(np.zeros(16), K, V)
    assert np.allclose(out, V.mean(axis=0), rtol=0, atol=1e-14)


def test_equal_keys_give_mean_and_constant_values_are_returned(oracle_mod):
    rng = np.random.default_rng(4)
    q = rng.standard_normal(16)
    K = np.tile(rng.standard_normal(16), (29, 1))
    V = rng.standard_normal((29, 16))
    assert np.allclose(oracle_mod.attention_rows(q, K, V), V.mean(axis=0), rtol=0, atol=1e-14)
    # weights sum to one: a constant value row comes back unchanged
    K2 = rng.standard_normal((29, 16)) * 4
    Vc = np.full((29, 16), 0.7)
    assert np.allclose(oracle_mod.attention_rows(q, K2, Vc), 0.7, rtol=0, atol=1e-15)


def test_dominant_key(oracle_mod):
    rng = np.random.default_rng(5)
    q = rng.standard_normal(8)
    K = rng.standard_normal((20, 8))
    K[13] = q * 200.0
    V = rng.standard_normal((20, 8))
    assert np.allclose(oracle_mod.attention_rows(q, K, V), V[13], rtol=0, atol=1e-12)


def test_empty_rows_give_zero(oracle_mod):
    out = oracle_mod.attention_rows(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)))
    assert np.array_equal(out, np.zeros(4))


def _decimal_attention(q, K, V):
    getcontext().prec = 60
    D = len(q)
    qd = [Decimal(float(x)) for x in q]
    s = [sum(qd[i] * Decimal(float(K[j][i])) for i in range(D)) / Decimal(D).sqrt()
         for j in range(len(K))]
    m = max(s)
    w = [(x - m).exp() for x in s]
    Z = sum(w)
    return [float(sum(w[j] * Decimal(float(V[j][i])) for j in range(len(K))) / Z) for i in range(D)]


def test_tiny_cases_against_60_digit_decimal(oracle_mod):
    rng = np.random.default_rng(6)
    for _ in range(40):
        n, D = int(rng.integers(1, 7)), int(rng.integers(1, 6))
        q = rng.standard_normal(D) * 2
        K, V = rng.standard_normal((n, D)) * 2, rng.standard_normal((n, D))
        want = np.array(_decimal_attention(q, K, V))
        got = oracle_mod.attention_rows(q, K, V)
        assert np.allclose(got, want, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------- paged ----

@pytest.mark.parametrize("cache_dtype,D", [(E4M3, 8), (BF16, 8), (E4M3, 128), (BF16, 64)])
def test_paged_equals_rows_gathered_by_test(oracle_mod, cache_dtype, D):
    P = Paged(oracle_mod, [1, 15, 16, 17, 50], Hq=6, Hkv=2, D=D, cache_dtype=cache_dtype)
    out = P.decode()
    g = P.Hq // P.Hkv
    for b in range(len(P.lens)):
        for hq in range(P.Hq):
            K, V = P.rows(b, hq // g)
            want = oracle_mod.attention_rows(P.qf(b, hq), K, V)
            assert np.array_equal(out[b, hq], want)


def test_paged_single_token_is_its_value(oracle_mod):
    P = Paged(oracle_mod, [1], Hq=4, Hkv=1, D=64)
    _, V = P.rows(0, 0)
    out = P.decode()
    for hq in range(4):
        assert np.array_equal(out[0, hq], V[0])


def test_window_of_one_and_covering_windows(oracle_mod):
    P = Paged(oracle_mod, [45, 33], Hq=4, Hkv=2, D=16)
    full = P.decode()
    assert np.array_equal(P.decode(window=45), full)
    assert np.array_equal(P.decode(window=1000), full)
    w1 = P.decode(window=1)
    for b, L in enumerate(P.lens):
        for hq in range(4):
            _, V = P.rows(b, hq // 2)
            assert np.array_equal(w1[b, hq], V[L - 1])


@pytest.mark.parametrize("window", [2, 5, 16, 17, 20])
def test_window_equals_attention_over_last_rows(oracle_mod, window):
    P = Paged(oracle_mod, [45, 33, 3], Hq=4, Hkv=2, D=16)
    out = P.decode(window=window)
    for b, L in enumerate(P.lens):
        for hq in range(4):
            K, V = P.rows(b, hq // 2)
            lo = max(0, int(L) - window)
            want = oracle_mod.attention_rows(P.qf(b, hq), K[lo:], V[lo:])
            assert np.array_equal(out[b, hq], want)


def test_empty_context_gives_zero(oracle_mod):
    P = Paged(oracle_mod, [0, 5], Hq=2, Hkv=1, D=8)
    out = P.decode()
    assert np.array_equal(out[0], np.zeros((2, 8)))
    assert np.all(np.abs(out[1]) > 0)


def test_value_scale_power_of_two_is_exact(oracle_mod):
    P = Paged(oracle_mod, [40], Hq=4, Hkv=1, D=16)
    base = P.decode()
    for k in (-3, 1, 5):
        assert np.array_equal(P.decode(v_scale=P.v_scale * 2.0 ** k), base * 2.0 ** k)


def test_key_scale_enters_the_scores(oracle_mod):
    """Scaling keys by c is the same as scaling the query by c (scores are bilinear)."""
    P = Paged(oracle_mod, [40], Hq=1, Hkv=1, D=8)
    K, V = P.rows(0, 0)
    out = P.decode(k_scale=P.k_scale * 4.0)
    want = oracle_mod.attention_rows(P.qf(0, 0) * 4.0, K, V)
    assert np.allclose(out[0, 0], want, rtol=0, atol=1e-14)


def test_block_placement_does_not_matter(oracle_mod):
    P = Paged(oracle_mod, [50, 20], Hq=4, Hkv=2, D=8, seed=9)
    base = P.decode()
    # move every physical block to a new place and rewrite the table accordingly
    rng = np.random.default_rng(10)
    newpos = rng.permutation(P.NB).astype(np.int32)
    tile = P.Hkv * P.bs * P.D
    kc, vc = np.empty_like(P.kc), np.empty_like(P.vc)
    for old in range(P.NB):
        kc[newpos[old] * tile:(newpos[old] + 1) * tile] = P.kc[old * tile:(old + 1) * tile]
        vc[newpos[old] * tile:(newpos[old] + 1) * tile] = P.vc[old * tile:(old + 1) * tile]
    P.kc, P.vc, P.bt = kc, vc, newpos[P.bt]
    assert np.array_equal(P.decode(), base)


def test_gqa_grouping(oracle_mod):
    P = Paged(oracle_mod, [30], Hq=6, Hkv=3, D=8, seed=11)
    P.q[0, 1] = P.q[0, 0]        # same group (kv head 0)
    P.q[0, 2] = P.q[0, 0]        # different group (kv head 1)
    out = P.decode()
    assert np.array_equal(out[0, 0], out[0, 1])
    assert not np.allclose(out[0, 0], out[0, 2])
    # overwriting kv head 2 changes only query heads 4 and 5
    before = out.copy()
    tile = P.bs * P.D
    for blk in range(P.NB):
        base = (blk * P.Hkv + 2) * tile
        P.kc[base:base + tile] = P.kc[base:base + tile][::-1]
    after = P.decode()
    assert np.array_equal(after[0, :4], before[0, :4])
    assert not np.allclose(after[0, 4:], before[0, 4:])


def test_tail_poison_is_never_read(oracle_mod):
    """Slots past L in the last block and the slack blocks hold NaN codes; the output is finite."""
    P = Paged(oracle_mod, [17, 31], Hq=2, Hkv=1, D=8)
    assert np.isnan(_dec(P.kc)).any()
    assert np.all(np.isfinite(P.decode()))


# -------------------------------------------------------- cache write ----

@pytest.mark.parametrize("D", [4, 128])
def test_cache_write_hand_layout(oracle_mod, D):
    Hkv, bs, NB = 2, 16, 4
    rng = np.random.default_rng(12)
    k = syn.f32_to_bf16_bits(rng.standard_normal((3, Hkv, D)).astype(np.float32))
    v = syn.f32_to_bf16_bits(rng.standard_normal((3, Hkv, D)).astype(np.float32))
    slots = np.array([5, 37, -1], dtype=np.int64)
    kc = np.full(NB * Hkv * bs * D, 0x7F, np.uint8)
    vc = np.full(NB * Hkv * bs * D, 0x7F, np.uint8)
    oracle_mod.cache_write(k, v, kc, vc, E4M3, slots, Hkv, D, bs, NB, 0.5, 0.25)
    want_k = np.full_like(kc, 0x7F)
    want_v = np.full_like(vc, 0x7F)
    for t, slot in enumerate([5, 37]):
        blk, off = slot // bs, slot % bs
        for h in range(Hkv):
            for i in range(D):
                want_k[(blk * Hkv + h) * bs * D + key_tile_offset(off, i, D, 1)] = \
                    oracle_mod.quantize(k[t, h, i:i + 1], 0.5)[0]
                want_v[((blk * Hkv + h) * D + i) * bs + off] = oracle_mod.quantize(v[t, h, i:i + 1], 0.25)[0]
    assert np.array_equal(kc, want_k) and np.array_equal(vc, want_v)
    # a code's value times the scale is the bf16 input rounded to e4m3 precision
    x = syn.bf16_bits_to_f32(k[0, 1, 2:3]).astype(np.float64)[0]
    code = kc[(0 * Hkv + 1) * bs * D + key_tile_offset(5, 2, D, 1)]
    assert abs(_dec(np.array([code]))[0] * 0.5 - x) <= abs(x) * 2.0 ** -4 + 2.0 ** -10 * 0.5


def test_cache_write_out_of_range_slots_write_nothing(oracle_mod):
    Hkv, D, bs, NB = 1, 8, 16, 2
    k = np.full((3, Hkv, D), 0x3F80, np.uint16)
    kc = np.full(NB * bs * D, 0x11, np.uint8)
    vc = np.full(NB * bs * D, 0x11, np.uint8)
    oracle_mod.cache_write(k, k, kc, vc, E4M3, np.array([-1, -7, NB * bs], np.int64),
                           Hkv, D, bs, NB, 1.0, 1.0)
    assert np.all(kc == 0x11) and np.all(vc == 0x11)


def test_cache_write_bf16_keeps_bits(oracle_mod):
    Hkv, D, bs, NB = 2, 8, 16, 2
    rng = np.random.default_rng(13)
    k = rng.integers(0, 65536, (4, Hkv, D)).astype(np.uint16)
    v = rng.integers(0, 65536, (4, Hkv, D)).astype(np.uint16)
    slots = np.array([0, 17, 31, 3], np.int64)
    kc = np.zeros(NB * Hkv * bs * D, np.uint16)
    vc = np.zeros(NB * Hkv * bs * D, np.uint16)
    oracle_mod.cache_write(k, v, kc, vc, BF16, slots, Hkv, D, bs, NB, 123.0, 456.0)
    for t, slot in enumerate(slots):
        blk, off = slot // bs, slot % bs
        for h in range(Hkv):
            assert np.array_equal(kc[(blk * Hkv + h) * bs * D + key_tile_offset(off, np.arange(D), D, 2)], k[t, h])
            assert np.array_equal(vc[((blk * Hkv + h) * D + np.arange(D)) * bs + off], v[t, h])


def test_quantised_decode_tracks_unquantised_attention(oracle_mod):
    """With amax/448 scales the fp8 path stays close to attention on the bf16 values
    themselves (3 mantissa bits: about 2^-4 relative error per element)."""
    P = Paged(oracle_mod, [200], Hq=4, Hkv=1, D=64, seed=14)
    amax_k = float(np.abs(syn.bf16_bits_to_f32(P.k)).max())
    amax_v = float(np.abs(syn.bf16_bits_to_f32(P.v)).max())
    P.k_scale, P.v_scale = float(np.float32(amax_k) / np.float32(448)), float(np.float32(amax_v) / np.float32(448))
    P.write()
    out = P.decode()
    K = syn.bf16_bits_to_f32(P.k[:, 0]).astype(np.float64)
    V = syn.bf16_bits_to_f32(P.v[:, 0]).astype(np.float64)
    for hq in range(4):
        ref = oracle_mod.attention_rows(P.qf(0, hq), K, V)
        assert np.max(np.abs(out[0, hq] - ref)) < 0.05
