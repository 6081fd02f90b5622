"""GPU parity of fp8kv_cache_write: cache bytes must equal the oracle's bit for bit."""
import numpy as np
import pytest
import torch

import fp8_kv_cache_reshape_amd as F
import oracle
import synthetic as syn
from gpu_util import (BF16, DEV, E4M3, dev_caches, gpu_write, host_caches, oracle_write, say,
                      to_host_bits, u16_dev)

pytestmark = pytest.mark.gpu


def _every_bf16_workload(Hkv=2, D=128, seed=0):
    """Every bf16 bit pattern once as a key element and once (reversed) as a value element,
    scattered to random slots of a pool with unused slots left poisoned."""
    T = 65536 // (Hkv * D)
    keys = np.arange(65536, dtype=np.uint16).reshape(T, Hkv, D)
    vals = keys[::-1].reshape(T, Hkv, D).copy()
    rng = np.random.default_rng(seed)
    NB = T // 16 + 7
    slots = rng.permutation(NB * 16)[:T].astype(np.int64)
    w = syn.Workload(name="every-bf16", num_seqs=0, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D,
                     block_size=16, num_blocks=NB, context_lens=np.zeros(0, np.int32),
                     block_tables=np.zeros((0, 1), np.int32), seq_offsets=np.zeros(1, np.int64),
                     slot_mapping=slots, q=np.zeros((0, Hkv, D), np.uint16), layers=[])
    return w, keys, vals


# (1.0, 1.0) and the last three pairs are powers of two on both tensors: the kernel then
# multiplies by the exact reciprocal instead of dividing (2^-126: the smallest normal scale;
# 2^127: a subnormal reciprocal); the others divide
@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.125, 3.0), (0.1, 36.5 / 448.0),
                                             (1e-3, 7.0), (4.40625 / 448.0, 0.0078125),
                                             (0.125, 2.0 ** -7), (2.0 ** -126, 2.0 ** 20),
                                             (2.0 ** 127, 2.0 ** -3)])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_every_bf16_input_bit_exact(k_scale, v_scale, D):
    say(f"cache_write every-bf16 D={D} scales={k_scale},{v_scale}")
    w, keys, vals = _every_bf16_workload(D=D)
    layer = syn.Layer(k=keys, v=vals, cache_dtype=syn.E4M3, k_scale=k_scale, v_scale=v_scale)
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc)
    torch.cuda.synchronize()
    okc, ovc = oracle_write(w, layer)
    gk, gv = to_host_bits(kc), to_host_bits(vc)
    bad_k, bad_v = np.nonzero(gk != okc)[0], np.nonzero(gv != ovc)[0]
    assert bad_k.size == 0, f"key bytes differ at {bad_k[:8]}: gpu {gk[bad_k[:8]]} oracle {okc[bad_k[:8]]}"
    assert bad_v.size == 0, f"value bytes differ at {bad_v[:8]}: gpu {gv[bad_v[:8]]} oracle {ovc[bad_v[:8]]}"


def test_bf16_cache_keeps_bits():
    say("cache_write bf16 cache")
    w, keys, vals = _every_bf16_workload(Hkv=1, D=256, seed=3)
    layer = syn.Layer(k=keys, v=vals, cache_dtype=syn.BF16, k_scale=1.0, v_scale=1.0)
    kc, vc = dev_caches(w, BF16)
    gpu_write(w, layer, kc, vc)
    torch.cuda.synchronize()
    okc, ovc = oracle_write(w, layer)
    assert np.array_equal(to_host_bits(kc), okc) and np.array_equal(to_host_bits(vc), ovc)


def test_out_of_range_slots_write_nothing():
    say("cache_write out-of-range slots")
    Hkv, D, NB = 2, 64, 3
    k = torch.ones(4 * Hkv * D, dtype=torch.bfloat16, device=DEV)
    kc = torch.full((NB * Hkv * 16 * D,), 0x5A, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0x5A)
    slots = torch.tensor([-1, -100, NB * 16, NB * 16 + 5], dtype=torch.int64, device=DEV)
    F.fp8kv_cache_write(k, k, kc, vc, E4M3, slots, 4, Hkv, D, 16, NB, 1.0, 1.0)
    torch.cuda.synchronize()
    assert bool((kc == 0x5A).all()) and bool((vc == 0x5A).all())


@pytest.mark.parametrize("make", [syn.tiny, lambda: syn.llama8b_batch("uncal", lens=[1, 17, 300, 4097]),
                                  lambda: syn.llama8b_batch("amax", lens=[64, 1000]),
                                  lambda: syn.gptoss_mixed(skip_sw=True, context_len=333, num_seqs=3),
                                  lambda: syn.gemma_d256(context_len=1500, num_seqs=2)])
def test_workload_caches_bit_exact(make):
    w = make()
    for layer in w.layers:
        say(f"cache_write {w.name} layer {layer.name} ({layer.cache_dtype})")
        kc, vc = dev_caches(w, E4M3 if layer.cache_dtype == syn.E4M3 else BF16)
        gpu_write(w, layer, kc, vc)
        torch.cuda.synchronize()
        okc, ovc = oracle_write(w, layer)
        assert np.array_equal(to_host_bits(kc), okc)
        assert np.array_equal(to_host_bits(vc), ovc)


def test_prefix_then_step_write_equals_one_write():
    """Writing the context first and each sequence's last token afterwards (a decode step)
    gives the same bytes as writing everything at once."""
    say("cache_write prefix + step")
    w = syn.llama8b_batch("amax", lens=[33, 200, 1])
    layer = w.layers[0]
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc, rows=w.prefix_token_rows())
    gpu_write(w, layer, kc, vc, rows=w.step_token_rows())
    torch.cuda.synchronize()
    okc, ovc = oracle_write(w, layer)
    assert np.array_equal(to_host_bits(kc), okc) and np.array_equal(to_host_bits(vc), ovc)


def _slot_pattern(name: str, T: int, NB: int, rng) -> np.ndarray:
    """Slot mappings that send token quads down the kernel's two store paths: runs of
    consecutive slots starting at a multiple of 4 (the transposed path) and everything else
    (the per-token path), with tails that do not fill a quad."""
    base = rng.permutation(NB)[: (T + 15) // 16 + 2].astype(np.int64) * 16
    if name == "in_order_blocks":         # whole blocks in order, T not a multiple of 4
        return np.concatenate([b + np.arange(16) for b in base])[:T]
    if name == "shifted_by_one":          # consecutive but never 4-aligned at a quad start
        return np.concatenate([b + np.arange(16) for b in base])[1:T + 1]
    if name == "shifted_by_four":         # aligned, but each quad starts 4 slots into a block
        s = np.concatenate([b + np.arange(16) for b in base])
        return s[4:T + 4]
    if name == "broken_runs":             # aligned starts with a gap or a skipped slot inside
        s = np.concatenate([b + np.arange(16) for b in base])[:T].copy()
        s[2::8] = -1                       # quads 0, 2, 4, ... lose their third token
        return s
    if name == "scattered":
        return rng.permutation(NB * 16)[:T].astype(np.int64)
    raise ValueError(name)


@pytest.mark.parametrize("pattern", ["in_order_blocks", "shifted_by_one", "shifted_by_four",
                                     "broken_runs", "scattered"])
@pytest.mark.parametrize("cache", [syn.E4M3, syn.BF16])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_slot_patterns_bit_exact(pattern, cache, D):
    Hkv, T = 3, 203
    rng = np.random.default_rng(D + len(pattern))
    NB = (T + 15) // 16 + 8
    slots = _slot_pattern(pattern, T, NB, rng)
    keys = syn.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32) * 3)
    vals = syn.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32) * 3)
    w = syn.Workload(name=f"slots-{pattern}", num_seqs=0, num_q_heads=Hkv, num_kv_heads=Hkv,
                     head_dim=D, block_size=16, num_blocks=NB, context_lens=np.zeros(0, np.int32),
                     block_tables=np.zeros((0, 1), np.int32), seq_offsets=np.zeros(1, np.int64),
                     slot_mapping=slots, q=np.zeros((0, Hkv, D), np.uint16), layers=[])
    layer = syn.Layer(k=keys, v=vals, cache_dtype=cache, k_scale=0.0213, v_scale=0.0172)
    cdt = E4M3 if cache == syn.E4M3 else BF16
    say(f"cache_write slot pattern {pattern} {cache} D={D}")
    kc, vc = dev_caches(w, cdt)
    gpu_write(w, layer, kc, vc)
    torch.cuda.synchronize()
    okc, ovc = oracle_write(w, layer)
    assert np.array_equal(to_host_bits(kc), okc), "key cache bytes differ"
    assert np.array_equal(to_host_bits(vc), ovc), "value cache bytes differ"


def _bf16_bits(x: float) -> int:
    b = int(np.array(x, np.float32).view(np.uint32))
    assert b & 0xFFFF == 0, x                   # exactly a bf16 value
    return b >> 16


def test_quotients_near_rounding_boundaries():
    """Scales s = x0 / m, and the floats either side of it, for every E4M3 rounding midpoint m
    (and the saturation threshold 464): x0 / s lands on or a few binary32 steps from a
    boundary of the cast, where the write's multiply-by-reciprocal shortcut must hand over to
    the division.  Per-head scales give 8 key and 8 value scales per call; every byte must
    equal the oracle's (correctly rounded division, then one cast)."""
    Hkv, D, T = 8, 64, 16
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = list((vals[:-1] + vals[1:]) / 2) + [464.0]
    combos = []
    for x0 in (1.5, 3.0, -0.3125, 7.0, 100.0):
        for m in mids:
            s0 = np.float32(abs(x0) / m)
            for s in (s0, np.nextafter(s0, np.float32(0)), np.nextafter(s0, np.float32(np.inf))):
                combos.append((x0, np.float32(s)))
    rng = np.random.default_rng(31)
    rng.shuffle(combos)
    slots = np.arange(T, dtype=np.int64)
    w = syn.Workload(name="boundaries", num_seqs=0, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D,
                     block_size=16, num_blocks=1, context_lens=np.zeros(0, np.int32),
                     block_tables=np.zeros((0, 1), np.int32), seq_offsets=np.zeros(1, np.int64),
                     slot_mapping=slots, q=np.zeros((0, Hkv, D), np.uint16), layers=[])
    say(f"cache_write boundaries: {len(combos)} scales")
    sign = np.where(np.arange(D) % 2 == 0, 0, 0x8000).astype(np.uint16)   # alternate signs
    for i in range(0, len(combos) - 2 * Hkv + 1, 2 * Hkv):
        kx, ks = zip(*combos[i:i + Hkv])
        vx, vs = zip(*combos[i + Hkv:i + 2 * Hkv])
        keys = np.empty((T, Hkv, D), np.uint16)
        vals_ = np.empty((T, Hkv, D), np.uint16)
        for h in range(Hkv):
            keys[:, h, :] = _bf16_bits(kx[h]) ^ sign
            vals_[:, h, :] = _bf16_bits(vx[h]) ^ sign
        layer = syn.Layer(k=keys, v=vals_, cache_dtype=syn.E4M3, k_scale=1.0, v_scale=1.0)
        heads = (np.array(ks, np.float32), np.array(vs, np.float32))
        kc, vc = dev_caches(w, E4M3)
        gpu_write(w, layer, kc, vc, heads=heads)
        okc, ovc = oracle_write(w, layer, heads=heads)
        assert np.array_equal(to_host_bits(kc), okc), f"key bytes differ, scales {ks}"
        assert np.array_equal(to_host_bits(vc), ovc), f"value bytes differ, scales {vs}"
