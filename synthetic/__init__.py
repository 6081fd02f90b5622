"""Seeded synthetic workloads for the fp8 paged KV-cache decode path.

Both the HIP path and the CPU oracle consume these arrays, so this module holds
none of the method's arithmetic: it only draws random values, rounds them to
bf16, lays out block tables and slot mappings, and picks the per-tensor scale
(1.0 uncalibrated, or amax/448 calibrated) that the caller passes to both sides.

Workload shapes follow the attention shapes the source pages measure
(Llama-3.1-8B, Llama-3.3-70B, gpt-oss-20b with 128-token windows, a head_dim-256
model with 512-token windows; "The State of FP8 KV-Cache and Attention
Quantization in vLLM", "DECODE COST").  The pages' model-level suites (needle
retrieval at 128K, mrcr) are stood in for by i.i.d. normal values, a 1% set of
x8 outlier key channels, and one planted needle key.

Seeds: workload c draws values (and random context lengths) from PCG64(1000+c),
the physical block permutation from PCG64(2000+c), and outlier channels and the
needle from PCG64(3000+c).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

BLOCK_SIZE = 16
E4M3 = "e4m3"
BF16 = "bf16"


# ------------------------------------------------------------- bf16 bits ----

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even), returned as uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        w = flat_u[s:s + step].astype(np.uint64)
        r = (w + 0x7FFF + ((w >> 16) & 1)) >> 16
        nan = (w & 0x7FFFFFFF) > 0x7F800000
        r = np.where(nan, ((w >> 16) | 0x0040), r)
        flat_o[s:s + step] = r.astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


# --------------------------------------------------------------- layout ----

@dataclasses.dataclass
class Layer:
    """One attention layer's new K/V rows (bf16 bits, [T][Hkv][D]) and cache settings."""
    k: np.ndarray
    v: np.ndarray
    cache_dtype: str
    k_scale: float
    v_scale: float
    sliding_window: int = 0
    name: str = "full"


@dataclasses.dataclass
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray      # int32 [B]
    block_tables: np.ndarray      # int32 [B][max_blocks]
    seq_offsets: np.ndarray       # int64 [B+1]; tokens of seq b are rows [o_b, o_{b+1})
    slot_mapping: np.ndarray      # int64 [T]; slot of every context token
    q: np.ndarray                 # uint16 [B][Hq][D]
    layers: List[Layer]
    needle: Optional[dict] = None
    config: Optional[dict] = None

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    def step_token_rows(self) -> np.ndarray:
        """Rows of each sequence's last token (position L_b - 1): the token a decode step writes."""
        L = self.context_lens.astype(np.int64)
        rows = self.seq_offsets[:-1] + L - 1
        return rows[L > 0]

    def prefix_token_rows(self) -> np.ndarray:
        """Rows of every context token except each sequence's last one."""
        keep = np.ones(self.num_tokens, dtype=bool)
        keep[self.step_token_rows()] = False
        return np.nonzero(keep)[0]


def _block_layout(context_lens: np.ndarray, bs: int, rng_perm: np.random.Generator,
                  slack: Optional[int] = None):
    """Random physical placement: a permutation of the block pool handed out in sequence order."""
    nb = [(int(L) + bs - 1) // bs for L in context_lens]
    used = sum(nb)
    if slack is None:
        slack = max(8, used // 64)
    NB = used + slack
    perm = rng_perm.permutation(NB).astype(np.int32)
    max_blocks = max(1, max(nb) if nb else 1)
    poison_block = perm[used]          # a slack block: never written, so it stays poisoned
    bt = np.full((len(nb), max_blocks), poison_block, dtype=np.int32)
    cur = 0
    for b, n in enumerate(nb):
        bt[b, :n] = perm[cur:cur + n]
        cur += n
    offsets = np.zeros(len(nb) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.asarray(context_lens, dtype=np.int64))
    T = int(offsets[-1])
    slots = np.empty(T, dtype=np.int64)
    for b, L in enumerate(context_lens):
        j = np.arange(int(L), dtype=np.int64)
        slots[offsets[b]:offsets[b + 1]] = bt[b, j // bs].astype(np.int64) * bs + j % bs
    return NB, bt, offsets, slots


def _amax_scale(bits: np.ndarray) -> float:
    """Calibrated per-tensor scale: amax over the whole tensor divided by 448, in f32."""
    amax = np.float32(0.0)
    flat = bits.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        amax = max(amax, np.float32(np.abs(bf16_bits_to_f32(flat[s:s + step])).max()))
    return float(np.float32(amax) / np.float32(448.0))


def per_head_amax_scales(bits: np.ndarray) -> np.ndarray:
    """Calibrated per-kv-head scales of bf16 rows [T][Hkv][D]: amax over each head's
    elements divided by 448, in f32 (1.0 for an all-zero head).  float32 [Hkv]."""
    T, Hkv, D = bits.shape
    amax = np.zeros(Hkv, dtype=np.float32)
    step = max(1, (1 << 22) // (Hkv * D))
    for s in range(0, T, step):
        blk = np.abs(bf16_bits_to_f32(bits[s:s + step]))
        amax = np.maximum(amax, blk.reshape(-1, Hkv, D).max(axis=(0, 2)).astype(np.float32))
    sc = amax / np.float32(448.0)
    sc[sc == 0] = np.float32(1.0)
    return sc.astype(np.float32)


def spread_head_scales(Hkv: int, cid: int, lo: float = 0.05, hi: float = 8.0) -> np.ndarray:
    """Seeded per-head scales spread log-uniformly over [lo, hi] (float32 [Hkv]): inputs
    that make a wrong head's scale visible."""
    rng = np.random.Generator(np.random.PCG64(4000 + cid))
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=Hkv)).astype(np.float32)


def with_head_magnitudes(w: "Workload", cid: int, max_exp: int = 3):
    """A copy of workload `w` whose every layer has kv heads of different magnitudes: the K
    and V rows of head h are multiplied by 2**e (seeded e in [-max_exp, max_exp], drawn
    separately for K and V; exact in bf16), with calibrated per-head scales.  Returns
    (workload, [(k_scales, v_scales) per layer]) -- the input a per-head calibration is for."""
    rng = np.random.Generator(np.random.PCG64(5000 + cid))
    layers, scales = [], []
    for L in w.layers:
        ek = rng.integers(-max_exp, max_exp + 1, size=w.num_kv_heads)
        ev = rng.integers(-max_exp, max_exp + 1, size=w.num_kv_heads)
        fk = np.exp2(ek).astype(np.float32)[None, :, None]
        fv = np.exp2(ev).astype(np.float32)[None, :, None]
        k = f32_to_bf16_bits(bf16_bits_to_f32(L.k) * fk)
        v = f32_to_bf16_bits(bf16_bits_to_f32(L.v) * fv)
        layers.append(Layer(k=k, v=v, cache_dtype=L.cache_dtype, k_scale=L.k_scale,
                            v_scale=L.v_scale, sliding_window=L.sliding_window, name=L.name))
        scales.append((per_head_amax_scales(k), per_head_amax_scales(v)))
    return Workload(**{**w.__dict__, "layers": layers}), scales


@dataclasses.dataclass
class PrefillQueries:
    """The query rows of one prefill / chunked-prefill call: sequence b's chunk is the
    last chunk_lens[b] positions of its context, rows [qsl[b], qsl[b+1]) of q."""
    q: np.ndarray                # bf16 bits [Tq][Hq][D]
    query_start_loc: np.ndarray  # int32 [B + 1]
    chunk_lens: np.ndarray       # int32 [B]

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_query_len(self) -> int:
        return int(self.chunk_lens.max()) if self.chunk_lens.size else 0


def prefill_queries(w: "Workload", chunk_lens, cid: int, std: float = 1.0) -> PrefillQueries:
    """Seeded N(0, std) bf16 query rows for a chunk of chunk_lens[b] tokens per sequence
    (seed 6000 + cid)."""
    rng = np.random.Generator(np.random.PCG64(6000 + cid))
    n = np.asarray(chunk_lens, dtype=np.int32)
    assert n.shape == (w.num_seqs,)
    qsl = np.zeros(w.num_seqs + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(n)
    q = f32_to_bf16_bits(_normal_bf16(rng, (int(qsl[-1]), w.num_q_heads, w.head_dim), std))
    return PrefillQueries(q=q, query_start_loc=qsl, chunk_lens=n)


def make_workload(name: str, cid: int, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  context_lens=None, num_seqs: int = 1, len_range=None, std: float = 1.0,
                  outlier_frac: float = 0.0, outlier_mult: float = 8.0, scale_mode: str = "amax",
                  needle: bool = False, layers=(("full", 0, E4M3),),
                  block_size: int = BLOCK_SIZE, slack: Optional[int] = None) -> Workload:
    """Generate one workload.

    context_lens: explicit lengths, or None with len_range=(lo, hi) inclusive drawn per sequence.
    layers: (name, sliding_window, cache_dtype) per layer; each gets its own K/V draw.
    scale_mode: "amax" (amax/448 per tensor) or "uncal" (1.0).
    """
    rng_v = np.random.Generator(np.random.PCG64(1000 + cid))
    rng_p = np.random.Generator(np.random.PCG64(2000 + cid))
    rng_x = np.random.Generator(np.random.PCG64(3000 + cid))
    if context_lens is None:
        lo, hi = len_range
        context_lens = rng_v.integers(lo, hi + 1, size=num_seqs)
    context_lens = np.asarray(context_lens, dtype=np.int32)
    B = context_lens.shape[0]
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    NB, bt, offsets, slots = _block_layout(context_lens, block_size, rng_p, slack)
    T = int(offsets[-1])

    q32 = _normal_bf16(rng_v, (B, Hq, D), std)
    q = f32_to_bf16_bits(q32)
    del q32

    n_out = int(round(outlier_frac * Hkv * D))
    out_channels = (np.sort(rng_x.choice(Hkv * D, size=n_out, replace=False))
                    if n_out > 0 else np.zeros(0, dtype=np.int64))

    needle_info = None
    if needle:
        p_star = int(rng_x.integers(0, int(context_lens[0])))
        chan = int(rng_x.integers(0, D))
        q0 = bf16_bits_to_f32(q[0, 0]).astype(np.float64)
        kstar = f32_to_bf16_bits((4.0 * q0 / np.linalg.norm(q0)).astype(np.float32))
        vstar = np.zeros(D, dtype=np.float32)
        vstar[chan] = 448.0
        needle_info = {"seq": 0, "q_head": 0, "kv_head": 0, "position": p_star,
                       "channel": chan, "row": int(offsets[0]) + p_star,
                       "key": kstar, "value": f32_to_bf16_bits(vstar)}

    out_layers: List[Layer] = []
    for (lname, window, cdt) in layers:
        k32 = _normal_bf16(rng_v, (T, Hkv, D), std)
        if n_out:
            flat = k32.reshape(T, Hkv * D)
            flat[:, out_channels] *= np.float32(outlier_mult)
        k = f32_to_bf16_bits(k32)
        del k32
        v = f32_to_bf16_bits(_normal_bf16(rng_v, (T, Hkv, D), std))
        if needle_info is not None:
            r = needle_info["row"]
            k[r, needle_info["kv_head"]] = needle_info["key"]
            v[r, needle_info["kv_head"]] = needle_info["value"]
        if cdt == E4M3 and scale_mode == "amax":
            ks, vs = _amax_scale(k), _amax_scale(v)
        else:
            ks, vs = 1.0, 1.0
        out_layers.append(Layer(k=k, v=v, cache_dtype=cdt, k_scale=ks, v_scale=vs,
                                sliding_window=int(window), name=lname))

    return Workload(name=name, num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    block_size=block_size, num_blocks=NB, context_lens=context_lens,
                    block_tables=bt, seq_offsets=offsets, slot_mapping=slots, q=q,
                    layers=out_layers, needle=needle_info,
                    config={"cid": cid, "scale_mode": scale_mode, "std": std,
                            "outlier_frac": outlier_frac, "needle": needle})


# -------------------------------------------------- the measured shapes ----

def tiny() -> Workload:
    """1 sequence of 256 tokens, 4 query heads on 1 KV head, head_dim 64, amax/448 scales."""
    return make_workload("tiny-g4-d64-L256", 1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                         context_lens=[256])


def llama8b_batch(scale_mode: str = "uncal", lens=None) -> Workload:
    """Llama-3.1-8B attention shape (32/8/128), batch 8, lengths uniform in [16384, 24576]."""
    kw = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, outlier_frac=0.01,
              scale_mode=scale_mode)
    if lens is None:
        return make_workload(f"llama8b-b8-L16k-24k-{scale_mode}", 2, num_seqs=8,
                             len_range=(16384, 24576), **kw)
    return make_workload(f"llama8b-b{len(lens)}-{scale_mode}", 2, context_lens=lens, **kw)


def llama8b_long(context_len: int = 131072, scale_mode: str = "uncal", num_seqs: int = 1) -> Workload:
    """Llama-3.1-8B attention shape at one long context: the headline decode shape."""
    return make_workload(f"llama8b-b{num_seqs}-L{context_len}-{scale_mode}", 6,
                         num_q_heads=32, num_kv_heads=8, head_dim=128,
                         context_lens=[context_len] * num_seqs, outlier_frac=0.01,
                         scale_mode=scale_mode)


def llama70b_needle(context_len: int, scale_mode: str = "amax", variant: int = 0) -> Workload:
    """Llama-3.3-70B attention shape (64/8/128, g 8), batch 1, outliers and a planted needle.

    variant > 0 draws an independent replicate (seed family 3 + 10 * variant)."""
    return make_workload(f"llama70b-needle-L{context_len}-{scale_mode}-v{variant}", 3 + 10 * variant,
                         num_q_heads=64, num_kv_heads=8, head_dim=128,
                         context_lens=[context_len], outlier_frac=0.01, scale_mode=scale_mode,
                         needle=True)


def gptoss_mixed(skip_sw: bool = False, context_len: int = 20480, num_seqs: int = 8) -> Workload:
    """gpt-oss-20b attention shape (64/8/64): one full layer and one 128-token-window layer.

    skip_sw keeps the window layer's cache in bf16 (the native dtype)."""
    sw_dtype = BF16 if skip_sw else E4M3
    return make_workload(f"gptoss-b{num_seqs}-L{context_len}-{'skipsw' if skip_sw else 'allfp8'}",
                         4, num_q_heads=64, num_kv_heads=8, head_dim=64,
                         context_lens=[context_len] * num_seqs,
                         layers=(("full", 0, E4M3), ("sw128", 128, sw_dtype)))


def gemma_d256(context_len: int = 65536, num_seqs: int = 16) -> Workload:
    """head_dim-256 shape (8/1/256, g 8), N(0, 0.5), one global and one 512-token-window layer."""
    return make_workload(f"d256-b{num_seqs}-L{context_len}", 5, num_q_heads=8, num_kv_heads=1,
                         head_dim=256, context_lens=[context_len] * num_seqs, std=0.5,
                         layers=(("global", 0, E4M3), ("sw512", 512, E4M3)))
