"""Helpers for the GPU parity tests: run the HIP path through the C-ABI binding and the CPU
oracle on the same seeded inputs, and compare.  Imported only by tests marked `gpu`."""
from __future__ import annotations

import sys

import numpy as np
import torch

import fp8_kv_cache_reshape_amd as F
import oracle
import synthetic as syn

DEV = "cuda"
E4M3, BF16 = F.FP8KV_E4M3, F.FP8KV_BF16
POISON = {E4M3: 0x7F, BF16: 0x7FC0}          # a NaN code / NaN bf16 in every untouched slot

# Decode tolerance for bf16 outputs, elementwise: |gpu - oracle| <= ATOL + RTOL * |oracle|.
ATOL, RTOL = 2e-3, 1e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def code(layer: syn.Layer) -> int:
    return E4M3 if layer.cache_dtype == syn.E4M3 else BF16


def u16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV)


def cache_numel(w: syn.Workload) -> int:
    return w.num_blocks * w.num_kv_heads * w.block_size * w.head_dim


def dev_caches(w: syn.Workload, cdt: int):
    n = cache_numel(w)
    if cdt == E4M3:
        return (torch.full((n,), POISON[E4M3], dtype=torch.uint8, device=DEV),
                torch.full((n,), POISON[E4M3], dtype=torch.uint8, device=DEV))
    return (torch.full((n,), POISON[BF16], dtype=torch.int16, device=DEV),
            torch.full((n,), POISON[BF16], dtype=torch.int16, device=DEV))


def host_caches(w: syn.Workload, cdt: int):
    n = cache_numel(w)
    dt = np.uint8 if cdt == E4M3 else np.uint16
    return np.full(n, POISON[cdt], dtype=dt), np.full(n, POISON[cdt], dtype=dt)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


# `heads`, where a helper takes it, is None (the layer's per-tensor scales) or a pair of
# float32 [Hkv] arrays (k_scales, v_scales): the per-head entry points and oracle functions.

def gpu_write(w: syn.Workload, layer: syn.Layer, kc, vc, rows=None, stream=None, heads=None) -> None:
    rows = np.arange(w.num_tokens) if rows is None else np.asarray(rows)
    k, v = u16_dev(layer.k[rows]), u16_dev(layer.v[rows])
    slots = torch.from_numpy(np.ascontiguousarray(w.slot_mapping[rows])).to(DEV)
    if heads is None:
        F.fp8kv_cache_write(k, v, kc, vc, code(layer), slots, len(rows), w.num_kv_heads, w.head_dim,
                            w.block_size, w.num_blocks, layer.k_scale, layer.v_scale, stream)
    else:
        F.fp8kv_cache_write_per_head(k, v, kc, vc, code(layer), slots, len(rows), w.num_kv_heads,
                                     w.head_dim, w.block_size, w.num_blocks, f32_dev(heads[0]),
                                     f32_dev(heads[1]), stream)


def oracle_write(w: syn.Workload, layer: syn.Layer, heads=None):
    kc, vc = host_caches(w, code(layer))
    if heads is None:
        oracle.cache_write(layer.k, layer.v, kc, vc, code(layer), w.slot_mapping, w.num_kv_heads,
                           w.head_dim, w.block_size, w.num_blocks, layer.k_scale, layer.v_scale)
    else:
        oracle.cache_write_per_head(layer.k, layer.v, kc, vc, code(layer), w.slot_mapping,
                                    w.num_kv_heads, w.head_dim, w.block_size, w.num_blocks,
                                    heads[0], heads[1])
    return kc, vc


class DeviceInputs:
    def __init__(self, w: syn.Workload, context_lens=None):
        self.q = u16_dev(w.q)
        self.bt = torch.from_numpy(np.ascontiguousarray(w.block_tables)).to(DEV)
        cl = w.context_lens if context_lens is None else context_lens
        self.cl = torch.from_numpy(np.ascontiguousarray(cl, dtype=np.int32)).to(DEV)


def new_counters(num_seqs: int, num_kv_heads: int) -> torch.Tensor:
    """A zero-filled counter buffer for decode calls of up to num_seqs sequences."""
    n = F.fp8kv_decode_counters_size(num_seqs, num_kv_heads)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV)


def gpu_decode(w: syn.Workload, layer: syn.Layer, kc, vc, out_f32=False, num_splits=0,
               window=None, dev: DeviceInputs = None, max_context_len=None, split_api=False,
               heads=None, counters=None):
    """fp8kv_paged_decode (per-head variant with `heads`, the two split passes with
    `split_api`); `counters` (a counter buffer) selects the in-kernel merge."""
    dev = dev or DeviceInputs(w)
    cn = counters.numel() if counters is not None else 0
    win = layer.sliding_window if window is None else window
    maxl = w.max_context_len if max_context_len is None else max_context_len
    B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    ws_bytes = F.fp8kv_paged_decode_workspace_size(B, Hq, Hkv, D, w.block_size, maxl, win, num_splits)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    out = torch.empty(B * Hq * D, dtype=torch.float32 if out_f32 else torch.bfloat16, device=DEV)
    odt = F.FP8KV_F32 if out_f32 else F.FP8KV_BF16
    cdt = code(layer)
    if heads is not None and split_api:
        F.fp8kv_paged_decode_partial_per_head(dev.q, kc, vc, cdt, dev.bt, w.max_blocks_per_seq, dev.cl,
                                              maxl, B, Hq, Hkv, D, w.block_size, w.num_blocks,
                                              f32_dev(heads[0]), win, num_splits, ws, ws_bytes)
        F.fp8kv_paged_decode_merge_per_head(out, odt, cdt, dev.cl, maxl, w.max_blocks_per_seq, B, Hq,
                                            Hkv, D, w.block_size, f32_dev(heads[1]), win, num_splits,
                                            ws, ws_bytes)
    elif heads is not None:
        F.fp8kv_paged_decode_per_head(out, odt, dev.q, kc, vc, cdt, dev.bt, w.max_blocks_per_seq,
                                      dev.cl, maxl, B, Hq, Hkv, D, w.block_size, w.num_blocks,
                                      f32_dev(heads[0]), f32_dev(heads[1]), win, num_splits,
                                      counters, cn, ws, ws_bytes)
    elif split_api:
        F.fp8kv_paged_decode_partial(dev.q, kc, vc, cdt, dev.bt, w.max_blocks_per_seq, dev.cl, maxl,
                                     B, Hq, Hkv, D, w.block_size, w.num_blocks, layer.k_scale, win,
                                     num_splits, ws, ws_bytes)
        F.fp8kv_paged_decode_merge(out, odt, dev.cl, maxl, w.max_blocks_per_seq, B, Hq, Hkv, D,
                                   w.block_size, layer.v_scale if cdt == E4M3 else 1.0, win,
                                   num_splits, ws, ws_bytes)
    else:
        F.fp8kv_paged_decode(out, odt, dev.q, kc, vc, cdt, dev.bt, w.max_blocks_per_seq, dev.cl, maxl,
                             B, Hq, Hkv, D, w.block_size, w.num_blocks, layer.k_scale, layer.v_scale,
                             win, num_splits, counters, cn, ws, ws_bytes)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64).reshape(B, Hq, D)


def oracle_decode(w: syn.Workload, layer: syn.Layer, okc, ovc, pairs=None, window=None,
                  context_lens=None, heads=None):
    win = layer.sliding_window if window is None else window
    cl = w.context_lens if context_lens is None else context_lens
    if heads is not None:
        args = (w.q, okc, ovc, code(layer), w.block_tables, cl, w.num_q_heads, w.num_kv_heads,
                w.head_dim, w.block_size, heads[0], heads[1], win)
        if pairs is None:
            return oracle.paged_decode_per_head(*args)
        return oracle.paged_decode_pairs_per_head(pairs, *args)
    args = (w.q, okc, ovc, code(layer), w.block_tables, cl, w.num_q_heads, w.num_kv_heads,
            w.head_dim, w.block_size, layer.k_scale, layer.v_scale, win)
    if pairs is None:
        return oracle.paged_decode(*args)
    return oracle.paged_decode_pairs(pairs, *args)


def oracle_decode_threaded(w: syn.Workload, layer: syn.Layer, okc, ovc, pairs, threads: int = 16):
    """oracle_decode for (b, hq) pairs, one pair per task on a thread pool (the oracle's C
    calls release the interpreter lock): [n][D]."""
    from concurrent.futures import ThreadPoolExecutor
    pairs = np.asarray(pairs, np.int32).reshape(-1, 2)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        rows = list(ex.map(lambda pr: oracle_decode(w, layer, okc, ovc, pairs=pr.reshape(1, 2)), pairs))
    return np.concatenate(rows) if rows else np.zeros((0, w.head_dim))


def assert_close(gpu: np.ndarray, ref: np.ndarray, atol=ATOL, rtol=RTOL, what=""):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if err.size:
        say(f"{what}: max abs err {err.max():.3g}, worst err/bound {(err / bound).max():.3f}")
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {idx}: "
                             f"gpu {gpu[idx]!r} oracle {ref[idx]!r} (max abs err {err.max():.3g})")
    return float(err.max())


def sample_pairs(w: syn.Workload, n_per_seq: int = 3, seed: int = 0) -> np.ndarray:
    """(b, hq) pairs: the first and last query head of every sequence plus random ones."""
    rng = np.random.default_rng(seed)
    pairs = []
    for b in range(w.num_seqs):
        heads = {0, w.num_q_heads - 1}
        heads |= set(rng.integers(0, w.num_q_heads, n_per_seq).tolist())
        pairs += [(b, h) for h in sorted(heads)]
    return np.array(pairs, dtype=np.int32)


def step_rows_by_seq(w: syn.Workload, layer: syn.Layer):
    """bf16 [B][Hkv][D] K and V of each sequence's token at position L_b - 1 (zeros for an
    empty sequence, whose row the step ignores)."""
    k = np.zeros((w.num_seqs, w.num_kv_heads, w.head_dim), np.uint16)
    v = np.zeros_like(k)
    for b in range(w.num_seqs):
        L = int(w.context_lens[b])
        if L > 0:
            r = int(w.seq_offsets[b]) + L - 1
            k[b], v[b] = layer.k[r], layer.v[r]
    return k, v


def gpu_decode_step(w: syn.Workload, layer: syn.Layer, kc, vc, out_f32=False, num_splits=0,
                    dev: DeviceInputs = None, counters=None, heads=None, workspace=None):
    """One fused step: writes each sequence's last token and decodes.  Returns (out,
    counters): the counter buffer given (zero on entry), or a new one for this batch."""
    dev = dev or DeviceInputs(w)
    B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    win = layer.sliding_window
    maxl = w.max_context_len
    if counters is None:
        counters = new_counters(B, Hkv)
    ws_bytes = F.fp8kv_paged_decode_workspace_size(B, Hq, Hkv, D, w.block_size, maxl, win, num_splits)
    if workspace is None:
        # filled with NaN bytes: the partials the step reads must all be its own
        workspace = torch.full((max(ws_bytes, 256),), 0xFF, dtype=torch.uint8, device=DEV)
    ws_bytes = workspace.numel()           # the library checks what it needs against this
    kn, vn = step_rows_by_seq(w, layer)
    out = torch.empty(B * Hq * D, dtype=torch.float32 if out_f32 else torch.bfloat16, device=DEV)
    odt = F.FP8KV_F32 if out_f32 else F.FP8KV_BF16
    if heads is None:
        F.fp8kv_decode_step(out, odt, dev.q, u16_dev(kn), u16_dev(vn), kc, vc, code(layer), dev.bt,
                            w.max_blocks_per_seq, dev.cl, maxl, B, Hq, Hkv, D, w.block_size,
                            w.num_blocks, layer.k_scale, layer.v_scale, win, num_splits, counters,
                            counters.numel(), workspace, ws_bytes)
    else:
        F.fp8kv_decode_step_per_head(out, odt, dev.q, u16_dev(kn), u16_dev(vn), kc, vc, code(layer),
                                     dev.bt, w.max_blocks_per_seq, dev.cl, maxl, B, Hq, Hkv, D,
                                     w.block_size, w.num_blocks, f32_dev(heads[0]),
                                     f32_dev(heads[1]), win, num_splits, counters,
                                     counters.numel(), workspace, ws_bytes)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64).reshape(B, Hq, D), counters


def gpu_prefill(w: syn.Workload, layer: syn.Layer, kc, vc, pq: syn.PrefillQueries, out_f32=False,
                window=None, heads=None, context_lens=None, max_query_len=None,
                max_context_len=None):
    """fp8kv_paged_prefill (or the per-head variant) over caches kc / vc: [Tq][Hq][D]."""
    win = layer.sliding_window if window is None else window
    dev = DeviceInputs(w, context_lens=context_lens)
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    Tq = pq.num_tokens
    out = torch.full((max(Tq, 1) * Hq * D,), float("nan"),
                     dtype=torch.float32 if out_f32 else torch.bfloat16, device=DEV)
    q = u16_dev(pq.q) if Tq else torch.zeros(8, dtype=torch.int16, device=DEV)
    qsl = torch.from_numpy(np.ascontiguousarray(pq.query_start_loc)).to(DEV)
    mql = pq.max_query_len if max_query_len is None else max_query_len
    odt = F.FP8KV_F32 if out_f32 else F.FP8KV_BF16
    maxl = w.max_context_len if context_lens is None else int(np.max(context_lens))
    if max_context_len is not None:
        maxl = max_context_len
    if heads is None:
        F.fp8kv_paged_prefill(out, odt, q, qsl, kc, vc, code(layer), dev.bt, w.max_blocks_per_seq,
                              dev.cl, maxl, w.num_seqs, mql, Hq, Hkv, D, w.block_size,
                              w.num_blocks, layer.k_scale, layer.v_scale, win)
    else:
        F.fp8kv_paged_prefill_per_head(out, odt, q, qsl, kc, vc, code(layer), dev.bt,
                                       w.max_blocks_per_seq, dev.cl, maxl, w.num_seqs, mql, Hq,
                                       Hkv, D, w.block_size, w.num_blocks, f32_dev(heads[0]),
                                       f32_dev(heads[1]), win)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)[: Tq * Hq * D].reshape(Tq, Hq, D)


def oracle_prefill(w: syn.Workload, layer: syn.Layer, okc, ovc, pq: syn.PrefillQueries,
                   pairs=None, window=None, heads=None, context_lens=None):
    """The oracle's prefill for (row, head) pairs ([n][D]) or every row ([Tq][Hq][D]); with
    per-head scales each kv head's pairs use that head's scales."""
    win = layer.sliding_window if window is None else window
    cl = w.context_lens if context_lens is None else context_lens
    full = pairs is None
    if full:
        pairs = np.array([(r, hq) for r in range(pq.num_tokens) for hq in range(w.num_q_heads)],
                         np.int32).reshape(-1, 2)
    pairs = np.asarray(pairs, np.int32).reshape(-1, 2)
    out = np.zeros((pairs.shape[0], w.head_dim))
    g = w.num_q_heads // w.num_kv_heads
    groups = [(None, np.arange(pairs.shape[0]))] if heads is None else \
        [(h, np.nonzero(pairs[:, 1] // g == h)[0]) for h in range(w.num_kv_heads)]
    for h, idx in groups:
        if idx.size == 0:
            continue
        ks, vs = (layer.k_scale, layer.v_scale) if h is None else (float(heads[0][h]), float(heads[1][h]))
        out[idx] = oracle.paged_prefill_pairs(pairs[idx], pq.q, pq.query_start_loc, okc, ovc,
                                              code(layer), w.block_tables, cl, w.num_q_heads,
                                              w.num_kv_heads, w.head_dim, w.block_size, ks, vs, win)
    return out.reshape(pq.num_tokens, w.num_q_heads, w.head_dim) if full else out
