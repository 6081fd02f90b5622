#!/usr/bin/env python3
"""Benchmark of the fp8 paged-KV decode hot path on one MI355X.

One step = one decode step of one attention layer for the whole batch: quantise-on-write of
each sequence's new K/V token into the paged fp8 cache, then GQA decode attention over the
cache (split partials + log-sum-exp merge).  The step runs as the single fused launch
fp8kv_decode_step; the same step as two calls (fp8kv_cache_write, fp8kv_paged_decode) is
timed beside it.  The
default workload is the Llama-3.1-8B attention shape (32 query heads, 8 KV heads, head_dim
128, 16-token blocks) at batch 1 and 131,072 tokens of context, the shape the pages' decode
cost figures are quoted on ("The State of FP8 KV-Cache and Attention Quantization in vLLM",
"DECODE COST").  Inputs are seeded synthetic bf16 N(0,1) values with 1% x8 key outlier
channels and amax/448 scales, already resident in HBM; the cache is held in several rotated
instances (>= 1 GiB together) so that repeated steps read HBM rather than the 256 MB
Infinity Cache.

Prints ONE JSON line.  `value` is algorithmic bytes per step / step time (GB/s): the bytes
the method must move (fp8 K and V of every attended position, block-table entries, q, out,
context lengths, and the step's K/V write), not what the kernels happen to fetch.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, published
BLOCK = 16


# ------------------------------------------------------------- byte counts ----

def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V bytes one cached token costs across all layers (2 x layers x heads x dim x bytes)."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def arithmetic_intensity(group: int, elem_bytes: int, head_dim: int = 128) -> float:
    """Decode-attention flop per KV byte: (2gd for q.K + 2gd for p.V) over 2d*e bytes."""
    return (4.0 * group * head_dim) / (2.0 * head_dim * elem_bytes)


def attended(L: int, window: int):
    lo = max(0, L - window) if window > 0 else 0
    n = max(0, L - lo)
    nblk = ((L + BLOCK - 1) // BLOCK - lo // BLOCK) if n > 0 else 0
    return n, nblk


def algorithmic_bytes(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      elem_bytes: int, window: int = 0) -> dict:
    """Bytes the method must move per decode step, split by kernel.

    pass1 (partials): K and V of every attended position, one int32 block-table entry per
      attended block, the bf16 query and the int32 context length of every sequence.
    pass2 (merge): the bf16 output (plus the context length it re-reads).
    write: the step's bf16 K/V rows in, their cache elements out, one int64 slot each.
    """
    p1 = p2 = 0
    flops = 0
    for L in context_lens:
        n, nblk = attended(int(L), window)
        p1 += 2 * n * num_kv_heads * head_dim * elem_bytes + 4 * nblk + 2 * num_q_heads * head_dim + 4
        p2 += 2 * num_q_heads * head_dim + 4
        flops += 4 * num_q_heads * head_dim * n
    B = len(context_lens)
    write = B * num_kv_heads * head_dim * (2 * 2 + 2 * elem_bytes) + 8 * B
    return {"pass1": p1, "pass2": p2, "write": write, "step": p1 + p2 + write, "flops": flops}


# ----------------------------------------------------------------- harness ----

class DecodeBench:
    """Device buffers for one workload layer and the calls of one decode step."""

    def __init__(self, F, torch, w, layer, instances: int, num_splits: int, heads=None, codec=None):
        """heads: None (the layer's per-tensor scales) or float32 [Hkv] (k_scales, v_scales)
        for the per-head entry points.  codec: a one-byte cache code (FP8KV_E5M2 /
        FP8KV_INT8) in place of the layer's E4M3 (with scales rescaled to its range)."""
        self.F, self.torch, self.w, self.layer = F, torch, w, layer
        dev = "cuda"
        self.cdt = F.FP8KV_E4M3 if layer.cache_dtype == "e4m3" else F.FP8KV_BF16
        if codec is not None:
            assert self.cdt == F.FP8KV_E4M3
            top = {F.FP8KV_E5M2: 57344.0, F.FP8KV_INT8: 127.0}[codec]
            import dataclasses
            layer = dataclasses.replace(layer, k_scale=float(np.float32(layer.k_scale) * 448 / top),
                                        v_scale=float(np.float32(layer.v_scale) * 448 / top))
            self.layer = layer
            self.cdt = codec
        self.ebytes = 2 if self.cdt == F.FP8KV_BF16 else 1
        B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
        n = w.num_blocks * Hkv * BLOCK * D
        u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
        cache_dtype = torch.uint8 if self.ebytes == 1 else torch.int16
        self.q = u16(w.q)
        self.bt = torch.from_numpy(w.block_tables).to(dev)
        self.cl = torch.from_numpy(w.context_lens).to(dev)
        self.stream = int(torch.cuda.current_stream().cuda_stream)
        self.heads = None if heads is None else tuple(
            torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev) for a in heads)
        # the context before this step, written once into every rotated cache instance
        prefix = w.prefix_token_rows()
        kp, vp = u16(layer.k[prefix]), u16(layer.v[prefix])
        sp = torch.from_numpy(w.slot_mapping[prefix]).to(dev)
        self.kc, self.vc = [], []
        # kept for the bulk cache-write measurement
        self.kp, self.vp, self.sp, self.T_prefix = kp, vp, sp, len(prefix)
        for i in range(instances):
            self.kc.append(torch.zeros(n, dtype=cache_dtype, device=dev))
            self.vc.append(torch.zeros(n, dtype=cache_dtype, device=dev))
            self._write_rows(kp, vp, sp, len(prefix), i)
        # the step's new token of every sequence (all sequences are non-empty here)
        rows = w.step_token_rows()
        assert len(rows) == B, "every sequence needs a step token"
        self.k_new, self.v_new = u16(layer.k[rows]), u16(layer.v[rows])
        self.slots_new = torch.from_numpy(w.slot_mapping[rows]).to(dev)
        self.T_new = len(rows)
        self.maxl = w.max_context_len
        self.win = layer.sliding_window
        self.splits = num_splits
        self.nsplits = F.fp8kv_paged_decode_num_splits(B, Hkv, D, BLOCK, self.maxl, self.win, num_splits)
        self.ws_bytes = F.fp8kv_paged_decode_workspace_size(B, Hq, Hkv, D, BLOCK, self.maxl,
                                                            self.win, num_splits)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        # counter buffer (zeroed once; every call leaves it zero): the fused step, and the
        # in-kernel merge of the two-call path's decode
        self.cnt_bytes = F.fp8kv_decode_counters_size(B, Hkv)
        self.cnt = torch.zeros(max(self.cnt_bytes, 256), dtype=torch.uint8, device=dev)
        self.out = torch.empty(B * Hq * D, dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        self.bytes = algorithmic_bytes(w.context_lens, Hq, Hkv, D, self.ebytes, self.win)
        self.footprint = 2 * n * self.ebytes

    # -- the three kernels of a step, called through the C-ABI binding
    def _write_rows(self, k, v, slots, T, i):
        w, L = self.w, self.layer
        if self.heads is None:
            self.F.fp8kv_cache_write(k, v, self.kc[i], self.vc[i], self.cdt, slots, T,
                                     w.num_kv_heads, w.head_dim, BLOCK, w.num_blocks, L.k_scale,
                                     L.v_scale, self.stream)
        else:
            self.F.fp8kv_cache_write_per_head(k, v, self.kc[i], self.vc[i], self.cdt, slots, T,
                                              w.num_kv_heads, w.head_dim, BLOCK, w.num_blocks,
                                              self.heads[0], self.heads[1], self.stream)

    def write(self, i):
        self._write_rows(self.k_new, self.v_new, self.slots_new, self.T_new, i)

    def decode(self, i):
        w, L = self.w, self.layer
        if self.heads is None:
            self.F.fp8kv_paged_decode(self.out, self.F.FP8KV_BF16, self.q, self.kc[i], self.vc[i],
                                      self.cdt, self.bt, w.max_blocks_per_seq, self.cl, self.maxl,
                                      w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, BLOCK,
                                      w.num_blocks, L.k_scale, L.v_scale, self.win, self.splits,
                                      self.cnt, self.cnt_bytes, self.ws, self.ws_bytes, self.stream)
        else:
            self.F.fp8kv_paged_decode_per_head(self.out, self.F.FP8KV_BF16, self.q, self.kc[i],
                                               self.vc[i], self.cdt, self.bt, w.max_blocks_per_seq,
                                               self.cl, self.maxl, w.num_seqs, w.num_q_heads,
                                               w.num_kv_heads, w.head_dim, BLOCK, w.num_blocks,
                                               self.heads[0], self.heads[1], self.win,
                                               self.splits, self.cnt, self.cnt_bytes, self.ws,
                                               self.ws_bytes, self.stream)

    def partial(self, i):
        w, L = self.w, self.layer
        self.F.fp8kv_paged_decode_partial(self.q, self.kc[i], self.vc[i], self.cdt, self.bt,
                                          w.max_blocks_per_seq, self.cl, self.maxl, w.num_seqs,
                                          w.num_q_heads, w.num_kv_heads, w.head_dim, BLOCK,
                                          w.num_blocks, L.k_scale, self.win, self.splits,
                                          self.ws, self.ws_bytes, self.stream)

    def merge(self):
        w, L = self.w, self.layer
        vs = L.v_scale if self.cdt == self.F.FP8KV_E4M3 else 1.0
        self.F.fp8kv_paged_decode_merge(self.out, self.F.FP8KV_BF16, self.cl, self.maxl,
                                        w.max_blocks_per_seq, w.num_seqs, w.num_q_heads,
                                        w.num_kv_heads, w.head_dim, BLOCK, vs, self.win,
                                        self.splits, self.ws, self.ws_bytes, self.stream)

    def _fused_args(self, i):
        """fp8kv_decode_step's arguments on cache instance i as plain numbers, converted once,
        so that a timed loop pays only the foreign call (about 2 us less host time per launch,
        which matters for the first launch of a timed region: the GPU idles until it arrives)."""
        if not hasattr(self, "_fused_cache"):
            F, w, L, a = self.F, self.w, self.layer, self.F._addr
            self._fused_cache = [
                (a(self.out), F.FP8KV_BF16, a(self.q), a(self.k_new), a(self.v_new), a(self.kc[j]),
                 a(self.vc[j]), self.cdt, a(self.bt), w.max_blocks_per_seq, a(self.cl), self.maxl,
                 w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, BLOCK, w.num_blocks,
                 float(L.k_scale), float(L.v_scale), self.win, self.splits, a(self.cnt),
                 self.cnt_bytes, a(self.ws), self.ws_bytes, self.stream)
                for j in range(len(self.kc))]
        return self._fused_cache[i]

    def fused_step(self, i):
        """The whole step in one launch: write each sequence's token at L-1, then decode."""
        w, L = self.w, self.layer
        if self.heads is None:
            st = self.F.lib.fp8kv_decode_step(*self._fused_args(i))
            if st < 0:
                raise self.F.Fp8kvError(st, "fp8kv_decode_step")
        else:
            self.F.fp8kv_decode_step_per_head(self.out, self.F.FP8KV_BF16, self.q, self.k_new,
                                              self.v_new, self.kc[i], self.vc[i], self.cdt, self.bt,
                                              w.max_blocks_per_seq, self.cl, self.maxl, w.num_seqs,
                                              w.num_q_heads, w.num_kv_heads, w.head_dim, BLOCK,
                                              w.num_blocks, self.heads[0], self.heads[1], self.win,
                                              self.splits, self.cnt, self.cnt_bytes, self.ws,
                                              self.ws_bytes, self.stream)

    def two_call_step(self, i):
        self.write(i)
        self.decode(i)

    step = fused_step

    # -- timing
    def time_steps(self, steps: int, warmup: int, step_fn=None):
        """Region A: `steps` whole steps bracketed by two events (no events inside)."""
        torch = self.torch
        R = len(self.kc)
        step_fn = step_fn or self.step
        for s in range(warmup):
            step_fn(s % R)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_cpu = time.perf_counter()
        e0.record()
        for s in range(steps):
            step_fn(s % R)
        e1.record()
        t_enq = time.perf_counter() - t_cpu
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, t_enq * 1e3 / steps

    def time_kernels(self, launches: int, two_call: bool = True):
        """Region B: each kernel of the step launched `launches` times back to back (rotating
        over the cache instances) between one pair of events: the average launch duration,
        including the short gap between dependent launches on one stream."""
        torch = self.torch
        R = len(self.kc)

        def avg(fn):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            fn(0)
            torch.cuda.synchronize()
            e0.record()
            for s in range(launches):
                fn(s % R)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / launches

        out = {"step_ms": avg(self.fused_step), "write_ms": float("nan"), "decode_ms": float("nan"),
               "pass1_ms": float("nan"), "merge_ms": float("nan")}
        if two_call:
            out["write_ms"] = avg(self.write)
            out["decode_ms"] = avg(self.decode)
            if self.heads is None:     # the split passes take per-tensor scales only
                out["pass1_ms"] = avg(self.partial)
                out["merge_ms"] = avg(lambda i: self.merge()) if self.nsplits > 1 else 0.0
        return out

    def step_percentiles(self, steps: int):
        """Region C: every step between its own pair of events (the events add a little
        work between steps): p10, median and p90 of the step time in ms."""
        torch = self.torch
        R = len(self.kc)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        self.step(0)
        torch.cuda.synchronize()
        for s, (a, b) in enumerate(ev):
            a.record()
            self.step(s % R)
            b.record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in ev])
        return {q: float(np.percentile(t, q)) for q in (10, 50, 90)}

    def bulk_write_ms(self, launches: int):
        """The whole context written by one fp8kv_cache_write call, back to back over the
        rotated instances: average ms per call."""
        torch, F, w, L = self.torch, self.F, self.w, self.layer
        R = len(self.kc)

        def write(i):
            self._write_rows(self.kp, self.vp, self.sp, self.T_prefix, i)
        write(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(launches):
            write(s % R)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / launches


PROFILE_SUMMARY = "profiles/decode_llama8b_b1_128k.txt"
KERNEL_SOURCES = ["fp8_kv_cache_reshape_amd/csrc/paged_decode.hip",
                  "fp8_kv_cache_reshape_amd/csrc/internal.h",
                  "fp8_kv_cache_reshape_amd/csrc/codec.h",
                  "fp8_kv_cache_reshape_amd/csrc/hadamard.h"]


def measured_traffic(root: str):
    """HBM bytes per pass-1 launch from the committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE scaled by a plain copy), or None when the kernel sources have changed since the
    counters were taken (the summary records a hash of them)."""
    import hashlib
    path = os.path.join(root, PROFILE_SUMMARY)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(root, f), "rb").read())
    text = open(path).read()
    if f"(paged_decode.hip + internal.h + codec.h + hadamard.h): {h.hexdigest()[:16]}" not in text:
        return None
    for line in text.splitlines():
        if line.startswith("decode_partial_traffic_bytes_per_launch"):
            return int(line.split()[1])
    return None


def read_ceiling(torch, root: str, gib: int = 2, launches: int = 20) -> dict:
    """Streaming-read ceiling of this GPU: a plain kernel reading `gib` GiB once with 16-byte
    nontemporal loads (libfp8kv_probe.so), averaged over back-to-back launches, swept over grid
    sizes, loads in flight per thread and two access patterns (grid-stride, and contiguous
    runs per workgroup); the best rate is the ceiling.  `converged` says whether the same
    pattern and loads in flight at half the best grid reach within 1 % of it (a plateau)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(root, "fp8_kv_cache_reshape_amd", "libfp8kv_probe.so"))
    lib.fp8kv_probe_read_granule.restype = ctypes.c_size_t
    lib.fp8kv_probe_read_granule.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.fp8kv_probe_read.restype = ctypes.c_int
    lib.fp8kv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    grids = (1024, 2048, 4096, 8192, 16384, 32768)
    unrolls = (8, 16)
    g = max(lib.fp8kv_probe_read_granule(grid, u) for grid in grids for u in unrolls)
    n = max(1, (gib << 30) // g) * g
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = int(torch.cuda.current_stream().cuda_stream)
    rates = {}
    for pat in (0, 1):
        for u in unrolls:
            for grid in grids:
                call = lambda: lib.fp8kv_probe_read(buf.data_ptr(), n, grid, u, pat, sink.data_ptr(), stream)
                for _ in range(2):
                    assert call() == 0, "read-ceiling probe launch failed"
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(launches):
                    call()
                e1.record()
                torch.cuda.synchronize()
                rates[(pat, grid, u)] = n / (e0.elapsed_time(e1) / launches * 1e-3) / 1e9
    del buf
    best = max(rates, key=rates.get)
    half = (best[0], best[1] // 2, best[2])
    converged = half in rates and rates[half] >= 0.99 * rates[best]
    # paged reads: 1 and 2 KiB pieces at scattered places over a power-of-two buffer, the
    # granule of a paged cache's reads (one 16-token block of one kv head: 1 KiB of keys or
    # values at head_dim 64 in one-byte codes, 2 KiB at 128)
    pn = 1 << 31
    pbuf = torch.ones(pn, dtype=torch.uint8, device="cuda")
    paged = {}
    for pat in (2, 3):
        for u in unrolls:
            for grid in (2048, 4096, 8192, 16384):
                call = lambda: lib.fp8kv_probe_read(pbuf.data_ptr(), pn, grid, u, pat, sink.data_ptr(), stream)
                for _ in range(2):
                    assert call() == 0, "paged read probe launch failed"
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(launches):
                    call()
                e1.record()
                torch.cuda.synchronize()
                paged[(pat, grid, u)] = pn / (e0.elapsed_time(e1) / launches * 1e-3) / 1e9
    del pbuf
    names = ("stride", "chunk", "paged1k", "paged2k")
    return {"GBps": round(rates[best], 1), "bytes": n, "pattern": names[best[0]], "grid": best[1],
            "loads_in_flight": best[2],
            "GBps_by_config": {f"{names[p]}-{grd}x{u}": round(r, 1) for (p, grd, u), r in rates.items()},
            "converged": bool(converged),
            "paged_GBps": {"1KiB": round(max(r for (p, _, _), r in paged.items() if p == 2), 1),
                           "2KiB": round(max(r for (p, _, _), r in paged.items() if p == 3), 1)},
            "paged_GBps_by_config": {f"{names[p]}-{grd}x{u}": round(r, 1) for (p, grd, u), r in paged.items()},
            "kernel": "16-byte nontemporal reads, 256 threads per workgroup; keys are pattern (grid-"
                      "stride or contiguous runs per workgroup; paged: 1 or 2 KiB pieces at "
                      "scattered places), grid x loads in flight per thread"}


def _oracle_threads() -> int:
    """Host threads for the multi-threaded oracle run: the CPUs this process may use, at most
    16 (one GPU's share of the box)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(w, layer, pairs_kv_heads: int = 2):
    """The oracle (plain C, fp64, single thread) on a bounded sample of the same workload:
    every query head of the first `pairs_kv_heads` KV heads over the full context.  A second
    run decodes the whole step on a thread pool.  Returns (the baseline record, the oracle's
    output of the whole step as float64 [B][Hq][D])."""
    import oracle
    pairs_kv_heads = min(pairs_kv_heads, w.num_kv_heads)
    okc = np.zeros(w.num_blocks * w.num_kv_heads * BLOCK * w.head_dim, np.uint8)
    ovc = np.zeros_like(okc)
    oracle.cache_write(layer.k, layer.v, okc, ovc, oracle.CACHE_E4M3, w.slot_mapping, w.num_kv_heads,
                       w.head_dim, BLOCK, w.num_blocks, layer.k_scale, layer.v_scale)
    g = w.num_q_heads // w.num_kv_heads
    pairs = np.array([(b, hq) for b in range(w.num_seqs) for hq in range(pairs_kv_heads * g)], np.int32)
    t0 = time.perf_counter()
    oracle.paged_decode_pairs(pairs, w.q, okc, ovc, oracle.CACHE_E4M3, w.block_tables, w.context_lens,
                              w.num_q_heads, w.num_kv_heads, w.head_dim, BLOCK, layer.k_scale,
                              layer.v_scale, layer.sliding_window)
    dt = time.perf_counter() - t0
    frac = pairs_kv_heads / w.num_kv_heads
    sample_bytes = algorithmic_bytes(w.context_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, 1,
                                     layer.sliding_window)["pass1"] * frac
    # the same oracle over every query head, one (sequence, head) pair per task on a thread
    # pool: the C calls release the interpreter lock, so the threads run in parallel
    from concurrent.futures import ThreadPoolExecutor
    threads = _oracle_threads()
    all_pairs = [np.array([(b, hq)], np.int32) for b in range(w.num_seqs) for hq in range(w.num_q_heads)]
    args = (w.q, okc, ovc, oracle.CACHE_E4M3, w.block_tables, w.context_lens, w.num_q_heads,
            w.num_kv_heads, w.head_dim, BLOCK, layer.k_scale, layer.v_scale, layer.sliding_window)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        rows = list(ex.map(lambda pr: oracle.paged_decode_pairs(pr, *args), all_pairs))
    dt_mt = time.perf_counter() - t0
    ref = np.concatenate(rows).reshape(w.num_seqs, w.num_q_heads, w.head_dim)
    full_bytes = algorithmic_bytes(w.context_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, 1,
                                   layer.sliding_window)["pass1"]
    return {"value": round(sample_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"fp64 C oracle decode of query heads 0..{pairs_kv_heads * g - 1} (KV heads "
                      f"0..{pairs_kv_heads - 1} of {w.num_kv_heads}) of each of the {w.num_seqs} sequences over "
                      f"its whole window (contexts {int(w.context_lens.min())}..{int(w.context_lens.max())}, "
                      f"window {layer.sliding_window}), single thread; GB/s = the sample's algorithmic "
                      f"KV+q+table bytes / time",
            "multi_thread": {"value": round(full_bytes / dt_mt / 1e9, 4), "unit": "GB/s", "cores": threads,
                             "seconds": round(dt_mt, 3), "ms_per_step": round(dt_mt * 1e3, 1),
                             "sample": f"every query head ({len(all_pairs)} (sequence, head) tasks) of the "
                                       f"whole step on {threads} threads"},
            "host": _host_cpu()}, ref


def _host_cpu() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


WORKLOADS = {
    "llama8b-b1-128k": lambda syn: syn.llama8b_long(131072, "amax"),
    "llama8b-b8-128k": lambda syn: syn.llama8b_long(131072, "amax", num_seqs=8),
    "llama8b-b8-16k-24k": lambda syn: syn.llama8b_batch("amax"),
    "llama70b-b1-128k": lambda syn: syn.llama70b_needle(131072),
    "gptoss-b8-20k": lambda syn: syn.gptoss_mixed(skip_sw=False),
    "gptoss-b8-20k-skipsw": lambda syn: syn.gptoss_mixed(skip_sw=True),
    "d256-b16-64k": lambda syn: syn.gemma_d256(),
}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the first ~10 ms of back-to-back steps after setup run about 2 % slow (clocks settling):
    # the default warmup covers them
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="llama8b-b1-128k", choices=sorted(WORKLOADS))
    ap.add_argument("--layer", type=int, default=0, help="layer of a mixed workload to time")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--rotate-bytes", type=float, default=1.0, help="GiB of rotated cache instances")
    ap.add_argument("--no-bf16", action="store_true", help="skip the bf16-KV instantiation")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true", help="skip the streaming-read probe")
    ap.add_argument("--profile", action="store_true",
                    help="short run for a profiler: fused step only, no bf16 variant, no CPU baseline")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (for counter scaling)")
    ap.add_argument("--per-head-scales", action="store_true",
                    help="kv heads of different magnitudes with calibrated per-head scales, through "
                         "the per-head entry points (fp8 cache)")
    ap.add_argument("--prefill", action="store_true",
                    help="only time fp8kv_paged_prefill (whole-prompt prefill, fp8 and bf16 caches) "
                         "on the --prefill-workload shapes")
    ap.add_argument("--prefill-workload", default="llama8b-8k,d256-8k",
                    help="comma-separated: " + ", ".join(sorted(PREFILL_WORKLOADS)))
    ap.add_argument("--prefill-caches", default="e4m3,bf16", help="cache dtypes to time")
    ap.add_argument("--prefill-rotated", action="store_true",
                    help="with --prefill: also time the prefill over rotated caches (head_dim <= 128)")
    ap.add_argument("--codec", choices=["e4m3", "e5m2", "int8"], default="e4m3",
                    help="one-byte cache codec of the timed fp8 layer (default e4m3)")
    ap.add_argument("--rotated", action="store_true",
                    help="only time the Hadamard-rotated path (rotated write of the step token + "
                         "rotated decode) against the plain two-call path on --workload")
    ap.add_argument("--slope", action="store_true",
                    help="only sweep the context length at the 8B shape (B = 1, fp8 and bf16 KV) and fit "
                         "us/step = slope * L + intercept")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "this path runs on one GPU; --gpus must be 1 (multi-GPU sharding "
                                   "of the decode is described in the design notes, not built)"}))
        return 2

    import torch
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return 0

    root = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, root)
    import fp8_kv_cache_reshape_amd as F
    import synthetic as syn

    if args.slope:
        print(json.dumps(slope_sweep(F, torch, syn, args)), flush=True)
        return 0
    if args.rotated:
        print(json.dumps(_finite(rotated_bench(F, torch, syn, args))), flush=True)
        return 0
    if args.prefill:
        for name in args.prefill_workload.split(","):
            print(json.dumps(_finite(prefill_bench(F, torch, syn, name, args))), flush=True)
        return 0

    t0 = time.perf_counter()
    w = WORKLOADS[args.workload](syn)
    heads = None
    if args.per_head_scales:
        w, scales = syn.with_head_magnitudes(w, 140)
        heads = scales[args.layer]
    layer = w.layers[args.layer]
    gen_s = time.perf_counter() - t0
    one = 2 * w.num_blocks * w.num_kv_heads * BLOCK * w.head_dim * (1 if layer.cache_dtype == "e4m3" else 2)
    R = max(1, math.ceil(args.rotate_bytes * (1 << 30) / one))
    codec = {"e4m3": None, "e5m2": F.FP8KV_E5M2, "int8": F.FP8KV_INT8}[args.codec]
    if codec is not None and layer.cache_dtype != "e4m3":
        codec = None
    bench = DecodeBench(F, torch, w, layer, R, args.num_splits, heads, codec)
    # The per-kernel timings run first: about 10 ms of back-to-back launches after setup run a
    # few percent slow while the GPU's clocks settle, and these take that time, so the timed
    # region below (W warmup steps, then exactly K steps) measures the steady state.
    kern = bench.time_kernels(100, two_call=not args.profile)
    # under a profiler (--profile) only the fused step runs, so every dispatch of the decode
    # kernel in the trace is a fused step
    pct = bench.step_percentiles(args.steps) if not args.profile else None
    bulk_ms = bench.bulk_write_ms(10) if not args.profile else float("nan")
    ms_two = bench.time_steps(args.steps, args.warmup, bench.two_call_step)[0] if not args.profile else float("nan")
    # the timed region: `value`, `ms_per_step`, and the roofline of the fused-step kernel, which
    # is the step's only launch whenever the partials merge inside it (every benchmarked shape
    # at its automatic split count); otherwise the merge launch that follows is counted too
    ms_step, ms_enqueue = bench.time_steps(args.steps, args.warmup)
    out_last = bench.out.float().cpu().numpy().astype(np.float64).reshape(
        w.num_seqs, w.num_q_heads, w.head_dim)
    bulk_tokens = bench.T_prefix
    by = bench.bytes
    value = by["step"] / (ms_step * 1e-3) / 1e9
    # the dominant (and only) kernel of a step is the fused decode-step kernel: it moves the
    # whole step's algorithmic bytes; its average launch over the timed region
    launch_ms = ms_step
    achieved = by["step"] / (launch_ms * 1e-3) / 1e9

    result = {
        "metric": "FP8 paged decode attn: KV HBM GB/s (% of peak) + µs/step, 8B shape @128K",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "us_per_step": round(ms_step * 1e3, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": (f"{args.codec if codec is not None else 'e4m3'} KV -> bf16 MFMA, f32 accumulate"
                  if bench.ebytes == 1 else "bf16 KV, f32 accumulate"),
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {w.name}, layer {layer.name} "
                               f"({layer.cache_dtype if codec is None else args.codec} cache, "
                               f"window {layer.sliding_window}"
                               f"{', per-head scales' if heads is not None else ''})",
                   "num_seqs": w.num_seqs, "context_lens": sorted(set(int(x) for x in w.context_lens))[:4],
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": BLOCK, "splits": bench.nsplits,
                   "rotated_instances": R, "instance_bytes": one, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (measured_traffic(root) if args.workload == "llama8b-b1-128k"
                                 and layer.cache_dtype == "e4m3" and args.num_splits == 0
                                 and heads is None and codec is None else None),
                     "kernel": "decode_partial_kernel (fp8kv_decode_step: write + decode + merge)",
                     "bytes_per_launch": by["step"],
                     "avg_launch_us": round(launch_ms * 1e3, 3),
                     "launch_timing": "the timed region: K step launches between two HIP events on "
                                      "the library's stream"},
        "kernels_us": {"decode_step": round(kern["step_ms"] * 1e3, 3),
                       "two_call_path": {"cache_write": round(kern["write_ms"] * 1e3, 3),
                                         "paged_decode_in_kernel_merge": round(kern["decode_ms"] * 1e3, 3),
                                         "decode_partial": round(kern["pass1_ms"] * 1e3, 3),
                                         "decode_merge": round(kern["merge_ms"] * 1e3, 3)}},
        "two_call_us_per_step": round(ms_two * 1e3, 2),
        "step_us_p10_p50_p90": ([round(pct[q] * 1e3, 2) for q in (10, 50, 90)] if pct else None),
        "cache_write_bulk": {"tokens": bulk_tokens, "us": round(bulk_ms * 1e3, 2),
                             "GBps": round(bulk_tokens * (w.num_kv_heads * w.head_dim * (2 * 2 + 2 * bench.ebytes) + 8)
                                           / (bulk_ms * 1e-3) / 1e9, 1),
                             "bytes_per_token": w.num_kv_heads * w.head_dim * (2 * 2 + 2 * bench.ebytes) + 8},
        "bytes_per_step": by["step"], "flops_per_step": by["flops"],
        "enqueue_us_per_step": round(ms_enqueue * 1e3, 2), "input_gen_s": round(gen_s, 1),
    }
    del bench
    torch.cuda.empty_cache()

    if not (args.profile or args.no_read_ceiling):
        rc = read_ceiling(torch, root)
        result["read_ceiling"] = rc
        result["pct_of_read_ceiling"] = round(100 * value / rc["GBps"], 2)
        # the paged ceiling at this layer's read granule (one block of one kv head)
        granule = BLOCK * w.head_dim * (1 if layer.cache_dtype == "e4m3" else 2)
        key = {1024: "1KiB", 2048: "2KiB"}.get(granule)
        if key is not None:
            result["pct_of_paged_read_ceiling"] = {"granule": key,
                                                   "pct": round(100 * value / rc["paged_GBps"][key], 2)}
        torch.cuda.empty_cache()

    if not (args.no_bf16 or args.profile or heads is not None or codec is not None) \
            and layer.cache_dtype == "e4m3":
        import dataclasses
        bl = dataclasses.replace(layer, cache_dtype="bf16", k_scale=1.0, v_scale=1.0)
        R2 = max(1, math.ceil(args.rotate_bytes * (1 << 30) / (2 * one)))
        b2 = DecodeBench(F, torch, w, bl, R2, args.num_splits)
        k2 = b2.time_kernels(100)
        ms2, _ = b2.time_steps(args.steps, args.warmup)
        result["bf16_kv"] = {"us_per_step": round(ms2 * 1e3, 2),
                             "GBps": round(b2.bytes["step"] / (ms2 * 1e-3) / 1e9, 2),
                             "decode_partial_us": round(k2["pass1_ms"] * 1e3, 3),
                             "fp8_over_bf16_time": round(ms_step / ms2, 4)}
        del b2
        torch.cuda.empty_cache()

    ok = True
    if not (args.no_cpu_baseline or args.profile or heads is not None or codec is not None) \
            and layer.cache_dtype == "e4m3":
        result["cpu_baseline"], ref = cpu_baseline(w, layer)
        # the last timed step's output against the oracle's whole step: after hundreds of
        # back-to-back steps on rotated caches, every output element within the decode bound
        err = np.abs(out_last - ref)
        bound = 2e-3 + 1e-2 * np.abs(ref)
        ok = bool(np.all(np.isfinite(out_last)) and np.all(err <= bound))
        result["output_check"] = {"elements": int(ref.size), "max_abs_err": float(err.max()),
                                  "worst_err_over_bound": round(float((err / bound).max()), 4),
                                  "within_tolerance": ok,
                                  "against": "the oracle's whole step (cpu_baseline.multi_thread)"}

    print(json.dumps(_finite(result)), flush=True)
    return 0 if ok else 3


SLOPE_CONTEXTS = (4096, 8192, 16384, 32768, 65536, 131072, 262144)


def slope_sweep(F, torch, syn, args) -> dict:
    """us/step of the fused step at the 8B shape, B = 1, over the context lengths above, for
    the fp8 cache and the bf16 cache; least-squares fit us = slope * L + intercept.  The
    slope x 32 layers / 1000 is the attention share of a 32-layer model's time per token
    per context token (ms/token), comparable to the inter-token-latency slopes the pages
    quote (Llama-3.1-8B: 2.37e-05 on H100 with fp8 KV, 9.72e-06 on B200)."""
    import dataclasses
    points = {"e4m3": [], "bf16": []}
    for L in SLOPE_CONTEXTS:
        w = syn.llama8b_long(L, "amax")
        for dt in ("e4m3", "bf16"):
            layer = w.layers[0] if dt == "e4m3" else dataclasses.replace(w.layers[0], cache_dtype="bf16",
                                                                         k_scale=1.0, v_scale=1.0)
            one = 2 * w.num_blocks * w.num_kv_heads * BLOCK * w.head_dim * (1 if dt == "e4m3" else 2)
            R = max(1, math.ceil((1 << 30) / one))
            b = DecodeBench(F, torch, w, layer, R, 0)
            ms, _ = b.time_steps(args.steps, args.warmup)
            points[dt].append((L, ms * 1e3, b.bytes["step"] / (ms * 1e-3) / 1e9))
            del b
            torch.cuda.empty_cache()
    out = {"metric": "decode step us vs context length, 8B shape, B = 1", "steps": args.steps,
           "warmup": args.warmup}
    for dt, pts in points.items():
        x = np.array([p[0] for p in pts], float)
        y = np.array([p[1] for p in pts], float)
        slope, icpt = np.polyfit(x, y, 1)
        out[dt] = {"points": [{"L": int(L), "us": round(us, 2), "GBps": round(g, 1)} for L, us, g in pts],
                   "slope_us_per_token": float(slope), "intercept_us": round(float(icpt), 2),
                   "ms_per_token_x32_layers": float(slope * 32 / 1000)}
    out["fp8_over_bf16_slope"] = round(out["e4m3"]["slope_us_per_token"] / out["bf16"]["slope_us_per_token"], 4)
    out["pages_ms_per_token"] = {"H100 FA3 fp8": 2.37e-05, "B200 FlashInfer fp8": 9.72e-06}
    return out


# Whole-prompt prefill shapes: (builder, chunk length per sequence).
PREFILL_WORKLOADS = {
    "llama8b-8k": (lambda syn: syn.llama8b_long(8192, "amax"), 8192),
    "llama8b-chunk2k-at-32k": (lambda syn: syn.llama8b_long(32768, "amax"), 2048),
    "d256-8k": (lambda syn: syn.make_workload("d256-b1-L8192", 5, num_q_heads=8, num_kv_heads=1,
                                              head_dim=256, context_lens=[8192], std=0.5),
                8192),
    "gptoss-8k": (lambda syn: syn.make_workload("gptoss-b1-L8192", 4, num_q_heads=64, num_kv_heads=8,
                                                head_dim=64, context_lens=[8192]), 8192),
    "gptoss-8k-sw128": (lambda syn: syn.make_workload("gptoss-b1-L8192-sw128", 4, num_q_heads=64,
                                                      num_kv_heads=8, head_dim=64, context_lens=[8192],
                                                      layers=(("sw128", 128, syn.E4M3),)), 8192),
}


def prefill_flops(context_lens, chunk_lens, num_q_heads: int, head_dim: int, window: int = 0) -> int:
    """Algorithmic flops of one prefill call: 4 * Hq * d per (query token, attended key)
    (2 d for q.K, 2 d for p.V)."""
    total = 0
    for L, n in zip(context_lens, chunk_lens):
        pos = np.arange(int(L) - int(n), int(L), dtype=np.int64)
        pos = pos[pos >= 0]
        keys = pos + 1 if window <= 0 else np.minimum(pos + 1, window)
        total += int(keys.sum())
    return 4 * num_q_heads * head_dim * total


def prefill_bench(F, torch, syn, name: str, args) -> dict:
    """Time fp8kv_paged_prefill over one whole-prompt chunk per sequence, for the fp8 cache
    and the same data in a bf16 cache (HIP events around `launches` back-to-back calls)."""
    build, chunk = PREFILL_WORKLOADS[name]
    w = build(syn)
    layer = w.layers[0]
    pq = syn.prefill_queries(w, [chunk] * w.num_seqs, 170)
    flops = prefill_flops(w.context_lens, pq.chunk_lens, w.num_q_heads, w.head_dim, layer.sliding_window)
    dev = "cuda"
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    q, qsl = u16(pq.q), torch.from_numpy(pq.query_start_loc).to(dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    cl = torch.from_numpy(w.context_lens).to(dev)
    k_all, v_all = u16(layer.k), u16(layer.v)
    slots = torch.from_numpy(w.slot_mapping).to(dev)
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    n = w.num_blocks * Hkv * BLOCK * D
    out = torch.empty(pq.num_tokens * Hq * D, dtype=torch.bfloat16, device=dev)
    res = {"metric": "prefill attention over the paged cache: TFLOP/s (% of bf16 MFMA peak)",
           "workload": f"{name}: {w.name}, chunk {chunk}, Hq {Hq}, Hkv {Hkv}, d {D}, "
                       f"window {layer.sliding_window}",
           "flops_per_call": flops}
    launches = 20
    # with --prefill-rotated, the e4m3 and bf16 caches are also timed as rotated caches
    # (fp8kv_cache_write_rotated, then fp8kv_paged_prefill_rotated: query rotation, prefill
    # with the two-term query, output rotation); head_dim 256 has no rotated prefill
    kinds = [(c, False) for c in args.prefill_caches.split(",")]
    if args.prefill_rotated and D <= 128:
        kinds += [(c, True) for c in args.prefill_caches.split(",")]
    rws = None
    for cache, rot in kinds:
        cdt = F.FP8KV_E4M3 if cache == "e4m3" else F.FP8KV_BF16
        dt = torch.uint8 if cache == "e4m3" else torch.int16
        kc, vc = torch.zeros(n, dtype=dt, device=dev), torch.zeros(n, dtype=dt, device=dev)
        ks = layer.k_scale if cache == "e4m3" else 1.0
        vs = layer.v_scale if cache == "e4m3" else 1.0
        write = F.fp8kv_cache_write_rotated if rot else F.fp8kv_cache_write
        write(k_all, v_all, kc, vc, cdt, slots, w.num_tokens, Hkv, D, BLOCK, w.num_blocks, ks, vs)
        if rot and rws is None:
            rws_bytes = F.fp8kv_paged_prefill_rotated_workspace_size(pq.num_tokens, Hq, D)
            rws = torch.empty(rws_bytes, dtype=torch.uint8, device=dev)

        def call():
            if rot:
                F.fp8kv_paged_prefill_rotated(out, F.FP8KV_BF16, q, qsl, kc, vc, cdt, bt,
                                              w.max_blocks_per_seq, cl, w.max_context_len,
                                              w.num_seqs, pq.max_query_len, pq.num_tokens, Hq, Hkv,
                                              D, BLOCK, w.num_blocks, ks, vs, layer.sliding_window,
                                              rws, rws.numel())
                return
            F.fp8kv_paged_prefill(out, F.FP8KV_BF16, q, qsl, kc, vc, cdt, bt, w.max_blocks_per_seq,
                                  cl, w.max_context_len, w.num_seqs, pq.max_query_len, Hq, Hkv, D,
                                  BLOCK, w.num_blocks, ks, vs, layer.sliding_window)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        tf = flops / (ms * 1e-3) / 1e12
        res[cache + ("_rotated" if rot else "")] = {
            "us_per_call": round(ms * 1e3, 2), "TFLOPs": round(tf, 1),
            "pct_of_bf16_mfma_peak": round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 2)}
        del kc, vc
        torch.cuda.empty_cache()
    if "e4m3" in res and "bf16" in res:
        res["fp8_over_bf16_time"] = round(res["e4m3"]["us_per_call"] / res["bf16"]["us_per_call"], 4)
    if "e4m3" in res and "e4m3_rotated" in res:
        res["rotated_over_plain_time"] = round(res["e4m3_rotated"]["us_per_call"] / res["e4m3"]["us_per_call"], 4)
    if "e4m3" in res:
        res["roofline"] = {"bound": "mfma", "achieved": res["e4m3"]["TFLOPs"],
                           "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(res["e4m3"]["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4)}
    return res


def rotated_bench(F, torch, syn, args) -> dict:
    """Per-step time of the rotated path, as two calls (fp8kv_cache_write_rotated of each
    sequence's token, then fp8kv_paged_decode_rotated: query rotation, decode, output rotation)
    and as the fused fp8kv_decode_step_rotated, next to the plain two-call path
    (fp8kv_cache_write + fp8kv_paged_decode) and the plain fused step; HIP events over
    back-to-back steps on rotated cache instances."""
    w = WORKLOADS[args.workload](syn)
    layer = w.layers[args.layer]
    one = 2 * w.num_blocks * w.num_kv_heads * BLOCK * w.head_dim
    R = max(1, math.ceil(args.rotate_bytes * (1 << 30) / one))
    b = DecodeBench(F, torch, w, layer, R, args.num_splits)
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    nbytes = F.fp8kv_paged_decode_rotated_workspace_size(w.num_seqs, Hq, Hkv, D, BLOCK, b.maxl,
                                                        b.win, args.num_splits)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def rotated_step(i):
        F.fp8kv_cache_write_rotated(b.k_new, b.v_new, b.kc[i], b.vc[i], b.cdt, b.slots_new, b.T_new,
                                    Hkv, D, BLOCK, w.num_blocks, layer.k_scale, layer.v_scale,
                                    b.stream)
        F.fp8kv_paged_decode_rotated(b.out, F.FP8KV_BF16, b.q, b.kc[i], b.vc[i], b.cdt, b.bt,
                                     w.max_blocks_per_seq, b.cl, b.maxl, w.num_seqs, Hq, Hkv, D,
                                     BLOCK, w.num_blocks, layer.k_scale, layer.v_scale, b.win,
                                     args.num_splits, ws, nbytes, b.stream)
    def rotated_fused_step(i):
        F.fp8kv_decode_step_rotated(b.out, F.FP8KV_BF16, b.q, b.k_new, b.v_new, b.kc[i], b.vc[i],
                                    b.cdt, b.bt, w.max_blocks_per_seq, b.cl, b.maxl, w.num_seqs, Hq,
                                    Hkv, D, BLOCK, w.num_blocks, layer.k_scale, layer.v_scale,
                                    b.win, args.num_splits, b.cnt, b.cnt_bytes, ws, nbytes,
                                    b.stream)
    ms_rot, _ = b.time_steps(args.steps, min(args.warmup, 200), rotated_step)
    ms_rot_fused, _ = b.time_steps(args.steps, min(args.warmup, 200), rotated_fused_step)
    ms_two, _ = b.time_steps(args.steps, min(args.warmup, 200), b.two_call_step)
    ms_fused, _ = b.time_steps(args.steps, min(args.warmup, 200))
    return {"metric": "Hadamard-rotated decode step: us per step",
            "workload": f"{args.workload}: {w.name}",
            "rotated_step_us": round(ms_rot * 1e3, 2),
            "rotated_fused_step_us": round(ms_rot_fused * 1e3, 2),
            "two_call_step_us": round(ms_two * 1e3, 2),
            "fused_step_us": round(ms_fused * 1e3, 2),
            "rotated_over_two_call": round(ms_rot / ms_two, 4),
            "rotated_fused_over_fused": round(ms_rot_fused / ms_fused, 4),
            "GBps_rotated": round(b.bytes["step"] / (ms_rot * 1e-3) / 1e9, 1),
            "GBps_rotated_fused": round(b.bytes["step"] / (ms_rot_fused * 1e-3) / 1e9, 1)}


def _finite(x):
    """JSON has no NaN: quantities not measured in this run become null."""
    if isinstance(x, dict):
        return {k: _finite(v) for k, v in x.items()}
    if isinstance(x, float) and x != x:
        return None
    return x


if __name__ == "__main__":
    sys.exit(main())
