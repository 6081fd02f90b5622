"""CPU oracle for the fp8 KV-cache hot path (test infrastructure only).

Plain, slow, obviously-correct reference: the OCP e4m3 codec, quantise-on-write
into the paged cache, and fp64 GQA decode attention over that cache.  The
arithmetic lives in ``oracle.c`` (plain C, built with gcc, no fast-math); this
module only marshals numpy arrays through ctypes.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and this package never imports the product.

Pages cited in ``oracle.c``:
  "FP8 KV Cache Quantization: Capacity Gains and Accuracy Risk" (format, scales,
  paging, dequant-in-attention), "ctx-fp8-kv-cache-long-context-accuracy"
  (GQA ratio g), "The State of FP8 KV-Cache and Attention Quantization in vLLM".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CACHE_E4M3 = 0
CACHE_BF16 = 1
CACHE_E5M2 = 3
CACHE_INT8 = 4

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, no fast-math).  Returns the path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _bind(path: str) -> ctypes.CDLL:
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f32, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    L.oracle_bf16_to_f32.restype = f32
    L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_e4m3_decode.restype = f64
    L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.oracle_e4m3_encode.restype = ctypes.c_uint8
    L.oracle_e4m3_encode.argtypes = [f64]
    L.oracle_quantize.restype = ctypes.c_uint8
    L.oracle_quantize.argtypes = [ctypes.c_uint16, f32]
    for name, args in {
        "oracle_e4m3_decode_n": [P, P, i64],
        "oracle_e4m3_encode_n": [P, P, i64],
        "oracle_quantize_n": [P, f32, P, i64],
        "oracle_div_f32_n": [P, f32, P, i64],
        "oracle_cache_write": [P, P, P, P, i32, P, i32, i32, i32, i32, i32, f32, f32],
        "oracle_attention_rows": [P, P, P, P, i64, i32],
        "oracle_paged_decode_head": [P, P, P, P, i32, P, i32, P, i32, i32, i32, i32,
                                     f64, f64, i32, i32, i32],
        "oracle_paged_decode": [P, P, P, P, i32, P, i32, P, i32, i32, i32, i32, i32,
                                f64, f64, i32],
        "oracle_paged_decode_pairs": [P, P, i32, P, P, P, i32, P, i32, P, i32, i32, i32,
                                      i32, f64, f64, i32],
        "oracle_cache_write_per_head": [P, P, P, P, i32, P, i32, i32, i32, i32, i32, P, P],
        "oracle_cache_write_rotated_per_head": [P, P, P, P, i32, P, i32, i32, i32, i32, i32, P, P],
        "oracle_paged_decode_pairs_per_head": [P, P, i32, P, P, P, i32, P, i32, P, i32, i32, i32,
                                               i32, P, P, i32],
        "oracle_paged_prefill_pairs": [P, P, i32, P, P, i32, P, P, i32, P, i32, P, i32, i32, i32,
                                       i32, f64, f64, i32],
        "oracle_paged_prefill_rotated_pairs": [P, P, i32, P, P, i32, P, P, i32, P, i32, P, i32, i32,
                                               i32, i32, f64, f64, i32],
        "oracle_hadamard_f32": [P, i32],
        "oracle_e5m2_decode_n": [P, P, i64],
        "oracle_e5m2_encode_n": [P, P, i64],
        "oracle_int8_encode_n": [P, P, i64],
        "oracle_cache_write_codec": [P, P, P, P, i32, P, i32, i32, i32, i32, i32, f32, f32],
        "oracle_hadamard_f64": [P, i32],
        "oracle_cache_write_rotated": [P, P, P, P, i32, P, i32, i32, i32, i32, i32, f32, f32],
        "oracle_paged_decode_rotated_pairs": [P, P, i32, P, P, P, i32, P, i32, P, i32, i32, i32,
                                              i32, f64, f64, i32],
        "oracle_paged_decode_rotated_pairs_per_head": [P, P, i32, P, P, P, i32, P, i32, P, i32, i32,
                                                       i32, i32, P, P, i32],
    }.items():
        fn = getattr(L, name)
        fn.restype = None
        fn.argtypes = args
    return L


def lib() -> ctypes.CDLL:
    """The oracle library.  FP8KV_ORACLE_LIB may name another build of oracle.c: the
    mutation tests use it to run the pins against deliberately broken copies."""
    global _lib
    if _lib is None:
        override = os.environ.get("FP8KV_ORACLE_LIB")
        _lib = _bind(override if override else build())
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


# --------------------------------------------------------------- codec ----

def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib().oracle_e4m3_decode_n(_ptr(c), _ptr(out), c.size)
    return out


def e4m3_encode(y) -> np.ndarray:
    v = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_n(_ptr(v), _ptr(out), v.size)
    return out


def quantize(x_bf16_bits, scale: float) -> np.ndarray:
    """e4m3 codes of bf16 elements (given as uint16 bit patterns) divided by scale."""
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_quantize_n(_ptr(x), ctypes.c_float(scale), _ptr(out), x.size)
    return out


def div_f32(x, scale: float) -> np.ndarray:
    v = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.float32)
    lib().oracle_div_f32_n(_ptr(v), ctypes.c_float(scale), _ptr(out), v.size)
    return out


# --------------------------------------------------------- cache write ----

def cache_write(key, value, key_cache: np.ndarray, value_cache: np.ndarray, cache_dtype: int,
                slot_mapping, num_kv_heads: int, head_dim: int, block_size: int,
                num_blocks: int, k_scale: float, v_scale: float) -> None:
    """In-place write into key_cache/value_cache (u8 for e4m3, uint16 for bf16)."""
    k = np.ascontiguousarray(key, dtype=np.uint16)
    v = np.ascontiguousarray(value, dtype=np.uint16)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T = sm.shape[0]
    assert k.size == T * num_kv_heads * head_dim and v.size == k.size
    assert head_dim % 4 == 0 and block_size == 16, "the paged layout needs head_dim % 4 == 0, 16-slot blocks"
    want = np.uint16 if cache_dtype == CACHE_BF16 else np.uint8
    for c in (key_cache, value_cache):
        assert c.dtype == want and c.flags["C_CONTIGUOUS"]
        assert c.size == num_blocks * num_kv_heads * block_size * head_dim
    lib().oracle_cache_write(_ptr(k), _ptr(v), _ptr(key_cache), _ptr(value_cache), cache_dtype,
                             _ptr(sm), T, num_kv_heads, head_dim, block_size, num_blocks,
                             ctypes.c_float(k_scale), ctypes.c_float(v_scale))


def cache_write_per_head(key, value, key_cache: np.ndarray, value_cache: np.ndarray,
                         cache_dtype: int, slot_mapping, num_kv_heads: int, head_dim: int,
                         block_size: int, num_blocks: int, k_scales, v_scales) -> None:
    """cache_write with one (k, v) scale pair per kv head (float32 [num_kv_heads] each)."""
    k = np.ascontiguousarray(key, dtype=np.uint16)
    v = np.ascontiguousarray(value, dtype=np.uint16)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    ks = np.ascontiguousarray(k_scales, dtype=np.float32)
    vs = np.ascontiguousarray(v_scales, dtype=np.float32)
    T = sm.shape[0]
    assert k.size == T * num_kv_heads * head_dim and v.size == k.size
    assert ks.shape == (num_kv_heads,) and vs.shape == (num_kv_heads,)
    assert head_dim % 4 == 0 and block_size == 16, "the paged layout needs head_dim % 4 == 0, 16-slot blocks"
    want = np.uint16 if cache_dtype == CACHE_BF16 else np.uint8
    for c in (key_cache, value_cache):
        assert c.dtype == want and c.flags["C_CONTIGUOUS"]
        assert c.size == num_blocks * num_kv_heads * block_size * head_dim
    lib().oracle_cache_write_per_head(_ptr(k), _ptr(v), _ptr(key_cache), _ptr(value_cache),
                                      cache_dtype, _ptr(sm), T, num_kv_heads, head_dim,
                                      block_size, num_blocks, _ptr(ks), _ptr(vs))


# ---------------------------------------------------- decode attention ----

def attention_rows(q, K, V) -> np.ndarray:
    """Unpaged fp64 softmax attention of one query over rows K, V ([n][D])."""
    qd = np.ascontiguousarray(q, dtype=np.float64)
    Kd = np.ascontiguousarray(K, dtype=np.float64)
    Vd = np.ascontiguousarray(V, dtype=np.float64)
    D = qd.shape[0]
    n = Kd.shape[0] if Kd.size else 0
    out = np.empty(D, dtype=np.float64)
    lib().oracle_attention_rows(_ptr(out), _ptr(qd), _ptr(Kd if Kd.size else np.zeros(1)),
                                _ptr(Vd if Vd.size else np.zeros(1)), n, D)
    return out


def _decode_common(q, key_cache, value_cache, cache_dtype, block_tables, context_lens):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    assert q.shape[-1] % 4 == 0, "the paged layout needs head_dim % 4 == 0"
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    want = np.uint16 if cache_dtype == CACHE_BF16 else np.uint8
    assert key_cache.dtype == want and value_cache.dtype == want
    assert key_cache.flags["C_CONTIGUOUS"] and value_cache.flags["C_CONTIGUOUS"]
    return q, bt, cl


def paged_decode(q, key_cache, value_cache, cache_dtype: int, block_tables, context_lens,
                 num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                 k_scale: float, v_scale: float, sliding_window: int = 0) -> np.ndarray:
    """fp64 decode attention for every (sequence, query head): [B][Hq][D]."""
    q, bt, cl = _decode_common(q, key_cache, value_cache, cache_dtype, block_tables, context_lens)
    B = cl.shape[0]
    out = np.empty((B, num_q_heads, head_dim), dtype=np.float64)
    lib().oracle_paged_decode(_ptr(out), _ptr(q), _ptr(key_cache), _ptr(value_cache), cache_dtype,
                              _ptr(bt), bt.shape[1], _ptr(cl), B, num_q_heads, num_kv_heads,
                              head_dim, block_size, float(k_scale), float(v_scale),
                              int(sliding_window))
    return out


def paged_decode_pairs(pairs, q, key_cache, value_cache, cache_dtype: int, block_tables,
                       context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                       block_size: int, k_scale: float, v_scale: float,
                       sliding_window: int = 0) -> np.ndarray:
    """fp64 decode attention for the selected (b, hq) pairs only: [n][D]."""
    q, bt, cl = _decode_common(q, key_cache, value_cache, cache_dtype, block_tables, context_lens)
    pr = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    out = np.empty((pr.shape[0], head_dim), dtype=np.float64)
    lib().oracle_paged_decode_pairs(_ptr(out), _ptr(pr), pr.shape[0], _ptr(q), _ptr(key_cache),
                                    _ptr(value_cache), cache_dtype, _ptr(bt), bt.shape[1],
                                    _ptr(cl), num_q_heads, num_kv_heads, head_dim, block_size,
                                    float(k_scale), float(v_scale), int(sliding_window))
    return out


def paged_decode_pairs_per_head(pairs, q, key_cache, value_cache, cache_dtype: int, block_tables,
                                context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                block_size: int, k_scales, v_scales,
                                sliding_window: int = 0) -> np.ndarray:
    """paged_decode_pairs with one (k, v) scale pair per kv head: [n][D]."""
    q, bt, cl = _decode_common(q, key_cache, value_cache, cache_dtype, block_tables, context_lens)
    pr = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    ks = np.ascontiguousarray(np.asarray(k_scales, dtype=np.float32), dtype=np.float64)
    vs = np.ascontiguousarray(np.asarray(v_scales, dtype=np.float32), dtype=np.float64)
    assert ks.shape == (num_kv_heads,) and vs.shape == (num_kv_heads,)
    out = np.empty((pr.shape[0], head_dim), dtype=np.float64)
    lib().oracle_paged_decode_pairs_per_head(_ptr(out), _ptr(pr), pr.shape[0], _ptr(q),
                                             _ptr(key_cache), _ptr(value_cache), cache_dtype,
                                             _ptr(bt), bt.shape[1], _ptr(cl), num_q_heads,
                                             num_kv_heads, head_dim, block_size, _ptr(ks), _ptr(vs),
                                             int(sliding_window))
    return out


def paged_decode_per_head(q, key_cache, value_cache, cache_dtype: int, block_tables, context_lens,
                          num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                          k_scales, v_scales, sliding_window: int = 0) -> np.ndarray:
    """Every (sequence, query head) with per-kv-head scales: [B][Hq][D]."""
    B = np.asarray(context_lens).shape[0]
    pairs = np.array([(b, hq) for b in range(B) for hq in range(num_q_heads)], np.int32)
    out = paged_decode_pairs_per_head(pairs, q, key_cache, value_cache, cache_dtype, block_tables,
                                      context_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                                      k_scales, v_scales, sliding_window)
    return out.reshape(B, num_q_heads, head_dim)


# ------------------------------------------------------------- prefill ----

def paged_prefill_pairs(pairs, q, query_start_loc, key_cache, value_cache, cache_dtype: int,
                        block_tables, context_lens, num_q_heads: int, num_kv_heads: int,
                        head_dim: int, block_size: int, k_scale: float, v_scale: float,
                        sliding_window: int = 0) -> np.ndarray:
    """fp64 prefill attention for the selected (query row, query head) pairs: [n][D].
    q is bf16 [Tq][Hq][D]; the rows of sequence b are [qsl[b], qsl[b+1]) and sit at the
    last positions of its context (see oracle.c)."""
    q, bt, cl = _decode_common(q, key_cache, value_cache, cache_dtype, block_tables, context_lens)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    B = cl.shape[0]
    assert qsl.shape == (B + 1,) and qsl[0] == 0 and np.all(np.diff(qsl) >= 0)
    assert q.shape[0] == qsl[-1]
    pr = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    assert np.all((pr[:, 0] >= 0) & (pr[:, 0] < qsl[-1]))
    out = np.empty((pr.shape[0], head_dim), dtype=np.float64)
    lib().oracle_paged_prefill_pairs(_ptr(out), _ptr(pr), pr.shape[0], _ptr(q), _ptr(qsl), B,
                                     _ptr(key_cache), _ptr(value_cache), cache_dtype, _ptr(bt),
                                     bt.shape[1], _ptr(cl), num_q_heads, num_kv_heads, head_dim,
                                     block_size, float(k_scale), float(v_scale),
                                     int(sliding_window))
    return out


def paged_prefill_rotated_pairs(pairs, q, query_start_loc, key_cache, value_cache,
                                cache_dtype: int, block_tables, context_lens, num_q_heads: int,
                                num_kv_heads: int, head_dim: int, block_size: int, k_scale: float,
                                v_scale: float, sliding_window: int = 0) -> np.ndarray:
    """paged_prefill_pairs over a rotated cache: each query row rotated, attention in the
    rotated space, each output row rotated back (fp64): [n][D]."""
    q, bt, cl = _decode_common(q, key_cache, value_cache, cache_dtype, block_tables, context_lens)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    B = cl.shape[0]
    assert qsl.shape == (B + 1,) and qsl[0] == 0 and np.all(np.diff(qsl) >= 0)
    assert q.shape[0] == qsl[-1] and head_dim & (head_dim - 1) == 0
    pr = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    assert np.all((pr[:, 0] >= 0) & (pr[:, 0] < qsl[-1]))
    out = np.empty((pr.shape[0], head_dim), dtype=np.float64)
    lib().oracle_paged_prefill_rotated_pairs(_ptr(out), _ptr(pr), pr.shape[0], _ptr(q), _ptr(qsl), B,
                                             _ptr(key_cache), _ptr(value_cache), cache_dtype,
                                             _ptr(bt), bt.shape[1], _ptr(cl), num_q_heads,
                                             num_kv_heads, head_dim, block_size, float(k_scale),
                                             float(v_scale), int(sliding_window))
    return out


def paged_prefill_rotated(q, query_start_loc, key_cache, value_cache, cache_dtype: int,
                          block_tables, context_lens, num_q_heads: int, num_kv_heads: int,
                          head_dim: int, block_size: int, k_scale: float, v_scale: float,
                          sliding_window: int = 0) -> np.ndarray:
    """Every (query row, query head) over a rotated cache: [Tq][Hq][D]."""
    Tq = int(np.asarray(query_start_loc)[-1])
    pairs = np.array([(r, hq) for r in range(Tq) for hq in range(num_q_heads)], np.int32)
    out = paged_prefill_rotated_pairs(pairs, q, query_start_loc, key_cache, value_cache,
                                      cache_dtype, block_tables, context_lens, num_q_heads,
                                      num_kv_heads, head_dim, block_size, k_scale, v_scale,
                                      sliding_window)
    return out.reshape(Tq, num_q_heads, head_dim)


def paged_prefill(q, query_start_loc, key_cache, value_cache, cache_dtype: int, block_tables,
                  context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  block_size: int, k_scale: float, v_scale: float,
                  sliding_window: int = 0) -> np.ndarray:
    """Every (query row, query head): [Tq][Hq][D]."""
    Tq = int(np.asarray(query_start_loc)[-1])
    pairs = np.array([(r, hq) for r in range(Tq) for hq in range(num_q_heads)], np.int32)
    out = paged_prefill_pairs(pairs, q, query_start_loc, key_cache, value_cache, cache_dtype,
                              block_tables, context_lens, num_q_heads, num_kv_heads, head_dim,
                              block_size, k_scale, v_scale, sliding_window)
    return out.reshape(Tq, num_q_heads, head_dim)


# ------------------------------------------------------------ rotation ----

def hadamard_f32(x) -> np.ndarray:
    """Normalized Hadamard rotation of the last axis in f32 (oracle.c's butterfly order)."""
    a = np.array(x, dtype=np.float32, order="C", copy=True)
    d = a.shape[-1]
    assert d & (d - 1) == 0
    rows = a.reshape(-1, d)
    for r in range(rows.shape[0]):
        row = np.ascontiguousarray(rows[r])
        lib().oracle_hadamard_f32(_ptr(row), d)
        rows[r] = row
    return rows.reshape(a.shape)


def hadamard_f64(x) -> np.ndarray:
    """The same rotation in double."""
    a = np.array(x, dtype=np.float64, order="C", copy=True)
    d = a.shape[-1]
    assert d & (d - 1) == 0
    rows = a.reshape(-1, d)
    for r in range(rows.shape[0]):
        row = np.ascontiguousarray(rows[r])
        lib().oracle_hadamard_f64(_ptr(row), d)
        rows[r] = row
    return rows.reshape(a.shape)


def cache_write_rotated(key, value, key_cache: np.ndarray, value_cache: np.ndarray,
                        cache_dtype: int, slot_mapping, num_kv_heads: int, head_dim: int,
                        block_size: int, num_blocks: int, k_scale: float, v_scale: float) -> None:
    """cache_write of Hadamard-rotated K and V rows (rotation in f32, then the quantiser)."""
    k = np.ascontiguousarray(key, dtype=np.uint16)
    v = np.ascontiguousarray(value, dtype=np.uint16)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T = sm.shape[0]
    assert k.size == T * num_kv_heads * head_dim and v.size == k.size
    assert head_dim & (head_dim - 1) == 0 and block_size == 16
    want = np.uint16 if cache_dtype == CACHE_BF16 else np.uint8
    assert key_cache.dtype == want and value_cache.dtype == want
    assert key_cache.flags["C_CONTIGUOUS"] and value_cache.flags["C_CONTIGUOUS"]
    lib().oracle_cache_write_rotated(_ptr(k), _ptr(v), _ptr(key_cache), _ptr(value_cache),
                                     cache_dtype, _ptr(sm), T, num_kv_heads, head_dim,
                                     block_size, num_blocks, float(k_scale), float(v_scale))


def paged_decode_rotated_pairs(pairs, q, key_cache, value_cache, cache_dtype: int, block_tables,
                               context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                               block_size: int, k_scale: float, v_scale: float,
                               sliding_window: int = 0) -> np.ndarray:
    """Decode over a rotated cache for selected (b, hq) pairs: q rotated, attention in the
    rotated space, output rotated back (fp64): [n][D]."""
    q, bt, cl = _decode_common(q, key_cache, value_cache, cache_dtype, block_tables, context_lens)
    pr = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    out = np.empty((pr.shape[0], head_dim), dtype=np.float64)
    lib().oracle_paged_decode_rotated_pairs(_ptr(out), _ptr(pr), pr.shape[0], _ptr(q),
                                            _ptr(key_cache), _ptr(value_cache), cache_dtype,
                                            _ptr(bt), bt.shape[1], _ptr(cl), num_q_heads,
                                            num_kv_heads, head_dim, block_size, float(k_scale),
                                            float(v_scale), int(sliding_window))
    return out


def cache_write_rotated_per_head(key, value, key_cache: np.ndarray, value_cache: np.ndarray,
                                 cache_dtype: int, slot_mapping, num_kv_heads: int, head_dim: int,
                                 block_size: int, num_blocks: int, k_scales, v_scales) -> None:
    """cache_write_rotated with one (k, v) scale pair per kv head (float32 [num_kv_heads])."""
    k = np.ascontiguousarray(key, dtype=np.uint16)
    v = np.ascontiguousarray(value, dtype=np.uint16)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    ks = np.ascontiguousarray(k_scales, dtype=np.float32)
    vs = np.ascontiguousarray(v_scales, dtype=np.float32)
    T = sm.shape[0]
    assert k.size == T * num_kv_heads * head_dim and v.size == k.size
    assert ks.shape == (num_kv_heads,) and vs.shape == (num_kv_heads,)
    assert head_dim & (head_dim - 1) == 0 and block_size == 16
    want = np.uint16 if cache_dtype == CACHE_BF16 else np.uint8
    assert key_cache.dtype == want and value_cache.dtype == want
    assert key_cache.flags["C_CONTIGUOUS"] and value_cache.flags["C_CONTIGUOUS"]
    lib().oracle_cache_write_rotated_per_head(_ptr(k), _ptr(v), _ptr(key_cache), _ptr(value_cache),
                                              cache_dtype, _ptr(sm), T, num_kv_heads, head_dim,
                                              block_size, num_blocks, _ptr(ks), _ptr(vs))


def paged_decode_rotated_pairs_per_head(pairs, q, key_cache, value_cache, cache_dtype: int,
                                        block_tables, context_lens, num_q_heads: int,
                                        num_kv_heads: int, head_dim: int, block_size: int,
                                        k_scales, v_scales, sliding_window: int = 0) -> np.ndarray:
    """paged_decode_rotated_pairs with one (k, v) scale pair per kv head: [n][D]."""
    q, bt, cl = _decode_common(q, key_cache, value_cache, cache_dtype, block_tables, context_lens)
    pr = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    ks = np.ascontiguousarray(np.asarray(k_scales, dtype=np.float32), dtype=np.float64)
    vs = np.ascontiguousarray(np.asarray(v_scales, dtype=np.float32), dtype=np.float64)
    assert ks.shape == (num_kv_heads,) and vs.shape == (num_kv_heads,)
    out = np.empty((pr.shape[0], head_dim), dtype=np.float64)
    lib().oracle_paged_decode_rotated_pairs_per_head(_ptr(out), _ptr(pr), pr.shape[0], _ptr(q),
                                                     _ptr(key_cache), _ptr(value_cache),
                                                     cache_dtype, _ptr(bt), bt.shape[1], _ptr(cl),
                                                     num_q_heads, num_kv_heads, head_dim,
                                                     block_size, _ptr(ks), _ptr(vs),
                                                     int(sliding_window))
    return out


def paged_decode_rotated_per_head(q, key_cache, value_cache, cache_dtype: int, block_tables,
                                  context_lens, num_q_heads: int, num_kv_heads: int,
                                  head_dim: int, block_size: int, k_scales, v_scales,
                                  sliding_window: int = 0) -> np.ndarray:
    """Every (sequence, query head) over a rotated cache with per-kv-head scales: [B][Hq][D]."""
    B = np.asarray(context_lens).shape[0]
    pairs = np.array([(b, hq) for b in range(B) for hq in range(num_q_heads)], np.int32)
    out = paged_decode_rotated_pairs_per_head(pairs, q, key_cache, value_cache, cache_dtype,
                                              block_tables, context_lens, num_q_heads,
                                              num_kv_heads, head_dim, block_size, k_scales,
                                              v_scales, sliding_window)
    return out.reshape(B, num_q_heads, head_dim)


def paged_decode_rotated(q, key_cache, value_cache, cache_dtype: int, block_tables, context_lens,
                         num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                         k_scale: float, v_scale: float, sliding_window: int = 0) -> np.ndarray:
    """Every (sequence, query head) over a rotated cache: [B][Hq][D]."""
    B = np.asarray(context_lens).shape[0]
    pairs = np.array([(b, hq) for b in range(B) for hq in range(num_q_heads)], np.int32)
    out = paged_decode_rotated_pairs(pairs, q, key_cache, value_cache, cache_dtype, block_tables,
                                     context_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                                     k_scale, v_scale, sliding_window)
    return out.reshape(B, num_q_heads, head_dim)


# -------------------------------------------------------- other codecs ----

def e5m2_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib().oracle_e5m2_decode_n(_ptr(c), _ptr(out), c.size)
    return out


def e5m2_encode(y) -> np.ndarray:
    v = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e5m2_encode_n(_ptr(v), _ptr(out), v.size)
    return out


def int8_encode(y) -> np.ndarray:
    v = np.ascontiguousarray(y, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_int8_encode_n(_ptr(v), _ptr(out), v.size)
    return out


def int8_decode(codes) -> np.ndarray:
    return np.ascontiguousarray(codes, dtype=np.uint8).view(np.int8).astype(np.float64)


def cache_write_codec(key, value, key_cache: np.ndarray, value_cache: np.ndarray, codec: int,
                      slot_mapping, num_kv_heads: int, head_dim: int, block_size: int,
                      num_blocks: int, k_scale: float, v_scale: float) -> None:
    """cache_write with a one-byte codec (CACHE_E4M3, CACHE_E5M2 or CACHE_INT8)."""
    assert codec in (CACHE_E4M3, CACHE_E5M2, CACHE_INT8)
    k = np.ascontiguousarray(key, dtype=np.uint16)
    v = np.ascontiguousarray(value, dtype=np.uint16)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T = sm.shape[0]
    assert k.size == T * num_kv_heads * head_dim and v.size == k.size
    assert key_cache.dtype == np.uint8 and value_cache.dtype == np.uint8
    assert key_cache.flags["C_CONTIGUOUS"] and value_cache.flags["C_CONTIGUOUS"]
    lib().oracle_cache_write_codec(_ptr(k), _ptr(v), _ptr(key_cache), _ptr(value_cache), codec,
                                   _ptr(sm), T, num_kv_heads, head_dim, block_size, num_blocks,
                                   float(k_scale), float(v_scale))
