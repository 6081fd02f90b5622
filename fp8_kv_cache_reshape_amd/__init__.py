"""Python binding of libfp8kv (fp8 E4M3 paged KV cache + GQA decode attention, gfx950).

Argument marshalling only: every function here has the name and argument list of the C
entry point in include/fp8kv.h, accepts torch tensors (or raw integer addresses) for the
pointer arguments, and raises Fp8kvError on a negative status.  All work runs in the HIP
kernels of libfp8kv.so on the caller's stream (torch's current stream by default); there
is no fallback of any kind: importing this package fails if the library is not built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libfp8kv.so")

FP8KV_OK = 0
FP8KV_ERR_NULL = -1
FP8KV_ERR_SHAPE = -2
FP8KV_ERR_UNSUPPORTED = -3
FP8KV_ERR_SCALE = -4
FP8KV_ERR_WORKSPACE = -5
FP8KV_ERR_HIP = -6
FP8KV_ERR_SCRATCH = -7

FP8KV_E4M3 = 0
FP8KV_BF16 = 1
FP8KV_F32 = 2
FP8KV_E5M2 = 3
FP8KV_INT8 = 4

BLOCK_SIZE = 16

# limits of fp8kv_decode_step_noalloc's fixed device array
FP8KV_NOALLOC_MAX_GROUPS = 2048
FP8KV_NOALLOC_MAX_PARTIAL_BYTES = 14155776

# bits of the device error word (fp8kv_set_error_word)
FP8KV_DEVERR_BLOCK_ID = 1
FP8KV_DEVERR_SLOT = 2
FP8KV_DEVERR_CONTEXT_LEN = 4
FP8KV_DEVERR_QUERY_LEN = 8

# Every symbol include/fp8kv.h declares, with its ctypes signature.
_P, _I, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "fp8kv_status_string": (ctypes.c_char_p, [_I]),
    "fp8kv_version": (_I, []),
    "fp8kv_last_hip_error": (ctypes.c_char_p, []),
    "fp8kv_set_error_word": (_I, [_P]),
    "fp8kv_decode_counters_size": (_SZ, [_I, _I]),
    "fp8kv_cache_write": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _F, _F, _P]),
    "fp8kv_cache_write_per_head": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "fp8kv_paged_decode_num_splits": (_I, [_I, _I, _I, _I, _I, _I, _I]),
    "fp8kv_paged_decode_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "fp8kv_paged_decode": (_I, [_P, _I, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I,
                                _F, _F, _I, _I, _P, _SZ, _P, _SZ, _P]),
    "fp8kv_paged_decode_per_head": (_I, [_P, _I, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I,
                                         _I, _I, _P, _P, _I, _I, _P, _SZ, _P, _SZ, _P]),
    "fp8kv_paged_decode_partial": (_I, [_P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I,
                                        _F, _I, _I, _P, _SZ, _P]),
    "fp8kv_paged_decode_merge": (_I, [_P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P,
                                      _SZ, _P]),
    "fp8kv_paged_decode_partial_per_head": (_I, [_P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I,
                                                 _I, _I, _P, _I, _I, _P, _SZ, _P]),
    "fp8kv_paged_decode_merge_per_head": (_I, [_P, _I, _I, _P, _I, _I, _I, _I, _I, _I, _I, _P,
                                               _I, _I, _P, _SZ, _P]),
    "fp8kv_decode_step": (_I, [_P, _I, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I,
                               _I, _F, _F, _I, _I, _P, _SZ, _P, _SZ, _P]),
    "fp8kv_decode_step_per_head": (_I, [_P, _I, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I,
                                        _I, _I, _I, _I, _P, _P, _I, _I, _P, _SZ, _P, _SZ, _P]),
    "fp8kv_decode_step_noalloc": (_I, [_P, _I, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I,
                                       _I, _I, _I, _F, _F, _I, _I, _P]),
    "fp8kv_paged_prefill": (_I, [_P, _I, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I,
                                 _I, _I, _F, _F, _I, _P]),
    "fp8kv_paged_prefill_per_head": (_I, [_P, _I, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I,
                                          _I, _I, _I, _I, _P, _P, _I, _P]),
    "fp8kv_cache_write_rotated": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _F, _F, _P]),
    "fp8kv_paged_decode_rotated_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "fp8kv_paged_decode_rotated": (_I, [_P, _I, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I,
                                        _I, _F, _F, _I, _I, _P, _SZ, _P]),
    "fp8kv_decode_step_rotated": (_I, [_P, _I, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I,
                                       _I, _I, _I, _F, _F, _I, _I, _P, _SZ, _P, _SZ, _P]),
    "fp8kv_cache_write_rotated_per_head": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P, _P,
                                                _P]),
    "fp8kv_paged_prefill_rotated_workspace_size": (_SZ, [_I, _I, _I]),
    "fp8kv_paged_prefill_rotated": (_I, [_P, _I, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I,
                                         _I, _I, _I, _I, _F, _F, _I, _P, _SZ, _P]),
    "fp8kv_paged_decode_rotated_per_head": (_I, [_P, _I, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I,
                                                 _I, _I, _I, _P, _P, _I, _I, _P, _SZ, _P]),
    "fp8kv_decode_step_rotated_per_head": (_I, [_P, _I, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I,
                                                _I, _I, _I, _I, _I, _P, _P, _I, _I, _P, _SZ, _P,
                                                _SZ, _P]),
}

if not os.path.exists(LIBRARY_PATH):
    raise ImportError(f"{LIBRARY_PATH} is not built: run `python fp8_kv_cache_reshape_amd/build.py` "
                      "(hipcc, gfx950) first; this package has no non-HIP fallback")

# torch ships its own HIP runtime under the same soname as the system one.  Loading torch
# first makes libfp8kv resolve libamdhip64.so.7 to that already-loaded copy, so the process
# has a single HIP runtime and torch's device pointers and stream handles are valid here.
import torch  # noqa: E402,F401  (imported for its HIP runtime, before the library)

lib = ctypes.CDLL(LIBRARY_PATH)
for _name, (_res, _args) in SIGNATURES.items():
    if not hasattr(lib, _name):
        raise ImportError(f"{LIBRARY_PATH} lacks {_name}: it is older than the sources; rebuild it "
                          "with `python fp8_kv_cache_reshape_amd/build.py`")
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class Fp8kvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = f", {fp8kv_last_hip_error()}" if status == FP8KV_ERR_HIP else ""
        super().__init__(f"{where}: {fp8kv_status_string(status)} (status {status}{detail})")


def _addr(x) -> int:
    """Device address of a tensor (or pass-through of an int / None)."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> int:
    if stream is not None:
        return stream if isinstance(stream, int) else int(stream.cuda_stream)
    import torch
    if torch.cuda.is_available():
        return int(torch.cuda.current_stream().cuda_stream)
    return 0


def _check(status: int, where: str) -> int:
    if status < 0:
        raise Fp8kvError(status, where)
    return status


def fp8kv_status_string(status: int) -> str:
    return lib.fp8kv_status_string(int(status)).decode()


def fp8kv_version() -> int:
    return int(lib.fp8kv_version())


def fp8kv_last_hip_error() -> str:
    return lib.fp8kv_last_hip_error().decode()


def fp8kv_set_error_word(word) -> int:
    return _check(lib.fp8kv_set_error_word(_addr(word)), "fp8kv_set_error_word")


def fp8kv_decode_counters_size(max_num_seqs, num_kv_heads) -> int:
    return int(lib.fp8kv_decode_counters_size(max_num_seqs, num_kv_heads))


def fp8kv_cache_write(key, value, key_cache, value_cache, cache_dtype, slot_mapping, num_tokens,
                      num_kv_heads, head_dim, block_size, num_blocks, k_scale, v_scale,
                      stream=None) -> int:
    return _check(lib.fp8kv_cache_write(_addr(key), _addr(value), _addr(key_cache),
                                        _addr(value_cache), cache_dtype, _addr(slot_mapping),
                                        num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                                        k_scale, v_scale, _stream(stream)), "fp8kv_cache_write")


def fp8kv_cache_write_per_head(key, value, key_cache, value_cache, cache_dtype, slot_mapping,
                               num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                               k_scales, v_scales, stream=None) -> int:
    return _check(lib.fp8kv_cache_write_per_head(_addr(key), _addr(value), _addr(key_cache),
                                                 _addr(value_cache), cache_dtype,
                                                 _addr(slot_mapping), num_tokens, num_kv_heads,
                                                 head_dim, block_size, num_blocks, _addr(k_scales),
                                                 _addr(v_scales), _stream(stream)),
                  "fp8kv_cache_write_per_head")


def fp8kv_paged_decode_num_splits(num_seqs, num_kv_heads, head_dim, block_size, max_context_len,
                                  sliding_window, num_splits) -> int:
    return _check(lib.fp8kv_paged_decode_num_splits(num_seqs, num_kv_heads, head_dim, block_size,
                                                    max_context_len, sliding_window, num_splits),
                  "fp8kv_paged_decode_num_splits")


def fp8kv_paged_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_context_len, sliding_window, num_splits) -> int:
    return int(lib.fp8kv_paged_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                     block_size, max_context_len, sliding_window,
                                                     num_splits))


def fp8kv_paged_decode(out, out_dtype, query, key_cache, value_cache, cache_dtype, block_tables,
                       max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, k_scale, v_scale,
                       sliding_window, num_splits, counters, counters_bytes, workspace,
                       workspace_bytes, stream=None) -> int:
    return _check(lib.fp8kv_paged_decode(_addr(out), out_dtype, _addr(query), _addr(key_cache),
                                         _addr(value_cache), cache_dtype, _addr(block_tables),
                                         max_blocks_per_seq, _addr(context_lens), max_context_len,
                                         num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                         num_blocks, k_scale, v_scale, sliding_window, num_splits,
                                         _addr(counters), counters_bytes, _addr(workspace),
                                         workspace_bytes, _stream(stream)),
                  "fp8kv_paged_decode")


def fp8kv_paged_decode_per_head(out, out_dtype, query, key_cache, value_cache, cache_dtype,
                                block_tables, max_blocks_per_seq, context_lens, max_context_len,
                                num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                num_blocks, k_scales, v_scales, sliding_window, num_splits,
                                counters, counters_bytes, workspace, workspace_bytes,
                                stream=None) -> int:
    return _check(lib.fp8kv_paged_decode_per_head(_addr(out), out_dtype, _addr(query),
                                                  _addr(key_cache), _addr(value_cache), cache_dtype,
                                                  _addr(block_tables), max_blocks_per_seq,
                                                  _addr(context_lens), max_context_len, num_seqs,
                                                  num_q_heads, num_kv_heads, head_dim, block_size,
                                                  num_blocks, _addr(k_scales), _addr(v_scales),
                                                  sliding_window, num_splits, _addr(counters),
                                                  counters_bytes, _addr(workspace),
                                                  workspace_bytes, _stream(stream)),
                  "fp8kv_paged_decode_per_head")


def fp8kv_paged_decode_partial(query, key_cache, value_cache, cache_dtype, block_tables,
                               max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                               num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, k_scale,
                               sliding_window, num_splits, workspace, workspace_bytes,
                               stream=None) -> int:
    return _check(lib.fp8kv_paged_decode_partial(_addr(query), _addr(key_cache), _addr(value_cache),
                                                 cache_dtype, _addr(block_tables), max_blocks_per_seq,
                                                 _addr(context_lens), max_context_len, num_seqs,
                                                 num_q_heads, num_kv_heads, head_dim, block_size,
                                                 num_blocks, k_scale, sliding_window, num_splits,
                                                 _addr(workspace), workspace_bytes, _stream(stream)),
                  "fp8kv_paged_decode_partial")


def fp8kv_paged_decode_merge(out, out_dtype, context_lens, max_context_len, max_blocks_per_seq,
                             num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, v_scale,
                             sliding_window, num_splits, workspace, workspace_bytes,
                             stream=None) -> int:
    return _check(lib.fp8kv_paged_decode_merge(_addr(out), out_dtype, _addr(context_lens),
                                               max_context_len, max_blocks_per_seq, num_seqs,
                                               num_q_heads, num_kv_heads, head_dim, block_size,
                                               v_scale, sliding_window, num_splits, _addr(workspace),
                                               workspace_bytes, _stream(stream)),
                  "fp8kv_paged_decode_merge")


def fp8kv_paged_decode_partial_per_head(query, key_cache, value_cache, cache_dtype, block_tables,
                                        max_blocks_per_seq, context_lens, max_context_len,
                                        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                        num_blocks, k_scales, sliding_window, num_splits,
                                        workspace, workspace_bytes, stream=None) -> int:
    return _check(lib.fp8kv_paged_decode_partial_per_head(
        _addr(query), _addr(key_cache), _addr(value_cache), cache_dtype, _addr(block_tables),
        max_blocks_per_seq, _addr(context_lens), max_context_len, num_seqs, num_q_heads,
        num_kv_heads, head_dim, block_size, num_blocks, _addr(k_scales), sliding_window,
        num_splits, _addr(workspace), workspace_bytes, _stream(stream)),
        "fp8kv_paged_decode_partial_per_head")


def fp8kv_paged_decode_merge_per_head(out, out_dtype, cache_dtype, context_lens, max_context_len,
                                      max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads,
                                      head_dim, block_size, v_scales, sliding_window, num_splits,
                                      workspace, workspace_bytes, stream=None) -> int:
    return _check(lib.fp8kv_paged_decode_merge_per_head(
        _addr(out), out_dtype, cache_dtype, _addr(context_lens), max_context_len,
        max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
        _addr(v_scales), sliding_window, num_splits, _addr(workspace), workspace_bytes,
        _stream(stream)), "fp8kv_paged_decode_merge_per_head")


def fp8kv_decode_step(out, out_dtype, query, key_new, value_new, key_cache, value_cache,
                      cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                      max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                      num_blocks, k_scale, v_scale, sliding_window, num_splits, counters,
                      counters_bytes, workspace, workspace_bytes, stream=None) -> int:
    return _check(lib.fp8kv_decode_step(_addr(out), out_dtype, _addr(query), _addr(key_new),
                                        _addr(value_new), _addr(key_cache), _addr(value_cache),
                                        cache_dtype, _addr(block_tables), max_blocks_per_seq,
                                        _addr(context_lens), max_context_len, num_seqs,
                                        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                        k_scale, v_scale, sliding_window, num_splits,
                                        _addr(counters), counters_bytes, _addr(workspace),
                                        workspace_bytes, _stream(stream)),
                  "fp8kv_decode_step")


def fp8kv_decode_step_per_head(out, out_dtype, query, key_new, value_new, key_cache, value_cache,
                               cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                               max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                               block_size, num_blocks, k_scales, v_scales, sliding_window,
                               num_splits, counters, counters_bytes, workspace, workspace_bytes,
                               stream=None) -> int:
    return _check(lib.fp8kv_decode_step_per_head(_addr(out), out_dtype, _addr(query),
                                                 _addr(key_new), _addr(value_new),
                                                 _addr(key_cache), _addr(value_cache), cache_dtype,
                                                 _addr(block_tables), max_blocks_per_seq,
                                                 _addr(context_lens), max_context_len, num_seqs,
                                                 num_q_heads, num_kv_heads, head_dim, block_size,
                                                 num_blocks, _addr(k_scales), _addr(v_scales),
                                                 sliding_window, num_splits, _addr(counters),
                                                 counters_bytes, _addr(workspace),
                                                 workspace_bytes, _stream(stream)),
                  "fp8kv_decode_step_per_head")


def fp8kv_decode_step_noalloc(out, out_dtype, query, key_new, value_new, key_cache, value_cache,
                              cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                              max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                              block_size, num_blocks, k_scale, v_scale, sliding_window, num_splits,
                              stream=None) -> int:
    return _check(lib.fp8kv_decode_step_noalloc(_addr(out), out_dtype, _addr(query), _addr(key_new),
                                                _addr(value_new), _addr(key_cache),
                                                _addr(value_cache), cache_dtype,
                                                _addr(block_tables), max_blocks_per_seq,
                                                _addr(context_lens), max_context_len, num_seqs,
                                                num_q_heads, num_kv_heads, head_dim, block_size,
                                                num_blocks, k_scale, v_scale, sliding_window,
                                                num_splits, _stream(stream)),
                  "fp8kv_decode_step_noalloc")


def fp8kv_paged_prefill(out, out_dtype, query, query_start_loc, key_cache, value_cache,
                        cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                        max_context_len, num_seqs, max_query_len, num_q_heads, num_kv_heads,
                        head_dim, block_size, num_blocks, k_scale, v_scale, sliding_window,
                        stream=None) -> int:
    return _check(lib.fp8kv_paged_prefill(_addr(out), out_dtype, _addr(query),
                                          _addr(query_start_loc), _addr(key_cache),
                                          _addr(value_cache), cache_dtype, _addr(block_tables),
                                          max_blocks_per_seq, _addr(context_lens), max_context_len,
                                          num_seqs, max_query_len, num_q_heads, num_kv_heads,
                                          head_dim, block_size, num_blocks, k_scale, v_scale,
                                          sliding_window, _stream(stream)),
                  "fp8kv_paged_prefill")


def fp8kv_paged_prefill_per_head(out, out_dtype, query, query_start_loc, key_cache, value_cache,
                                 cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                                 max_context_len, num_seqs, max_query_len, num_q_heads,
                                 num_kv_heads, head_dim, block_size, num_blocks, k_scales,
                                 v_scales, sliding_window, stream=None) -> int:
    return _check(lib.fp8kv_paged_prefill_per_head(_addr(out), out_dtype, _addr(query),
                                                   _addr(query_start_loc), _addr(key_cache),
                                                   _addr(value_cache), cache_dtype,
                                                   _addr(block_tables), max_blocks_per_seq,
                                                   _addr(context_lens), max_context_len, num_seqs,
                                                   max_query_len, num_q_heads, num_kv_heads,
                                                   head_dim, block_size, num_blocks,
                                                   _addr(k_scales), _addr(v_scales),
                                                   sliding_window, _stream(stream)),
                  "fp8kv_paged_prefill_per_head")


def fp8kv_cache_write_rotated(key, value, key_cache, value_cache, cache_dtype, slot_mapping,
                              num_tokens, num_kv_heads, head_dim, block_size, num_blocks, k_scale,
                              v_scale, stream=None) -> int:
    return _check(lib.fp8kv_cache_write_rotated(_addr(key), _addr(value), _addr(key_cache),
                                                _addr(value_cache), cache_dtype, _addr(slot_mapping),
                                                num_tokens, num_kv_heads, head_dim, block_size,
                                                num_blocks, k_scale, v_scale, _stream(stream)),
                  "fp8kv_cache_write_rotated")


def fp8kv_paged_decode_rotated_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              block_size, max_context_len, sliding_window,
                                              num_splits) -> int:
    return int(lib.fp8kv_paged_decode_rotated_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                             head_dim, block_size, max_context_len,
                                                             sliding_window, num_splits))


def fp8kv_paged_decode_rotated(out, out_dtype, query, key_cache, value_cache, cache_dtype,
                               block_tables, max_blocks_per_seq, context_lens, max_context_len,
                               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               num_blocks, k_scale, v_scale, sliding_window, num_splits, workspace,
                               workspace_bytes, stream=None) -> int:
    return _check(lib.fp8kv_paged_decode_rotated(_addr(out), out_dtype, _addr(query),
                                                 _addr(key_cache), _addr(value_cache), cache_dtype,
                                                 _addr(block_tables), max_blocks_per_seq,
                                                 _addr(context_lens), max_context_len, num_seqs,
                                                 num_q_heads, num_kv_heads, head_dim, block_size,
                                                 num_blocks, k_scale, v_scale, sliding_window,
                                                 num_splits, _addr(workspace), workspace_bytes,
                                                 _stream(stream)),
                  "fp8kv_paged_decode_rotated")


def fp8kv_decode_step_rotated(out, out_dtype, query, key_new, value_new, key_cache, value_cache,
                              cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                              max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
                              block_size, num_blocks, k_scale, v_scale, sliding_window, num_splits,
                              counters, counters_bytes, workspace, workspace_bytes,
                              stream=None) -> int:
    return _check(lib.fp8kv_decode_step_rotated(_addr(out), out_dtype, _addr(query), _addr(key_new),
                                                _addr(value_new), _addr(key_cache),
                                                _addr(value_cache), cache_dtype,
                                                _addr(block_tables), max_blocks_per_seq,
                                                _addr(context_lens), max_context_len, num_seqs,
                                                num_q_heads, num_kv_heads, head_dim, block_size,
                                                num_blocks, k_scale, v_scale, sliding_window,
                                                num_splits, _addr(counters), counters_bytes,
                                                _addr(workspace), workspace_bytes, _stream(stream)),
                  "fp8kv_decode_step_rotated")


def fp8kv_cache_write_rotated_per_head(key, value, key_cache, value_cache, cache_dtype, slot_mapping,
                                       num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                                       k_scales, v_scales, stream=None) -> int:
    return _check(lib.fp8kv_cache_write_rotated_per_head(_addr(key), _addr(value), _addr(key_cache),
                                                         _addr(value_cache), cache_dtype,
                                                         _addr(slot_mapping), num_tokens,
                                                         num_kv_heads, head_dim, block_size,
                                                         num_blocks, _addr(k_scales),
                                                         _addr(v_scales), _stream(stream)),
                  "fp8kv_cache_write_rotated_per_head")


def fp8kv_paged_decode_rotated_per_head(out, out_dtype, query, key_cache, value_cache, cache_dtype,
                                        block_tables, max_blocks_per_seq, context_lens,
                                        max_context_len, num_seqs, num_q_heads, num_kv_heads,
                                        head_dim, block_size, num_blocks, k_scales, v_scales,
                                        sliding_window, num_splits, workspace, workspace_bytes,
                                        stream=None) -> int:
    return _check(lib.fp8kv_paged_decode_rotated_per_head(
        _addr(out), out_dtype, _addr(query), _addr(key_cache), _addr(value_cache), cache_dtype,
        _addr(block_tables), max_blocks_per_seq, _addr(context_lens), max_context_len, num_seqs,
        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, _addr(k_scales),
        _addr(v_scales), sliding_window, num_splits, _addr(workspace), workspace_bytes,
        _stream(stream)), "fp8kv_paged_decode_rotated_per_head")


def fp8kv_decode_step_rotated_per_head(out, out_dtype, query, key_new, value_new, key_cache,
                                       value_cache, cache_dtype, block_tables, max_blocks_per_seq,
                                       context_lens, max_context_len, num_seqs, num_q_heads,
                                       num_kv_heads, head_dim, block_size, num_blocks, k_scales,
                                       v_scales, sliding_window, num_splits, counters,
                                       counters_bytes, workspace, workspace_bytes,
                                       stream=None) -> int:
    return _check(lib.fp8kv_decode_step_rotated_per_head(
        _addr(out), out_dtype, _addr(query), _addr(key_new), _addr(value_new), _addr(key_cache),
        _addr(value_cache), cache_dtype, _addr(block_tables), max_blocks_per_seq,
        _addr(context_lens), max_context_len, num_seqs, num_q_heads, num_kv_heads, head_dim,
        block_size, num_blocks, _addr(k_scales), _addr(v_scales), sliding_window, num_splits,
        _addr(counters), counters_bytes, _addr(workspace), workspace_bytes, _stream(stream)),
        "fp8kv_decode_step_rotated_per_head")


def fp8kv_paged_prefill_rotated_workspace_size(num_query_tokens, num_q_heads, head_dim) -> int:
    return int(lib.fp8kv_paged_prefill_rotated_workspace_size(num_query_tokens, num_q_heads, head_dim))


def fp8kv_paged_prefill_rotated(out, out_dtype, query, query_start_loc, key_cache, value_cache,
                                cache_dtype, block_tables, max_blocks_per_seq, context_lens,
                                max_context_len, num_seqs, max_query_len, num_query_tokens,
                                num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                k_scale, v_scale, sliding_window, workspace, workspace_bytes,
                                stream=None) -> int:
    return _check(lib.fp8kv_paged_prefill_rotated(
        _addr(out), out_dtype, _addr(query), _addr(query_start_loc), _addr(key_cache),
        _addr(value_cache), cache_dtype, _addr(block_tables), max_blocks_per_seq,
        _addr(context_lens), max_context_len, num_seqs, max_query_len, num_query_tokens,
        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, k_scale, v_scale,
        sliding_window, _addr(workspace), workspace_bytes, _stream(stream)),
        "fp8kv_paged_prefill_rotated")
