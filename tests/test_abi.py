"""The C-ABI library loads, exports every symbol include/fp8kv.h declares, and rejects bad
arguments on the host before any HIP call (CPU only: no kernel is launched here)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8kv.h")

import fp8_kv_cache_reshape_amd as F


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8kv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_what_the_binding_binds():
    assert _declared() == sorted(F.SIGNATURES)


def test_library_exports_every_declared_symbol():
    out = subprocess.check_output(["nm", "-D", "--defined-only", F.LIBRARY_PATH], text=True)
    exported = set(re.findall(r"\bT (fp8kv_[a-z0-9_]+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name


def test_status_strings_and_version():
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert F.fp8kv_status_string(st) and F.fp8kv_status_string(st) != "unknown status"
    assert F.fp8kv_status_string(-99) == "unknown status"
    assert F.fp8kv_version() >= 100


FAKE = 1 << 20   # a 256-byte-aligned non-null address; never dereferenced by the host checks


def _write(**kw):
    a = dict(key=FAKE, value=FAKE, key_cache=FAKE, value_cache=FAKE, cache_dtype=F.FP8KV_E4M3,
             slot_mapping=FAKE, num_tokens=4, num_kv_heads=8, head_dim=128, block_size=16,
             num_blocks=10, k_scale=1.0, v_scale=1.0, stream=0)
    a.update(kw)
    return F.lib.fp8kv_cache_write(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(key=0), F.FP8KV_ERR_NULL), (dict(value_cache=0), F.FP8KV_ERR_NULL),
    (dict(slot_mapping=0), F.FP8KV_ERR_NULL),
    (dict(num_tokens=-1), F.FP8KV_ERR_SHAPE), (dict(num_kv_heads=0), F.FP8KV_ERR_SHAPE),
    (dict(num_blocks=-1), F.FP8KV_ERR_SHAPE), (dict(key=FAKE + 8), F.FP8KV_ERR_SHAPE),
    (dict(head_dim=96), F.FP8KV_ERR_UNSUPPORTED), (dict(block_size=32), F.FP8KV_ERR_UNSUPPORTED),
    (dict(cache_dtype=7), F.FP8KV_ERR_UNSUPPORTED),
    (dict(k_scale=0.0), F.FP8KV_ERR_SCALE), (dict(v_scale=-1.0), F.FP8KV_ERR_SCALE),
    (dict(k_scale=float("nan")), F.FP8KV_ERR_SCALE), (dict(v_scale=float("inf")), F.FP8KV_ERR_SCALE),
])
def test_cache_write_rejects(kw, status):
    assert _write(**kw) == status


def test_cache_write_accepts_edge_cases_without_launch():
    assert _write(num_tokens=0) == F.FP8KV_OK                       # nothing to do
    # bf16 caches ignore the scales, so a zero scale is not an error there: but this would
    # launch, so only check that the scale test is skipped by asking for zero tokens
    assert _write(num_tokens=0, cache_dtype=F.FP8KV_BF16, k_scale=0.0) == F.FP8KV_OK


def _write_ph(**kw):
    a = dict(key=FAKE, value=FAKE, key_cache=FAKE, value_cache=FAKE, cache_dtype=F.FP8KV_E4M3,
             slot_mapping=FAKE, num_tokens=4, num_kv_heads=8, head_dim=128, block_size=16,
             num_blocks=10, k_scales=FAKE, v_scales=FAKE, stream=0)
    a.update(kw)
    return F.lib.fp8kv_cache_write_per_head(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(k_scales=0), F.FP8KV_ERR_NULL), (dict(v_scales=0), F.FP8KV_ERR_NULL),
    (dict(k_scales=FAKE + 2), F.FP8KV_ERR_SHAPE), (dict(v_scales=FAKE + 1), F.FP8KV_ERR_SHAPE),
    (dict(key=0), F.FP8KV_ERR_NULL), (dict(head_dim=96), F.FP8KV_ERR_UNSUPPORTED),
    # the arrays are checked with the other scale arguments, before the zero-token exit
    (dict(k_scales=0, num_tokens=0), F.FP8KV_ERR_NULL),
])
def test_cache_write_per_head_rejects(kw, status):
    assert _write_ph(**kw) == status


def test_cache_write_per_head_edge_cases_without_launch():
    assert _write_ph(num_tokens=0) == F.FP8KV_OK
    # bf16 caches ignore the scale arrays, which may then be NULL
    assert _write_ph(num_tokens=0, cache_dtype=F.FP8KV_BF16, k_scales=0, v_scales=0) == F.FP8KV_OK


def _decode(**kw):
    a = dict(out=FAKE, out_dtype=F.FP8KV_BF16, query=FAKE, key_cache=FAKE, value_cache=FAKE,
             cache_dtype=F.FP8KV_E4M3, block_tables=FAKE, max_blocks_per_seq=64, context_lens=FAKE,
             max_context_len=1024, num_seqs=2, num_q_heads=32, num_kv_heads=8, head_dim=128,
             block_size=16, num_blocks=200, k_scale=1.0, v_scale=1.0, sliding_window=0,
             num_splits=4, counters=0, counters_bytes=0, workspace=FAKE, workspace_bytes=0,
             stream=0)
    a.update(kw)
    return F.lib.fp8kv_paged_decode(*a.values())


def _step(**kw):
    """fp8kv_decode_step with the same arguments as _decode plus the token rows."""
    a = dict(out=FAKE, out_dtype=F.FP8KV_BF16, query=FAKE, key_new=FAKE, value_new=FAKE,
             key_cache=FAKE, value_cache=FAKE, cache_dtype=F.FP8KV_E4M3, block_tables=FAKE,
             max_blocks_per_seq=64, context_lens=FAKE, max_context_len=1024, num_seqs=2,
             num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=200,
             k_scale=1.0, v_scale=1.0, sliding_window=0, num_splits=4, counters=FAKE,
             counters_bytes=1 << 20, workspace=FAKE, workspace_bytes=1 << 30, stream=0)
    a.update(kw)
    return F.lib.fp8kv_decode_step(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(query=0), F.FP8KV_ERR_NULL), (dict(block_tables=0), F.FP8KV_ERR_NULL),
    (dict(context_lens=0), F.FP8KV_ERR_NULL), (dict(key_cache=0), F.FP8KV_ERR_NULL),
    (dict(num_seqs=-1), F.FP8KV_ERR_SHAPE), (dict(num_q_heads=30), F.FP8KV_ERR_SHAPE),
    (dict(num_kv_heads=0), F.FP8KV_ERR_SHAPE), (dict(max_context_len=-5), F.FP8KV_ERR_SHAPE),
    (dict(sliding_window=-1), F.FP8KV_ERR_SHAPE), (dict(num_splits=-2), F.FP8KV_ERR_SHAPE),
    (dict(max_blocks_per_seq=0), F.FP8KV_ERR_SHAPE), (dict(query=FAKE + 4), F.FP8KV_ERR_SHAPE),
    (dict(num_blocks=0), F.FP8KV_ERR_SHAPE),
    (dict(head_dim=80), F.FP8KV_ERR_UNSUPPORTED), (dict(block_size=8), F.FP8KV_ERR_UNSUPPORTED),
    (dict(num_q_heads=136, num_kv_heads=4), F.FP8KV_ERR_UNSUPPORTED),   # g = 34 > 16
    (dict(cache_dtype=2), F.FP8KV_ERR_UNSUPPORTED), (dict(out_dtype=0), F.FP8KV_ERR_UNSUPPORTED),
    (dict(num_splits=5000), F.FP8KV_ERR_UNSUPPORTED),
    (dict(k_scale=0.0), F.FP8KV_ERR_SCALE), (dict(v_scale=float("nan")), F.FP8KV_ERR_SCALE),
    (dict(workspace=0), F.FP8KV_ERR_WORKSPACE), (dict(workspace_bytes=100), F.FP8KV_ERR_WORKSPACE),
    (dict(workspace=FAKE + 16, workspace_bytes=1 << 30), F.FP8KV_ERR_WORKSPACE),
    # optional counters: checked when given (2 sequences x 8 kv heads need 16 records)
    (dict(workspace_bytes=1 << 30, counters=FAKE, counters_bytes=16 * 1280 - 1), F.FP8KV_ERR_WORKSPACE),
    (dict(workspace_bytes=1 << 30, counters=FAKE + 64, counters_bytes=1 << 20), F.FP8KV_ERR_WORKSPACE),
])
def test_decode_rejects(kw, status):
    assert _decode(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(key_new=0), F.FP8KV_ERR_NULL), (dict(value_new=0), F.FP8KV_ERR_NULL),
    (dict(key_new=FAKE + 2), F.FP8KV_ERR_SHAPE),
    # several splits: the counter buffer is required, large enough and 256-byte aligned
    (dict(counters=0), F.FP8KV_ERR_WORKSPACE),
    (dict(counters_bytes=16 * 1280 - 4), F.FP8KV_ERR_WORKSPACE),
    (dict(counters=FAKE + 128), F.FP8KV_ERR_WORKSPACE),
    (dict(workspace=0), F.FP8KV_ERR_WORKSPACE), (dict(out_dtype=0), F.FP8KV_ERR_UNSUPPORTED),
])
def test_decode_step_rejects(kw, status):
    assert _step(**kw) == status


def test_decode_step_counters_optional_for_one_split():
    # one split (33 blocks or fewer): no counters and no workspace are needed; with no
    # sequences nothing is launched
    assert _step(num_seqs=0, counters=0, workspace=0) == F.FP8KV_OK


def test_counter_buffer_size():
    assert F.fp8kv_decode_counters_size(8, 8) == 64 * 1280
    assert F.fp8kv_decode_counters_size(0, 8) == 0
    assert F.lib.fp8kv_decode_counters_size(-1, 8) == 0
    assert F.lib.fp8kv_decode_counters_size(4, 0) == 0


def test_error_word_setter():
    assert F.lib.fp8kv_set_error_word(FAKE + 2) == F.FP8KV_ERR_SHAPE
    assert F.lib.fp8kv_set_error_word(FAKE + 4) == F.FP8KV_OK
    assert F.lib.fp8kv_set_error_word(0) == F.FP8KV_OK


def _decode_ph(step=False, **kw):
    a = dict(out=FAKE, out_dtype=F.FP8KV_BF16, query=FAKE, key_cache=FAKE, value_cache=FAKE,
             cache_dtype=F.FP8KV_E4M3, block_tables=FAKE, max_blocks_per_seq=64, context_lens=FAKE,
             max_context_len=1024, num_seqs=2, num_q_heads=32, num_kv_heads=8, head_dim=128,
             block_size=16, num_blocks=200, k_scales=FAKE, v_scales=FAKE, sliding_window=0,
             num_splits=4, counters=FAKE, counters_bytes=1 << 20, workspace=FAKE,
             workspace_bytes=0, stream=0)
    a.update(kw)
    if step:
        v = list(a.values())
        return F.lib.fp8kv_decode_step_per_head(*v[:3], FAKE, FAKE, *v[3:])
    return F.lib.fp8kv_paged_decode_per_head(*a.values())


@pytest.mark.parametrize("step", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(k_scales=0), F.FP8KV_ERR_NULL), (dict(v_scales=0), F.FP8KV_ERR_NULL),
    (dict(k_scales=FAKE + 2), F.FP8KV_ERR_SHAPE), (dict(v_scales=FAKE + 3), F.FP8KV_ERR_SHAPE),
    (dict(query=0), F.FP8KV_ERR_NULL), (dict(num_q_heads=30), F.FP8KV_ERR_SHAPE),
    (dict(workspace=0), F.FP8KV_ERR_WORKSPACE), (dict(out_dtype=0), F.FP8KV_ERR_UNSUPPORTED),
])
def test_decode_per_head_rejects(kw, status, step):
    assert _decode_ph(step=step, **kw) == status


def test_decode_per_head_bf16_ignores_scale_arrays():
    # a bf16 cache needs no scales: NULL arrays pass validation (the workspace check follows)
    assert _decode_ph(cache_dtype=F.FP8KV_BF16, k_scales=0, v_scales=0, workspace=0) == \
        F.FP8KV_ERR_WORKSPACE
    assert _decode_ph(num_seqs=0, query=0, out=0, workspace=0) == F.FP8KV_OK


def test_decode_with_no_sequences_is_a_no_op():
    assert _decode(num_seqs=0, query=0, out=0, workspace=0) == F.FP8KV_OK


def test_split_planning():
    ns = F.fp8kv_paged_decode_num_splits
    assert ns(1, 8, 128, 16, 131072, 0, 0) * 8 >= 256        # B=1 long context: a workgroup per CU
    assert ns(1, 8, 128, 16, 131072, 0, 16) == 16            # requested count
    assert ns(8, 8, 64, 16, 20480, 128, 0) == 1              # 128-token window: one split
    assert ns(16, 1, 256, 16, 65536, 512, 0) == 1            # 512-token window (33 blocks): one split
    assert ns(1, 8, 128, 16, 528, 0, 0) == 1                 # 33 blocks of context: one split
    assert ns(1, 8, 128, 16, 529, 0, 0) > 1                  # 34 blocks: split
    assert ns(16, 1, 256, 16, 65536, 1024, 0) > 1            # 1024-token window (65 blocks)
    assert ns(8, 8, 64, 16, 20480, 0, 0) == 8                # head_dim 64: two workgroups per CU
    assert ns(4, 8, 128, 16, 0, 0, 0) == 1                   # empty contexts
    assert ns(1, 1, 256, 16, 65536, 0, 4) == 4
    assert ns(1, 8, 128, 16, 20, 0, 64) == 2                 # never more splits than blocks
    assert F.lib.fp8kv_paged_decode_num_splits(1, 8, 80, 16, 1024, 0, 0) == F.FP8KV_ERR_UNSUPPORTED
    with pytest.raises(F.Fp8kvError):
        ns(1, 8, 80, 16, 1024, 0, 0)
    ws = F.fp8kv_paged_decode_workspace_size
    s = ns(1, 8, 128, 16, 131072, 0, 0)
    rows = 1 * 32 * s
    assert ws(1, 32, 8, 128, 16, 131072, 0, 0) == (rows * 8 + 255) // 256 * 256 + rows * 128 * 4
    assert ws(1, 32, 8, 100, 16, 131072, 0, 0) == 0


def test_single_hip_runtime_in_process():
    """The library must bind to the HIP runtime torch loaded, not a second copy."""
    import subprocess, sys
    code = ("import fp8_kv_cache_reshape_amd\nimport torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(len(set(l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l)))\n")
    out = subprocess.check_output([sys.executable, "-c", code], cwd=ROOT, text=True)
    assert out.strip() == "1"


def _noalloc(**kw):
    a = dict(out=FAKE, out_dtype=F.FP8KV_BF16, query=FAKE, key_new=FAKE, value_new=FAKE,
             key_cache=FAKE, value_cache=FAKE, cache_dtype=F.FP8KV_E4M3, block_tables=FAKE,
             max_blocks_per_seq=1 << 14, context_lens=FAKE, max_context_len=4096, num_seqs=2,
             num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=1 << 20,
             k_scale=1.0, v_scale=1.0, sliding_window=0, num_splits=0, stream=0)
    a.update(kw)
    return F.lib.fp8kv_decode_step_noalloc(*a.values())


@pytest.mark.parametrize("kw,status", [
    # more (sequence, kv head) groups than the array has counter records for, in a call that
    # needs counters (two splits); a one-split call needs neither counters nor partials
    (dict(num_seqs=F.FP8KV_NOALLOC_MAX_GROUPS // 8 + 1, num_splits=2), F.FP8KV_ERR_SCRATCH),
    # 1024 splits x 32 heads x 130 floats of partials: more than the array's 13.5 MiB
    (dict(num_seqs=1, max_context_len=1 << 18, num_splits=1024), F.FP8KV_ERR_SCRATCH),
    # the step's own checks, before the array is touched
    (dict(head_dim=96), F.FP8KV_ERR_UNSUPPORTED), (dict(num_q_heads=30), F.FP8KV_ERR_SHAPE),
    (dict(k_scale=0.0), F.FP8KV_ERR_SCALE),
])
def test_decode_step_noalloc_rejects_on_the_host(kw, status):
    assert _noalloc(**kw) == status


def test_decode_step_noalloc_empty_batch_is_a_no_op():
    assert _noalloc(num_seqs=0, query=0, out=0) == F.FP8KV_OK


def test_split_passes_per_head_reject():
    f = F.lib.fp8kv_paged_decode_partial_per_head
    args = [FAKE, FAKE, FAKE, F.FP8KV_E4M3, FAKE, 64, FAKE, 1024, 2, 32, 8, 128, 16, 200, FAKE, 0, 4,
            FAKE, 1 << 30, 0]
    bad = list(args); bad[14] = 0
    assert f(*bad) == F.FP8KV_ERR_NULL                      # key scales missing
    bad = list(args); bad[14] = FAKE + 2
    assert f(*bad) == F.FP8KV_ERR_SHAPE                     # misaligned
    bad = list(args); bad[17] = FAKE + 16
    assert f(*bad) == F.FP8KV_ERR_WORKSPACE
    m = F.lib.fp8kv_paged_decode_merge_per_head
    margs = [FAKE, F.FP8KV_BF16, F.FP8KV_E4M3, FAKE, 1024, 64, 2, 32, 8, 128, 16, FAKE, 0, 4, FAKE,
             1 << 30, 0]
    bad = list(margs); bad[11] = 0
    assert m(*bad) == F.FP8KV_ERR_NULL                      # value scales missing
    bad = list(margs); bad[2] = 9
    assert m(*bad) == F.FP8KV_ERR_UNSUPPORTED
    bad = list(margs); bad[15] = 100
    assert m(*bad) == F.FP8KV_ERR_WORKSPACE
    bad = list(margs); bad[0] = 0
    assert m(*bad) == F.FP8KV_ERR_NULL


def _rot_ph(kind, **kw):
    """The per-head rotated calls with plausible arguments (fake device addresses)."""
    if kind == "write":
        a = dict(key=FAKE, value=FAKE, key_cache=FAKE, value_cache=FAKE, cache_dtype=F.FP8KV_E4M3,
                 slot_mapping=FAKE, num_tokens=4, num_kv_heads=8, head_dim=128, block_size=16,
                 num_blocks=10, k_scales=FAKE, v_scales=FAKE, stream=0)
        a.update(kw)
        return F.lib.fp8kv_cache_write_rotated_per_head(*a.values())
    a = dict(out=FAKE, out_dtype=F.FP8KV_BF16, query=FAKE, key_new=FAKE, value_new=FAKE,
             key_cache=FAKE, value_cache=FAKE, cache_dtype=F.FP8KV_E4M3, block_tables=FAKE,
             max_blocks_per_seq=64, context_lens=FAKE, max_context_len=1024, num_seqs=2,
             num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=200,
             k_scales=FAKE, v_scales=FAKE, sliding_window=0, num_splits=4, counters=FAKE,
             counters_bytes=1 << 20, workspace=FAKE, workspace_bytes=0, stream=0)
    a.update(kw)
    if kind == "step":
        return F.lib.fp8kv_decode_step_rotated_per_head(*a.values())
    for k in ("key_new", "value_new", "counters", "counters_bytes"):
        del a[k]
    return F.lib.fp8kv_paged_decode_rotated_per_head(*a.values())


@pytest.mark.parametrize("kind", ["write", "decode", "step"])
@pytest.mark.parametrize("kw,status", [
    (dict(k_scales=0), F.FP8KV_ERR_NULL), (dict(v_scales=0), F.FP8KV_ERR_NULL),
    (dict(k_scales=FAKE + 2), F.FP8KV_ERR_SHAPE), (dict(v_scales=FAKE + 1), F.FP8KV_ERR_SHAPE),
    (dict(cache_dtype=F.FP8KV_E5M2), F.FP8KV_ERR_UNSUPPORTED),
    (dict(head_dim=96), F.FP8KV_ERR_UNSUPPORTED),
])
def test_rotated_per_head_rejects(kind, kw, status):
    assert _rot_ph(kind, **kw) == status


def test_rotated_per_head_bf16_ignores_scale_arrays():
    assert _rot_ph("write", cache_dtype=F.FP8KV_BF16, k_scales=0, v_scales=0, num_tokens=0) == F.FP8KV_OK
    for kind in ("decode", "step"):
        assert _rot_ph(kind, cache_dtype=F.FP8KV_BF16, k_scales=0, v_scales=0, workspace=0) == \
            F.FP8KV_ERR_WORKSPACE
        assert _rot_ph(kind, num_seqs=0, query=0, out=0, workspace=0) == F.FP8KV_OK


def _prefill_rot(**kw):
    a = dict(out=FAKE, out_dtype=F.FP8KV_BF16, query=FAKE, query_start_loc=FAKE, key_cache=FAKE,
             value_cache=FAKE, cache_dtype=F.FP8KV_E4M3, block_tables=FAKE, max_blocks_per_seq=64,
             context_lens=FAKE, max_context_len=1024, num_seqs=2, max_query_len=64,
             num_query_tokens=100, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
             num_blocks=200, k_scale=1.0, v_scale=1.0, sliding_window=0, workspace=FAKE,
             workspace_bytes=0, stream=0)
    a.update(kw)
    return F.lib.fp8kv_paged_prefill_rotated(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=256), F.FP8KV_ERR_UNSUPPORTED), (dict(cache_dtype=F.FP8KV_E5M2), F.FP8KV_ERR_UNSUPPORTED),
    (dict(cache_dtype=F.FP8KV_INT8), F.FP8KV_ERR_UNSUPPORTED), (dict(num_query_tokens=-1), F.FP8KV_ERR_SHAPE),
    (dict(workspace=0), F.FP8KV_ERR_WORKSPACE), (dict(workspace=FAKE + 16, workspace_bytes=1 << 30), F.FP8KV_ERR_WORKSPACE),
    (dict(k_scale=0.0), F.FP8KV_ERR_SCALE), (dict(query=0), F.FP8KV_ERR_NULL),
    (dict(out_dtype=7), F.FP8KV_ERR_UNSUPPORTED), (dict(num_q_heads=30), F.FP8KV_ERR_SHAPE),
])
def test_prefill_rotated_rejects(kw, status):
    assert _prefill_rot(**kw) == status


def test_prefill_rotated_no_work_and_workspace_size():
    assert _prefill_rot(num_query_tokens=0) == F.FP8KV_OK
    assert _prefill_rot(num_seqs=0, query=0, out=0) == F.FP8KV_OK
    ws = F.fp8kv_paged_prefill_rotated_workspace_size
    assert ws(100, 32, 128) == 2 * 100 * 32 * 128 * 2 + 100 * 32 * 128 * 4
    assert ws(1, 1, 64) == 256 + 256 + 256
    assert ws(-1, 32, 128) == 0 and ws(10, 32, 96) == 0 and ws(10, 0, 128) == 0
