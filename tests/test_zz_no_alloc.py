"""fp8kv_decode_step_noalloc (counters and split partials in the library's fixed device array)
against fp8kv_decode_step with caller buffers, through the C-ABI: two calls in a row, the
second with a smaller input, both against the caller-buffer step's output and the oracle, and
the array's limits rejected on the host."""
import numpy as np
import pytest
import torch

import fp8_kv_cache_reshape_amd as F
import synthetic as syn
from gpu_util import (E4M3, DeviceInputs, assert_close, dev_caches, gpu_decode_step, gpu_write,
                      oracle_decode, oracle_write, say, step_rows_by_seq, to_host_bits, u16_dev)

pytestmark = pytest.mark.gpu


def _noalloc_step(w, layer, kc, vc, num_splits, dev):
    B, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    kn, vn = step_rows_by_seq(w, layer)
    # device copies held in variables: a temporary's memory could be reused before the launch
    kd, vd = u16_dev(kn), u16_dev(vn)
    out = torch.empty(B * Hq * D, dtype=torch.float32, device="cuda")
    st = F.lib.fp8kv_decode_step_noalloc(
        out.data_ptr(), F.FP8KV_F32, dev.q.data_ptr(), kd.data_ptr(), vd.data_ptr(),
        kc.data_ptr(), vc.data_ptr(), E4M3, dev.bt.data_ptr(), w.max_blocks_per_seq, dev.cl.data_ptr(),
        w.max_context_len, B, Hq, Hkv, D, 16, w.num_blocks, layer.k_scale, layer.v_scale,
        layer.sliding_window, num_splits, int(torch.cuda.current_stream().cuda_stream))
    assert st == F.FP8KV_OK, F.fp8kv_status_string(st)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64).reshape(B, Hq, D)


def _case(w, num_splits):
    """The same step through both entry points on two copies of the cache: identical cache
    bytes, outputs equal (bit for bit with a fixed split count, within the run-to-run bound of
    the automatic plan otherwise) and within the f32-output tolerance of the oracle."""
    layer = w.layers[0]
    dev = DeviceInputs(w)
    kc, vc = dev_caches(w, E4M3)
    gpu_write(w, layer, kc, vc, rows=w.prefix_token_rows())
    kc2, vc2 = kc.clone(), vc.clone()
    ref_step, _ = gpu_decode_step(w, layer, kc, vc, out_f32=True, num_splits=num_splits, dev=dev)
    got = _noalloc_step(w, layer, kc2, vc2, num_splits, dev)
    assert torch.equal(kc, kc2) and torch.equal(vc, vc2), "cache bytes differ between the entry points"
    okc, ovc = oracle_write(w, layer)
    assert np.array_equal(to_host_bits(kc2), okc) and np.array_equal(to_host_bits(vc2), ovc)
    if num_splits > 0:
        assert np.array_equal(got, ref_step), "fixed split count: outputs differ between the entry points"
    else:
        vmax = 448.0 * layer.v_scale        # every decoded value is at most 448 * v_scale
        bound = 2 * (2.0 ** -18 + (256 + 64) * 2.0 ** -24) * vmax
        assert np.abs(got - ref_step).max() <= bound
    assert_close(got, oracle_decode(w, layer, okc, ovc), atol=2e-4, rtol=2e-3, what=f"noalloc {w.name}")


def _mk(lens, cid, Hq=32, Hkv=8, D=128, window=0):
    return syn.make_workload(f"noalloc-{Hq}-{Hkv}-{D}-{len(lens)}", cid, num_q_heads=Hq,
                             num_kv_heads=Hkv, head_dim=D, context_lens=lens, outlier_frac=0.01,
                             layers=(("l0", window, syn.E4M3),))


@pytest.mark.parametrize("num_splits", [0, 7])
def test_noalloc_step_twice_second_smaller(num_splits):
    """Two calls in a row on the shared array: 6 sequences, then 2 shorter ones (fewer
    counter records and fewer partials than the first call left behind)."""
    first = _mk([9000, 700, 2049, 16, 4100, 33], cid=400)
    second = _mk([1500, 530], cid=401)
    for w in (first, second):
        say(f"noalloc step {w.name} lens={w.context_lens.tolist()} splits={num_splits}")
        _case(w, num_splits)


def test_noalloc_step_other_shapes():
    for w in (_mk([3000, 17, 600], cid=402, Hq=64, Hkv=8, D=64, window=128),
              _mk([5000, 800], cid=403, Hq=8, Hkv=1, D=256)):
        say(f"noalloc step {w.name}")
        _case(w, 0)


def test_noalloc_limits_rejected_on_the_host():
    """More groups or partials than the array holds: FP8KV_ERR_SCRATCH before any launch."""
    fake = 1 << 20
    call = lambda B, Hkv, L, ns: F.lib.fp8kv_decode_step_noalloc(
        fake, F.FP8KV_BF16, fake, fake, fake, fake, fake, E4M3, fake, 1 << 14, fake, L, B, Hkv * 4,
        Hkv, 128, 16, 1 << 20, 1.0, 1.0, 0, ns, 0)
    assert call(F.FP8KV_NOALLOC_MAX_GROUPS // 8 + 1, 8, 4096, 2) == F.FP8KV_ERR_SCRATCH
    # 1024 splits x 32 heads x 130 floats: 16.6 MiB of partials
    assert call(1, 8, 1 << 18, 1024) == F.FP8KV_ERR_SCRATCH
