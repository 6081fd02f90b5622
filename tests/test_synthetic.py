"""Seeded synthetic workloads: determinism, bf16 rounding, and paged layout validity (CPU)."""
import numpy as np
import torch

import synthetic as syn


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(100000) * 1e30).astype(np.float32),
        (rng.standard_normal(100000) * 1e-38).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38], np.float32),
        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32),  # exact ties
    ])
    ours = syn.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    fin = np.isfinite(x) | np.isinf(x)
    assert np.array_equal(ours[fin], ref[fin])
    nan = syn.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(syn.bf16_bits_to_f32(nan)).all()


def test_workload_is_deterministic_and_well_formed():
    a = syn.make_workload("t", 9, num_q_heads=8, num_kv_heads=2, head_dim=64, num_seqs=3,
                          len_range=(5, 70), outlier_frac=0.01, needle=True)
    b = syn.make_workload("t", 9, num_q_heads=8, num_kv_heads=2, head_dim=64, num_seqs=3,
                          len_range=(5, 70), outlier_frac=0.01, needle=True)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.layers[0].k, b.layers[0].k)
    assert np.array_equal(a.block_tables, b.block_tables)
    bs = a.block_size
    used = set()
    for s, L in enumerate(a.context_lens):
        n = (int(L) + bs - 1) // bs
        blocks = a.block_tables[s, :n].tolist()
        assert not (used & set(blocks))
        used |= set(blocks)
        rows = np.arange(a.seq_offsets[s], a.seq_offsets[s + 1])
        j = np.arange(int(L))
        assert np.array_equal(a.slot_mapping[rows], a.block_tables[s, j // bs].astype(np.int64) * bs + j % bs)
    assert all(0 <= x < a.num_blocks for x in a.block_tables.reshape(-1))
    assert len(used) < a.num_blocks          # slack blocks exist and are never written
    assert a.slot_mapping.max() < a.num_blocks * bs
    # the step token rows are each sequence's last token
    assert np.array_equal(a.step_token_rows(), a.seq_offsets[1:] - 1)
    assert len(a.prefix_token_rows()) + len(a.step_token_rows()) == a.num_tokens


def test_amax_scale_and_outliers():
    w = syn.make_workload("t", 10, num_q_heads=4, num_kv_heads=2, head_dim=64,
                          context_lens=[300], outlier_frac=0.05, scale_mode="amax")
    L = w.layers[0]
    k = syn.bf16_bits_to_f32(L.k)
    assert L.k_scale == float(np.float32(np.abs(k).max()) / np.float32(448.0))
    col_std = k.reshape(300, -1).std(axis=0)
    n_out = int(round(0.05 * 2 * 64))
    assert (col_std > 4.0).sum() == n_out     # x8 channels stand out from N(0,1)
    u = syn.make_workload("t", 10, num_q_heads=4, num_kv_heads=2, head_dim=64,
                          context_lens=[300], scale_mode="uncal")
    assert u.layers[0].k_scale == 1.0 and u.layers[0].v_scale == 1.0


def test_needle_is_planted():
    w = syn.llama70b_needle(4096)
    n = w.needle
    L = w.layers[0]
    q0 = syn.bf16_bits_to_f32(w.q[0, 0]).astype(np.float64)
    key = syn.bf16_bits_to_f32(L.k[n["row"], 0]).astype(np.float64)
    assert abs(np.dot(key, q0) / np.linalg.norm(q0) - 4.0) < 0.05
    val = syn.bf16_bits_to_f32(L.v[n["row"], 0])
    assert val[n["channel"]] == 448.0 and np.count_nonzero(val) == 1
    assert L.v_scale == 1.0          # amax of V is the needle's 448
