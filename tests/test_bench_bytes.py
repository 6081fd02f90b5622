"""The benchmark's byte and intensity formulas against the pages' worked numbers (CPU)."""
import os

import numpy as np
import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            parts = line.split()
            vals[parts[0]] = [float(x) for x in parts[1:]]
    return vals


def test_bytes_per_token_matches_worked_capacity_example():
    g = {k: v[0] for k, v in _golden("capacity_worked_example.txt").items()}
    L, H, D = int(g["num_layers"]), int(g["num_kv_heads"]), int(g["head_dim"])
    assert bench.kv_bytes_per_token(L, H, D, 1) == g["elements_per_token"] == g["bytes_per_token_fp8"]
    assert bench.kv_bytes_per_token(L, H, D, 2) == g["bytes_per_token_bf16"]
    tok = int(g["sequence_tokens"])
    assert round(bench.kv_bytes_per_token(L, H, D, 2) * tok / 1e9, 2) == g["gb_per_sequence_bf16"]
    assert round(bench.kv_bytes_per_token(L, H, D, 1) * tok / 1e9, 2) == g["gb_per_sequence_fp8"]


def test_arithmetic_intensity_is_g_then_2g():
    rows = _golden("arithmetic_intensity.txt")
    for line in open(os.path.join(GOLDEN, "arithmetic_intensity.txt")):
        if line.strip() and not line.startswith("#"):
            g, bf16, fp8 = (float(x) for x in line.split())
            assert bench.arithmetic_intensity(int(g), 2) == bf16
            assert bench.arithmetic_intensity(int(g), 1) == fp8


def test_algorithmic_bytes_per_step():
    # one sequence of 131072 tokens at the 8B shape: 2 * L * Hkv * d fp8 bytes of K and V
    b = bench.algorithmic_bytes([131072], 32, 8, 128, 1)
    assert b["pass1"] == 2 * 131072 * 8 * 128 + 4 * 8192 + 2 * 32 * 128 + 4
    assert b["pass2"] == 2 * 32 * 128 + 4
    assert b["flops"] == 4 * 32 * 128 * 131072
    # the pages' 2x: bf16 KV doubles the dominant term
    b2 = bench.algorithmic_bytes([131072], 32, 8, 128, 2)
    assert b2["pass1"] - b["pass1"] == 2 * 131072 * 8 * 128
    # a window only charges the attended positions and the blocks they touch
    w = bench.algorithmic_bytes([1000], 64, 8, 64, 1, window=128)
    assert w["pass1"] == 2 * 128 * 8 * 64 + 4 * (63 - 54) + 2 * 64 * 64 + 4


def test_gpus_above_one_exits():
    assert bench.main(["--gpus", "2"]) == 2


def test_cpu_baseline_with_one_kv_head():
    """The oracle sample takes at most the workload's kv heads (the tiny shape has one)."""
    import synthetic as syn
    w = syn.tiny()
    r, ref = bench.cpu_baseline(w, w.layers[0])
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0
    assert "query heads 0..3 (KV heads 0..0 of 1)" in r["sample"]
    assert r["multi_thread"]["value"] > 0
    # the whole step's oracle output, which the bench compares with the last timed step
    assert ref.shape == (w.num_seqs, w.num_q_heads, w.head_dim) and np.all(np.isfinite(ref))
