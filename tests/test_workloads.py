"""Seeded input generator: shapes, statistics from the pages, determinism."""
import json
from pathlib import Path

import numpy as np

import workloads as W

GOLDEN = Path(__file__).parent / "golden"


def test_kv_bytes_model_matches_page_example():
    g = json.loads((GOLDEN / "kv_bytes.json").read_text())
    spec = W.Spec("x", "gqa", 1, g["num_kv_heads"], g["num_kv_heads"], g["head_dim"],
                  g["head_dim"], 16, 1, "bf16", 1, 1.0, 0)
    per_layer = spec.kv_bytes_per_token()
    assert per_layer == g["bytes_per_token_per_layer"]
    assert per_layer * g["layers"] == g["bytes_per_token_all_layers"]
    # The page rounds 819,200 B to "800KB" before multiplying; allow that 2.4 %.
    total_gb = per_layer * g["layers"] * g["seq_len_for_total"] / 1e9
    assert abs(total_gb - g["total_gb_approx"]) / g["total_gb_approx"] < 0.03
    per_gpu = total_gb / g["tp"]
    assert abs(per_gpu - g["per_gpu_gb_approx"]) / g["per_gpu_gb_approx"] < 0.03


def test_bimodal_lengths_match_trace_statistics():
    # Agentic trace statistics as the pages give them (A4): median ~67K,
    # 53 % above 64K, ~8 % above 128K, 3-4 % above 256K, 18 % below 8K, tail ~1M.
    for batch in (64, 128, 1024):
        lens = W.bimodal_lengths(batch, 3)
        assert abs((lens > 64 * 1024).mean() - 0.53) <= 1.0 / batch + 1e-9
        assert abs((lens > 128 * 1024).mean() - 0.08) <= 1.0 / batch + 1e-9
        assert abs((lens > 256 * 1024).mean() - 0.035) <= 1.0 / batch + 1e-9
        assert abs((lens < 8 * 1024).mean() - 0.18) <= 1.0 / batch + 1e-9
        assert 60 * 1024 < np.median(lens) < 72 * 1024
        assert lens.min() >= 1024 and lens.max() <= 1024 * 1024


def test_block_table_is_a_permutation():
    w = W.make(W.scaled(W.SPECS["mla_bf16_b64_bimodal"]))
    nb = (w.seq_lens + w.spec.block_size - 1) // w.spec.block_size
    ids = np.concatenate([w.block_table[b, :nb[b]] for b in range(w.spec.batch)])
    assert sorted(ids.tolist()) == list(range(w.num_blocks))
    for b in range(w.spec.batch):
        assert np.all(w.block_table[b, nb[b]:] == -1)
    assert w.k_cache.shape == (w.num_blocks, 64, 576) and w.k_cache.dtype == np.uint16


def test_deterministic_and_seed_sensitive():
    s = W.scaled(W.SPECS["mla_fp8_b128_bimodal"], 16, 256)
    a, b = W.make(s), W.make(s)
    assert np.array_equal(a.k_cache, b.k_cache) and np.array_equal(a.kv_scale, b.kv_scale)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.block_table, b.block_table)
    c = W.make(s, seed=99)
    assert not np.array_equal(a.q, c.q)
    assert a.kv_scale.min() >= 0.5 and a.kv_scale.max() <= 2.0


def test_gqa_shapes():
    w = W.make(W.scaled(W.SPECS["gqa_bf16_b32_L32k"]))
    assert w.k_cache.shape == (w.num_blocks, 16, 8, 128)
    assert w.v_cache.shape == w.k_cache.shape
    assert w.q.shape == (4, 64, 128)
    assert np.all(w.seq_lens == 512)
