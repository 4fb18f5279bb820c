"""fp8 latent caches over the whole range of token scales and query magnitudes.

Both products of an fp8 cache run on fp16 MFMAs; the kernels bring each head's
query and each tile's probability-times-scale weights into fp16's range with
exact powers of two. These cases put the scales far outside the U[0.5, 2] of
the workloads (up to 2^40, down to 2^-60) and the queries at 2^+-24, on the
64-head producer/consumer kernel and on the general 16-head kernel.

With scales around s0 the cached values, and therefore the outputs, are of
size s0, while the softmax scale 1 / (24 s0) keeps the scores of unit size
(24 = sqrt(576)). The output bar (relative L2 <= 5e-3, max |O - O*| <= 1e-2)
is applied to O / s0, the output in the units of the values' own spread; the
LSE bar (1e-3) is applied as it is.
"""
import math
from dataclasses import replace

import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import oracle
import workloads as W
from gpu_helpers import TOL, compare, desc_for, need_gpu, run_all_shards, to_np

pytestmark = pytest.mark.gpu

LENS = [1, 33, 700, 5000, 12345]
SCALES = [4095.0, 8192.0, 65504.0, 2.0 ** 40, 2.0 ** -20, 2.0 ** -60]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _fp8_workload(hq, bs, s0, lens=LENS, seed=21):
    w = W.custom("mla", lens, num_q_heads=hq, num_kv_heads=1, qk_dim=576, v_dim=512,
                 block_size=bs, num_shards=8, kv_dtype="fp8",
                 softmax_scale=1.0 / (24.0 * s0), seed=seed)
    w.kv_scale = (w.kv_scale * np.float32(s0)).astype(np.float32)
    return w


def _scaled_query(w, k):
    """The workload's bf16 queries times 2^k (exact), with the softmax scale
    times 2^-k, so the scores are unchanged."""
    q = (w.q.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** k)
    w.q = W.encode_bf16(q)
    w.spec = replace(w.spec, softmax_scale=w.spec.softmax_scale * 2.0 ** -k)
    return w


@pytest.mark.parametrize("hq", [64, 16])
@pytest.mark.parametrize("s0", SCALES, ids=lambda s: f"s2^{math.log2(s):.1f}")
def test_token_scales_far_from_one(hq, s0):
    w = _fp8_workload(hq, 64, s0)
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse, _, _ = run_all_shards(w)
    compare(o / s0, lse, o_ref / s0, lse_ref, **TOL["fp8"], label=f"sigma ~ {s0:g}, {hq} heads")


@pytest.mark.parametrize("hq", [64, 16])
@pytest.mark.parametrize("k", [24, -24])
def test_query_magnitudes(hq, k):
    w = _scaled_query(_fp8_workload(hq, 64, 1.0), k)
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse, _, _ = run_all_shards(w)
    compare(o, lse, o_ref, lse_ref, **TOL["fp8"], label=f"query x 2^{k}, {hq} heads")


def test_sharp_softmax_with_large_scales():
    """Scores spread over tens of log2 units (many reference raises) with
    scales around 2^20 that vary 4x between tokens."""
    s0 = 2.0 ** 20
    w = _fp8_workload(64, 64, s0, lens=[3000, 777, 4096])
    w.spec = replace(w.spec, softmax_scale=0.5 / s0)
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse, _, _ = run_all_shards(w)
    compare(o / s0, lse, o_ref / s0, lse_ref, **TOL["fp8"], label="sharp softmax, sigma ~ 2^20")


def test_decode_after_appending_large_rows():
    """Rows of magnitude ~1e7 appended through dcp_kv_append get scales near
    2^15 (amax / 448); the next decode over them matches the oracle run on the
    oracle's own append of the same rows (the two caches are bit-identical)."""
    lens = [0, 31, 64, 700, 2047]
    # softmax scale 1 / (24 * 3e6): the new rows' scores are of unit size
    w = W.custom("mla", [x + 1 for x in lens], num_q_heads=64, num_kv_heads=1, qk_dim=576,
                 v_dim=512, block_size=64, num_shards=8, kv_dtype="fp8",
                 softmax_scale=1.0 / (24.0 * 3e6), seed=5)
    rng = np.random.default_rng(99)
    rows = (rng.standard_normal((len(lens), 576)) * 3e6).astype(np.float32)
    rows16 = W.encode_bf16(rows)
    pos = np.array(lens, dtype=np.int32)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    kd = torch.from_numpy(rows16.view(np.int16)).cuda().view(torch.bfloat16)
    dcp.kv_append(desc, torch.from_numpy(pos).cuda(), kd, None, dev.block_table, dev.k_cache,
                  None, dev.kv_scale)
    k2, _, s2 = oracle.kv_append(w.k_cache, None, w.kv_scale, w.block_table, pos, rows16, None,
                                 kv_dtype="fp8", block_size=64)
    torch.cuda.synchronize()
    assert np.array_equal(dev.k_cache.cpu().numpy(), k2)
    assert np.array_equal(dev.kv_scale.cpu().numpy().view(np.uint32), s2.view(np.uint32))
    assert float(s2.max()) > 8192.0  # the appended rows' scales
    w.k_cache, w.kv_scale = k2, s2
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse = dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                   dev.block_table, dev.seq_lens)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(to_np(o)))
    # The appended tokens' values are ~3e6; the others' are ~1.
    compare(o / 3e6, lse, o_ref / 3e6, lse_ref, **TOL["fp8"], label="decode after large append")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_blocks_larger_than_the_tile_table_reach(dtype):
    """16384-token blocks (beyond what the 64-head kernel's tile table encodes)
    are served by the general kernel."""
    w = W.custom("mla", [20000, 40000, 16384, 1], num_q_heads=64, num_kv_heads=1, qk_dim=576,
                 v_dim=512, block_size=16384, num_shards=2, kv_dtype=dtype, seed=8)
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse, _, _ = run_all_shards(w)
    compare(o, lse, o_ref, lse_ref, **TOL[dtype], label=f"block size 16384, {dtype}")
