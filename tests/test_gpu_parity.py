"""HIP path vs the fp64 oracle on the workloads' shapes (small and scaled-down sizes).

Every comparison is element by element over the whole output, at sizes that
span several tiles, several shards per sequence and ragged last blocks.
"""
import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import oracle
import workloads as W
from gpu_helpers import TOL, compare, need_gpu, run_all_shards, run_per_shard, to_np

pytestmark = pytest.mark.gpu

SMALL = [
    W.SPECS["gqa_f32_b1_L256"],
    W.scaled(W.SPECS["gqa_bf16_b32_L32k"]),        # B 4, L 512, 64/8 heads, D 4
    W.scaled(W.SPECS["mla_bf16_b64_bimodal"]),     # B 8, ragged 32..2681 tokens, D 8
    W.scaled(W.SPECS["mla_fp8_b128_bimodal"]),     # B 16, ragged, fp8 + scales
    W.scaled(W.SPECS["mla_bf16_b8_L1m"], 8, 64),   # B 1, L 16384
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_all_shards_matches_oracle(spec):
    w = W.make(spec)
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse, _, _ = run_all_shards(w)
    compare(o, lse, o_ref, lse_ref, **TOL[spec.kv_dtype], label=spec.name)


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_per_shard_partials_and_merge(spec):
    w = W.make(spec)
    op_ref, lp_ref = oracle.shard_partials(w)
    op, lp, _, _ = run_per_shard(w)
    for r in range(spec.num_shards):
        compare(op[r], lp[r], op_ref[r], lp_ref[r], **TOL[spec.kv_dtype], label=f"shard {r}")
    # dcp_lse_merge over the D shard partials reproduces unsharded attention.
    o, lse = dcp.lse_merge(op, lp)
    o_ref, lse_ref = oracle.decode_reference(w)
    compare(o, lse, o_ref, lse_ref, **TOL[spec.kv_dtype], label="merged shards")


@pytest.mark.parametrize("num_shards", [1, 2, 3, 5, 8, 13])
def test_any_shard_count_gives_unsharded_result(num_shards):
    spec = W.scaled(W.SPECS["mla_bf16_b64_bimodal"], 16, 128)
    w = W.make(spec)
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse, _, _ = run_all_shards(w, num_shards=num_shards)
    compare(o, lse, o_ref, lse_ref, **TOL["bf16"], label=f"D={num_shards}")
    op, lp, _, _ = run_per_shard(w, num_shards=num_shards)
    opr, lpr = oracle.shard_partials(w, num_shards)
    for r in range(num_shards):
        compare(op[r], lp[r], opr[r], lpr[r], **TOL["bf16"], label=f"D={num_shards} r={r}")


@pytest.mark.parametrize("spec", SMALL[1:4], ids=lambda s: s.name)
def test_contiguous_ownership_partials_and_merge(spec):
    """Contiguous runs of blocks per shard: other partials, the same merged result."""
    w = W.make(spec)
    op_ref, lp_ref = oracle.shard_partials(w, ownership="contiguous")
    op, lp, _, _ = run_per_shard(w, ownership="contiguous")
    for r in range(spec.num_shards):
        compare(op[r], lp[r], op_ref[r], lp_ref[r], **TOL[spec.kv_dtype], label=f"shard {r}")
    o, lse = dcp.lse_merge(op, lp)
    o_ref, lse_ref = oracle.decode_reference(w)
    compare(o, lse, o_ref, lse_ref, **TOL[spec.kv_dtype], label="merged contiguous shards")


def test_bf16_output():
    spec = W.scaled(W.SPECS["mla_bf16_b64_bimodal"], 16, 64)
    w = W.make(spec)
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse, _, _ = run_all_shards(w, out_dtype=dcp.BF16)
    assert o.dtype == torch.bfloat16
    # bf16 rounding of the output adds at most 2^-9 relative per element.
    compare(o, lse, o_ref, lse_ref, rel_l2=6e-3, max_abs=1.5e-2, lse_abs=1e-3, label="bf16 out")


@pytest.mark.parametrize("spec", SMALL[1:3], ids=lambda s: s.name)
def test_deterministic(spec):
    w = W.make(spec)
    o1, l1, dev, desc = run_all_shards(w)
    o2, l2 = dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                   dev.block_table, dev.seq_lens)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_shard_permutation_and_empty_shard_on_gpu():
    spec = W.scaled(W.SPECS["mla_bf16_b64_bimodal"], 16, 64)
    w = W.make(spec)
    op, lp, _, _ = run_per_shard(w)
    o, l = dcp.lse_merge(op, lp)
    perm = torch.randperm(op.shape[0], generator=torch.Generator().manual_seed(0))
    o2, l2 = dcp.lse_merge(op[perm].contiguous(), lp[perm].contiguous())
    assert np.allclose(to_np(o2), to_np(o), rtol=1e-6, atol=1e-6)
    assert np.allclose(to_np(l2), to_np(l), rtol=1e-6, atol=1e-6)
    # An extra empty shard (LSE = -inf, output never read) changes nothing, bit for bit.
    junk = torch.full_like(op[:1], float("nan"))
    o3, l3 = dcp.lse_merge(torch.cat([op, junk]), torch.cat([lp, torch.full_like(lp[:1], -np.inf)]))
    torch.cuda.synchronize()
    assert torch.equal(o3, o) and torch.equal(l3, l)
