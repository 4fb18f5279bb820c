"""Whole-batch parity at full size: every sequence of each workload, in the
launch configuration the benchmark times (one fused dcp_decode_all_shards
call), against the fp64 oracle's unsharded attention ("Efficient Decode
Context Parallelism with vLLM for Long Context Workloads", summary section:
the sharded partials merged by the LSE equation equal attention over the
whole sequence; "vLLM长序列推理优化：DCP切分KV Cache原理与实战", section 7, for
the fp8 cache with per-token scales).

Each case prints its error figures (run with -s to see them): the relative L2
error over the whole batch, the worst sequence's relative L2 error, the
largest absolute output error and the largest LSE error.
"""
from dataclasses import replace

import pytest
import torch

import decode_attention_sequence_amd as dcp
import oracle
import workloads as W
from gpu_helpers import TOL, compare, need_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# (workload, query tokens per sequence, query heads if not the workload's)
CASES = [("mla_bf16_b64_bimodal", 1, None), ("mla_bf16_b64_bimodal", 1, 16),
         ("mla_fp8_b128_bimodal", 1, None),
         ("mla_fp8_b128_bimodal", 2, None),
         ("gqa_bf16_b32_L32k", 1, None), ("mla_bf16_b8_L1m", 1, None)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("name,q_len,heads", CASES,
                         ids=[f"{n}-q{q}" + (f"-h{h}" if h else "") for n, q, h in CASES])
def test_every_sequence(name, q_len, heads):
    spec = replace(W.SPECS[name], q_len=q_len)
    if heads:
        spec = replace(spec, num_q_heads=heads)
    w = W.make(spec)
    dev = W.to_torch(w, "cuda")
    kind = dcp.KV_LATENT if spec.kind == "mla" else dcp.KV_SEPARATE
    desc = dcp.make_desc(kind, dev.q, dev.k_cache, dev.block_table, num_shards=spec.num_shards,
                         v_dim=spec.v_dim, softmax_scale=spec.softmax_scale,
                         max_seq_len=int(w.seq_lens.max()), q_len=q_len)
    o, lse = dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                   dev.block_table, dev.seq_lens)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_reference(w)
    stats = compare(o, lse, o_ref, lse_ref, **TOL[spec.kv_dtype], label=f"{name} q{q_len}")
    print(f"\nwhole batch {name} q_len={q_len} heads={spec.num_q_heads}: {spec.batch} sequences, "
          f"{int(w.seq_lens.sum())} tokens: rel L2 {stats['rel_l2']:.3e}, worst sequence rel L2 "
          f"{stats['worst_seq_rel_l2']:.3e}, max |dO| {stats['max_abs']:.3e}, "
          f"max |dLSE| {stats['lse_abs']:.3e}", flush=True)
    assert stats["worst_seq_rel_l2"] <= TOL[spec.kv_dtype]["rel_l2"]
