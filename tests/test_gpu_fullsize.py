"""HIP path at the workloads' full sizes, in the launch configuration the
benchmark times (one fused dcp_decode_all_shards call with a reused
workspace), checked against the fp64 oracle on sampled sequences: the
shortest, the median and the longest. The oracle computes each sampled
sequence on its own, so the sample costs seconds even at a million tokens.

Every output row is also checked for properties that hold at any size: all
values finite, LSE finite exactly for non-empty sequences, and each output
row a convex combination of value rows (bounded by the largest cached
magnitude).
"""
import gc

import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import oracle
import workloads as W
from gpu_helpers import TOL, compare, need_gpu, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

FULL = ["gqa_bf16_b32_L32k", "mla_bf16_b64_bimodal", "mla_fp8_b128_bimodal", "mla_bf16_b8_L1m"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _value_bound(spec, dev):
    """Largest magnitude of any cached value (an output row is a convex
    combination of value rows, so no output can exceed it)."""
    v = dev.v_cache if spec.kind == "gqa" else dev.k_cache[..., : spec.v_dim]
    if spec.kv_dtype == "fp8":
        cmax = int((v & 0x7F).max())
        vmax = float(torch.tensor([cmax], dtype=torch.uint8).view(torch.float8_e4m3fn).float())
        return vmax * float(dev.kv_scale.max())
    return float(v.abs().max().float())


def _sample(lens):
    order = np.argsort(lens, kind="stable")
    picks = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    return sorted(set(picks))


# (workload, query tokens per sequence): single-token decode at every size,
# and multi-token decode as `bench.py --q-len 2` times it.
CASES = [(n, 1) for n in FULL] + [("mla_bf16_b64_bimodal", 2), ("gqa_bf16_b32_L32k", 2)]


@pytest.mark.parametrize("name,q_len", CASES, ids=[f"{n}-q{q}" for n, q in CASES])
def test_full_size_sampled_rows(name, q_len):
    from dataclasses import replace

    spec = replace(W.SPECS[name], q_len=q_len)
    w = W.make(spec)
    dev = W.to_torch(w, "cuda")
    kind = dcp.KV_LATENT if spec.kind == "mla" else dcp.KV_SEPARATE
    desc = dcp.make_desc(kind, dev.q, dev.k_cache, dev.block_table, num_shards=spec.num_shards,
                         v_dim=spec.v_dim, softmax_scale=spec.softmax_scale,
                         max_seq_len=int(w.seq_lens.max()), q_len=q_len)
    ws = dcp.alloc_workspace(desc, "cuda")
    rows_per_seq = q_len * spec.num_q_heads
    out = torch.empty((spec.batch, rows_per_seq, spec.v_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((spec.batch, rows_per_seq), dtype=torch.float32, device="cuda")
    for _ in range(2):  # the second call reuses the workspace as the benchmark does
        dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                              dev.block_table, dev.seq_lens, workspace=ws, out=out, lse_out=lse)
    torch.cuda.synchronize()
    o_np, lse_np = to_np(out), to_np(lse)

    # Properties of every row.
    assert np.all(np.isfinite(o_np)), name
    nonempty = w.seq_lens > 0
    assert np.all(np.isfinite(lse_np[nonempty])), name
    bound = _value_bound(spec, dev)
    assert np.abs(o_np).max() <= bound * (1 + 1e-3), name

    # Element-wise parity on the sampled sequences.
    rows = _sample(w.seq_lens)
    o_ref, lse_ref = oracle.decode_reference(w, batch_indices=rows)
    stats = compare(out, lse, o_ref, lse_ref, rows=rows, **TOL[spec.kv_dtype], label=name)
    print(f"{name}: rows {rows} lengths {[int(w.seq_lens[r]) for r in rows]} {stats}", flush=True)
    del dev, ws, out, lse, w
    gc.collect()
    torch.cuda.empty_cache()
