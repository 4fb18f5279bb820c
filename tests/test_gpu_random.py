"""Seeded random shapes through the fused path and one shard's partial: block
sizes, shard counts, head counts, query tokens and ragged lengths (empty
sequences included) drawn from the supported ranges, each against the oracle."""
import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import oracle
import workloads as W
from gpu_helpers import TOL, compare, desc_for, need_gpu, run_all_shards

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _draw(i):
    rng = np.random.default_rng([2024, i])
    kind = "mla" if i % 3 else "gqa"
    d = int(rng.integers(1, 10))
    if kind == "mla":
        dtype = ["bf16", "fp8"][int(rng.integers(0, 2))]
        bs = int(rng.choice([1, 16, 32, 48, 64, 128]))
        hq = int(rng.choice([16, 32, 64, 128]))
        q_len = int(rng.choice([1, 1, 2, 4])) if hq <= 64 else 1
        if (q_len * hq) not in (16, 32) and (q_len * hq) % 64:
            q_len = 1
        hkv, dqk, dv = 1, 576, 512
    else:
        dtype = ["bf16", "f32"][int(rng.integers(0, 2))]
        bs = int(rng.choice([1, 5, 16, 32]))
        hkv = int(rng.choice([1, 2, 4, 8]))
        hq = hkv * int(rng.choice([1, 2, 4, 8, 16]))
        q_len = int(rng.choice([1, 1, 2, 3]))
        dqk = dv = int(rng.choice([64, 128]))
    batch = int(rng.integers(1, 7))
    lens = rng.integers(0, 1500, batch)
    lens[rng.random(batch) < 0.2] = 0
    lens[rng.random(batch) < 0.2] = rng.integers(1, 4)
    return (kind, dtype, bs, d, hq, hkv, dqk, dv, q_len, [int(x) for x in lens])


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    kind, dtype, bs, d, hq, hkv, dqk, dv, q_len, lens = case = _draw(i)
    print("case", case, flush=True)
    w = W.custom(kind, lens, num_q_heads=hq, num_kv_heads=hkv, qk_dim=dqk, v_dim=dv,
                 block_size=bs, num_shards=d, kv_dtype=dtype, seed=100 + i, q_len=q_len)
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse, dev, desc = run_all_shards(w)
    compare(o, lse, o_ref, lse_ref, **TOL[dtype], label=f"fused {case}")
    # One shard's partial through its local table (the multi-token form when q_len > 1).
    r = i % d
    lt, ll = dcp.block_remap(dev.block_table, dev.seq_lens, bs, d)
    op_ref, lp_ref = oracle.shard_partials(w, batch_indices=range(len(lens)))
    if q_len == 1:
        o_r, l_r = dcp.decode_partial(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                      lt[r].contiguous(), ll[r].contiguous())
    else:
        q_pos = (dev.seq_lens - q_len).to(torch.int32).contiguous()
        o_r, l_r = dcp.decode_partial_mtp(desc, r, q_pos, dev.q, dev.k_cache, dev.v_cache,
                                          dev.kv_scale, lt[r].contiguous(), ll[r].contiguous())
    compare(o_r, l_r, op_ref[r], lp_ref[r], **TOL[dtype], label=f"shard {r} {case}")
