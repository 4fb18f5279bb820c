"""Token-level interleave ownership on the GPU (position t on shard t % D,
"vLLM长序列推理优化：DCP切分KV Cache原理与实战", section 2.2): every shard's
partial from dcp_decode_partial_token equals the oracle's partial over the
same positions, and merging the D partials gives the unsharded attention --
the merge does not depend on which shard owns which token."""
import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import oracle
import workloads as W
from gpu_helpers import TOL, compare, desc_for, need_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # kind, kv dtype, block size, shards, Hq, Hkv, qk_dim
    ("mla", "bf16", 64, 8, 64, 1, 576),    # 8 tokens of a shard per block: general kernel
    ("mla", "bf16", 256, 8, 64, 1, 576),   # 32 per block: the 64-head kernel
    ("mla", "fp8", 64, 4, 64, 1, 576),     # strided token scales
    ("mla", "fp8", 128, 4, 64, 1, 576),
    ("mla", "bf16", 16, 4, 16, 1, 576),
    ("gqa", "bf16", 16, 4, 64, 8, 128),
    ("gqa", "bf16", 12, 3, 12, 4, 64),
    ("gqa", "f32", 16, 2, 4, 1, 64),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _lens(bs, d):
    return [0, 1, d - 1, d, d + 1, bs - 1, bs, bs + 1, 3 * bs + 5, 1000, 4097]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_token_partials_and_merge(case):
    kind, dtype, bs, d, hq, hkv, dim = case
    w = W.custom(kind, _lens(bs, d), num_q_heads=hq, num_kv_heads=hkv, qk_dim=dim,
                 v_dim=512 if kind == "mla" else dim, block_size=bs, num_shards=d,
                 kv_dtype=dtype, seed=17)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    ws = dcp.alloc_workspace(desc, dev.q.device)
    parts, lses = [], []
    for r in range(d):
        o, l = dcp.decode_partial_token(desc, r, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                        dev.block_table, dev.seq_lens, workspace=ws)
        parts.append(o.clone())
        lses.append(l.clone())
    torch.cuda.synchronize()
    op_ref, lp_ref = oracle.shard_partials(w, ownership="token")
    for r in range(d):
        compare(parts[r], lses[r], op_ref[r], lp_ref[r], **TOL[dtype], label=f"token shard {r}")
    o, lse = dcp.lse_merge(torch.stack(parts), torch.stack(lses))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_reference(w)
    compare(o, lse, o_ref, lse_ref, **TOL[dtype], label="merged token shards")


def test_token_shards_at_full_size():
    """One rank's share of the batch-64 absorbed-MLA workload (D = 8) under
    token-level interleave, checked on three sampled sequences (shortest,
    median, longest), and the merged result of all eight shards on the same."""
    spec = W.SPECS["mla_bf16_b64_bimodal"]
    w = W.make(spec)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    ws = dcp.alloc_workspace(desc, dev.q.device)
    order = np.argsort(w.seq_lens, kind="stable")
    rows = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    d = spec.num_shards
    parts = torch.empty((d, spec.batch, spec.num_q_heads, spec.v_dim), device="cuda")
    lses = torch.empty((d, spec.batch, spec.num_q_heads), device="cuda")
    for r in range(d):
        dcp.decode_partial_token(desc, r, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                 dev.block_table, dev.seq_lens, workspace=ws, o_partial=parts[r],
                                 lse_partial=lses[r])
    o, lse = dcp.lse_merge(parts, lses)
    torch.cuda.synchronize()
    op_ref, lp_ref = oracle.shard_partials(w, batch_indices=rows, ownership="token")
    compare(parts[0], lses[0], op_ref[0], lp_ref[0], rows=rows, **TOL["bf16"], label="shard 0")
    o_ref, lse_ref = oracle.decode_reference(w, batch_indices=rows)
    compare(o, lse, o_ref, lse_ref, rows=rows, **TOL["bf16"], label="merged")
