"""Multi-token (draft / MTP) decode against the oracle: q_len query tokens per
sequence at its last q_len positions, each seeing the positions up to its own,
fused over all shards and per shard through global positions."""
import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import oracle
import workloads as W
from gpu_helpers import TOL, compare, desc_for, need_gpu, run_all_shards

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


LENS = [1, 2, 3, 5, 31, 32, 33, 63, 64, 65, 129, 700, 2000]

CASES = [
    # kind, dtype, block size, shards, Hq, Hkv, qk_dim, v_dim, q_len   (kernel)
    ("mla", "bf16", 64, 8, 64, 1, 576, 512, 2),    # producer/consumer, 2 head groups
    ("mla", "bf16", 64, 3, 64, 1, 576, 512, 4),
    ("mla", "fp8", 64, 8, 64, 1, 576, 512, 3),
    ("mla", "bf16", 64, 4, 16, 1, 576, 512, 4),    # general kernel, 32-token tiles
    ("mla", "bf16", 16, 4, 32, 1, 576, 512, 2),    # general kernel, tiles over blocks
    ("mla", "fp8", 48, 5, 16, 1, 576, 512, 2),
    ("gqa", "bf16", 16, 4, 64, 8, 128, 128, 2),    # group 8 x 2 tokens = one column tile
    ("gqa", "bf16", 16, 3, 32, 8, 128, 128, 3),    # group 4 x 3 = 12 columns
    ("gqa", "bf16", 5, 2, 12, 4, 64, 64, 7),       # group 3 x 7 = 21: two column tiles
    ("gqa", "f32", 16, 2, 8, 2, 64, 64, 5),        # group 4 x 5 = 20: two column tiles
    ("gqa", "f32", 5, 3, 4, 1, 128, 128, 2),
]


def _workload(case, lens=LENS, seed=7):
    kind, dtype, bs, d, hq, hkv, dqk, dv, n = case
    return W.custom(kind, lens, num_q_heads=hq, num_kv_heads=hkv, qk_dim=dqk, v_dim=dv,
                    block_size=bs, num_shards=d, kv_dtype=dtype, seed=seed, q_len=n)


def _ids(c):
    return f"{c[0]}-{c[1]}-bs{c[2]}-D{c[3]}-h{c[4]}-q{c[8]}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_mtp_all_shards_matches_oracle(case):
    w = _workload(case)
    o_ref, lse_ref = oracle.decode_reference(w)
    assert np.isinf(lse_ref).any()  # lengths below q_len leave early queries without tokens
    o, lse, _, _ = run_all_shards(w)
    compare(o, lse, o_ref, lse_ref, **TOL[case[1]], label=f"mtp {_ids(case)}")


@pytest.mark.parametrize("case", CASES[::2], ids=_ids)
def test_mtp_per_shard_partials_and_merge(case):
    """Each shard sees only its local table; global positions come from
    shard + D * (local block). The merged shards equal unsharded attention."""
    w = _workload(case)
    dev = W.to_torch(w)
    d = case[3]
    desc = desc_for(w, dev)
    lt, ll = dcp.block_remap(dev.block_table, dev.seq_lens, case[2], d)
    q_pos = (dev.seq_lens - case[8]).to(torch.int32).contiguous()
    ws = dcp.alloc_workspace(desc, dev.q.device)
    op_ref, lp_ref = oracle.shard_partials(w)
    outs, lses = [], []
    for r in range(d):
        o, l = dcp.decode_partial_mtp(desc, r, q_pos, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                      lt[r].contiguous(), ll[r].contiguous(), workspace=ws)
        outs.append(o.clone())
        lses.append(l.clone())
        compare(o, l, op_ref[r], lp_ref[r], **TOL[case[1]], label=f"shard {r}")
    o, lse = dcp.lse_merge(torch.stack(outs), torch.stack(lses))
    o_ref, lse_ref = oracle.decode_reference(w)
    compare(o, lse, o_ref, lse_ref, **TOL[case[1]], label="merged shards")


@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[7]], ids=_ids)
def test_mtp_explicit_query_positions(case):
    """Query positions below the cache's end hide the positions after them: q_pos = L - q_len - 9."""
    kind, dtype, bs, d, hq, hkv, dqk, dv, n = case
    w = _workload(case)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    qp = np.maximum(w.seq_lens.astype(np.int64) - n - 9, -n).astype(np.int32)
    lt, ll = dcp.block_remap(dev.block_table, dev.seq_lens, bs, d)
    op_ref, lp_ref = oracle.shard_partials(w, q_pos=qp)
    q_pos = torch.from_numpy(qp).cuda()
    for r in range(d):
        o, l = dcp.decode_partial_mtp(desc, r, q_pos, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                      lt[r].contiguous(), ll[r].contiguous())
        compare(o, l, op_ref[r], lp_ref[r], **TOL[dtype], label=f"shard {r}")


def test_mtp_single_token_positions_hide_tail():
    """q_len 1 with explicit positions: each shard sees positions <= q_pos only."""
    case = ("mla", "bf16", 64, 4, 64, 1, 576, 512, 1)
    w = _workload(case, lens=[100, 700, 64, 1])
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    qp = np.array([37, 650, 63, 0], dtype=np.int32)
    lt, ll = dcp.block_remap(dev.block_table, dev.seq_lens, 64, 4)
    op_ref, lp_ref = oracle.shard_partials(w, q_pos=qp)
    for r in range(4):
        o, l = dcp.decode_partial_mtp(desc, r, torch.from_numpy(qp).cuda(), dev.q, dev.k_cache,
                                      None, None, lt[r].contiguous(), ll[r].contiguous())
        compare(o, l, op_ref[r], lp_ref[r], **TOL["bf16"], label=f"shard {r}")


def test_mtp_argument_errors():
    w = _workload(CASES[0], lens=[70, 3])
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    lt, ll = dcp.block_remap(dev.block_table, dev.seq_lens, 64, 8)
    with pytest.raises(dcp.DcpValueError):  # several query tokens need positions
        dcp.decode_partial(desc, dev.q, dev.k_cache, None, None, lt[0].contiguous(),
                           ll[0].contiguous())
    q_pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(dcp.DcpValueError):  # shard out of range
        dcp.decode_partial_mtp(desc, 8, q_pos, dev.q, dev.k_cache, None, None, lt[0].contiguous(),
                               ll[0].contiguous())
    bad = desc_for(w, dev)
    bad.q_len = 65
    with pytest.raises(dcp.DcpValueError):
        dcp.workspace_size(bad)
