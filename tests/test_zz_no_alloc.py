"""dcp_decode_all_shards_noalloc (static device scratch, no workspace argument)
against dcp_decode_all_shards on the same inputs, through the C ABI.

Two calls in a row, the second on a smaller batch with shorter sequences, so the
second call runs on scratch that still holds the first call's plan and
partials; both must equal the workspace entry point's results bit for bit (the
same kernels on the same inputs) and the oracle within the bf16 / fp8 bars. A
descriptor that needs more scratch than the array holds is rejected before
anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import oracle
import workloads as W
from gpu_helpers import TOL, compare, desc_for, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _both(w):
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    rows = w.spec.q_len * w.spec.num_q_heads
    o_ws, lse_ws = dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                         dev.block_table, dev.seq_lens)
    o_na = torch.full((w.spec.batch, rows, w.spec.v_dim), float("nan"), device="cuda")
    lse_na = torch.full((w.spec.batch, rows), float("nan"), device="cuda")
    dcp.decode_all_shards_noalloc(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                  dev.block_table, dev.seq_lens, o_na, lse_na)
    torch.cuda.synchronize()
    return o_ws, lse_ws, o_na, lse_na


@pytest.mark.parametrize("kind,dtype,bs,hq,hkv,dim,q_len", [
    ("mla", "bf16", 64, 64, 1, 576, 1),
    ("mla", "fp8", 64, 64, 1, 576, 1),
    ("mla", "bf16", 64, 32, 1, 576, 2),
    ("mla", "bf16", 16, 32, 1, 576, 1),
    ("gqa", "bf16", 16, 64, 8, 128, 1),
])
def test_noalloc_matches_workspace_entry_point(kind, dtype, bs, hq, hkv, dim, q_len):
    big = [40000, 1, 0, 777, 129000, 5000, 64, 65, 20000, 3]
    small = [300, 4096, 1]
    for lens, seed in ((big, 3), (small, 4)):
        w = W.custom(kind, lens, num_q_heads=hq, num_kv_heads=hkv, qk_dim=dim,
                     v_dim=512 if kind == "mla" else dim, block_size=bs, num_shards=8,
                     kv_dtype=dtype, seed=seed, q_len=q_len)
        o_ws, lse_ws, o_na, lse_na = _both(w)
        assert torch.equal(o_na, o_ws), f"{len(lens)} sequences: outputs differ"
        assert torch.equal(lse_na, lse_ws), f"{len(lens)} sequences: LSEs differ"
        o_ref, lse_ref = oracle.decode_reference(w)
        compare(o_na, lse_na, o_ref, lse_ref, **TOL[dtype], label=f"noalloc, {len(lens)} sequences")


@pytest.mark.parametrize("batch,q_len", [(2048, 1), (4, 2)])
def test_noalloc_rejects_descriptors_beyond_the_scratch(batch, q_len):
    """Partials beyond the static array (a large batch; 128 query rows per
    sequence, whose 255+ partial slots take 67 MB): DCP_ERR_WORKSPACE, nothing
    enqueued."""
    w = W.custom("mla", [64] * 4, num_q_heads=64, num_kv_heads=1, qk_dim=576, v_dim=512,
                 block_size=64, num_shards=8, kv_dtype="bf16", seed=1, q_len=q_len)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    desc.batch = batch  # (never launched: the size check comes first)
    need = dcp.lib().dcp_workspace_size(ctypes.byref(desc))
    assert need > 64 << 20
    out = torch.zeros(1, device="cuda")
    status = dcp.lib().dcp_decode_all_shards_noalloc(
        ctypes.byref(desc), dev.q.data_ptr(), dev.k_cache.data_ptr(), None, None,
        dev.block_table.data_ptr(), dev.seq_lens.data_ptr(), out.data_ptr(), None, None)
    assert status == dcp.DCP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert float(out.item()) == 0.0
