"""Block-table remap (bit-exact) and the standalone LSE merge against the oracle."""
import json
from pathlib import Path

import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import oracle
import workloads as W
from gpu_helpers import need_gpu, to_np

pytestmark = pytest.mark.gpu
GOLDEN = Path(__file__).parent / "golden"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _remap_gpu(table, lens, bs, d, ownership="interleaved"):
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
    l = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
    lt, ll = dcp.block_remap(t, l, bs, d, ownership=ownership)
    torch.cuda.synchronize()
    return lt.cpu().numpy(), ll.cpu().numpy()


def test_remap_worked_example():
    g = json.loads((GOLDEN / "remap_ragged.json").read_text())
    lt, ll = _remap_gpu(np.array([g["block_table"]]), np.array([g["seq_len"]]),
                        g["block_size"], g["num_shards"])
    assert lt[:, 0, :].tolist() == g["local_tables"]
    assert ll[:, 0].tolist() == g["local_lens"]


@pytest.mark.parametrize("name", list(W.SPECS))
def test_remap_full_size_tables(name):
    spec = W.SPECS[name]
    lens = W.seq_lengths(spec)
    table, _ = W.build_block_table(lens, spec.block_size, spec.seed)
    lt, ll = _remap_gpu(table, lens, spec.block_size, spec.num_shards)
    rt, rl = oracle.remap_block_table(table, lens, spec.block_size, spec.num_shards)
    assert np.array_equal(lt, rt) and np.array_equal(ll, rl)


# Block-level ownerships only: under token-level interleave every block holds
# tokens of every shard, so there is no per-shard table to remap.
@pytest.mark.parametrize("ownership", ["interleaved", "contiguous"])
def test_remap_edges(ownership):
    rng = np.random.default_rng(5)
    for bs in (1, 3, 16, 64):
        for d in (1, 2, 3, 4, 7, 8, 9):
            lens = np.array([0, 1, bs - 1, bs, bs + 1, 2 * bs, d * bs - 1, d * bs, d * bs + 1,
                             5 * d * bs + 3, (d - 1) * bs + 1], dtype=np.int32)
            lens = np.maximum(lens, 0)
            mb = int(-(-lens.max() // bs)) + 1
            table = rng.permutation(100000)[: len(lens) * mb].reshape(len(lens), mb).astype(np.int32)
            lt, ll = _remap_gpu(table, lens, bs, d, ownership)
            rt, rl = oracle.remap_block_table(table, lens, bs, d, ownership)
            assert np.array_equal(lt, rt), (bs, d)
            assert np.array_equal(ll, rl), (bs, d)


def test_remap_contiguous_page_example():
    g = json.loads((GOLDEN / "contiguous_split.json").read_text())
    bs, d, L = g["block_size"], g["num_shards"], g["seq_len"]
    nb = L // bs
    table = (7 + np.arange(nb, dtype=np.int32))[None, :]
    lt, ll = _remap_gpu(table, np.array([L]), bs, d, "contiguous")
    assert ll[:, 0].tolist() == [hi - lo for lo, hi in g["token_ranges"]]
    for r, (lo, hi) in enumerate(g["token_ranges"]):
        row = lt[r, 0]
        assert row.tolist() == (7 + np.arange(lo // bs, hi // bs)).tolist()


@pytest.mark.parametrize("name", ["mla_bf16_b64_bimodal", "mla_fp8_b128_bimodal"])
def test_remap_contiguous_full_size_tables(name):
    spec = W.SPECS[name]
    lens = W.seq_lengths(spec)
    table, _ = W.build_block_table(lens, spec.block_size, spec.seed)
    lt, ll = _remap_gpu(table, lens, spec.block_size, spec.num_shards, "contiguous")
    rt, rl = oracle.remap_block_table(table, lens, spec.block_size, spec.num_shards, "contiguous")
    assert np.array_equal(lt, rt) and np.array_equal(ll, rl)


def test_remap_rejects_unknown_ownership():
    t = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    l = torch.ones(1, dtype=torch.int32, device="cuda")
    out_t = torch.empty((2, 1, 2), dtype=torch.int32, device="cuda")
    out_l = torch.empty((2, 1), dtype=torch.int32, device="cuda")
    status = dcp.lib().dcp_block_remap_ex(t.data_ptr(), l.data_ptr(), 1, 4, 16, 2, 5,
                                          out_t.data_ptr(), out_l.data_ptr(), None)
    assert status == dcp.DCP_ERR_INVALID_ARG


def _rand_partials(p, b, h, dv, seed):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((p, b, h, dv)).astype(np.float32)
    lse = (rng.standard_normal((p, b, h)) * 4).astype(np.float32)
    lse[rng.random((p, b, h)) < 0.2] = -np.inf
    lse[:, 0, 0] = -np.inf  # one row with no tokens anywhere
    return o, lse


@pytest.mark.parametrize("p,dv", [(1, 64), (2, 128), (8, 512), (13, 512), (4, 4), (3, 96),
                                  (2, 1024), (5, 12), (40, 256)])
def test_merge_matches_oracle(p, dv):
    o, lse = _rand_partials(p, 3, 5, dv, p * 31 + dv)
    go, gl = dcp.lse_merge(torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda())
    ro, rl = oracle.lse_merge(o.astype(np.float64), lse.astype(np.float64))
    go, gl = to_np(go), to_np(gl)
    assert np.all(go[0, 0] == 0) and gl[0, 0] == -np.inf
    live = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), live)
    assert np.allclose(go, ro, rtol=2e-6, atol=2e-6)
    assert np.allclose(gl[live], rl[live], rtol=0, atol=2e-6)


def test_merge_bf16_out_and_no_lse():
    o, lse = _rand_partials(8, 2, 4, 512, 3)
    out, l = dcp.lse_merge(torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda(),
                           out_dtype=torch.bfloat16, want_lse=False)
    assert l is None and out.dtype == torch.bfloat16
    ro, _ = oracle.lse_merge(o.astype(np.float64), lse.astype(np.float64))
    assert np.allclose(to_np(out), ro, rtol=2 ** -8, atol=1e-6)


def test_merge_permutation_associativity_identity():
    o, lse = _rand_partials(9, 4, 6, 128, 8)
    to, tl = torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda()
    base_o, base_l = dcp.lse_merge(to, tl)
    perm = torch.tensor([3, 8, 0, 5, 1, 7, 2, 6, 4], device="cuda")
    po, pl = dcp.lse_merge(to[perm].contiguous(), tl[perm].contiguous())
    assert torch.allclose(po, base_o, rtol=1e-6, atol=1e-6)
    assert torch.allclose(pl, base_l, rtol=1e-6, atol=1e-6)
    ao, al = dcp.lse_merge(to[:4].contiguous(), tl[:4].contiguous())
    co, cl = dcp.lse_merge(torch.cat([ao[None], to[4:]]), torch.cat([al[None], tl[4:]]))
    assert torch.allclose(co, base_o, rtol=1e-5, atol=1e-6)
    assert torch.allclose(cl, base_l, rtol=1e-6, atol=1e-6)
    eo = torch.cat([to, torch.full_like(to[:1], float("nan"))])
    el = torch.cat([tl, torch.full_like(tl[:1], -np.inf)])
    xo, xl = dcp.lse_merge(eo, el)
    torch.cuda.synchronize()
    assert torch.equal(xo, base_o) and torch.equal(xl, base_l)
