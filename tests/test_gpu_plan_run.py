"""Plan once, run per layer (dcp_decode_partial_plan / _run and
dcp_decode_all_shards_plan / _run).

A plan depends only on the descriptor's shape and the sequence lengths, which
every layer of a decode step shares (the remap of "vLLM长序列推理优化"
section 6.2 is kept and reused the same way). Checked here: several "layers"
(different queries and caches of one shape) run on one plan give exactly the
unplanned calls' results, bit for bit, and those match the fp64 oracle; a run
after the caller changed its lengths array uses the planned lengths; a run on a
workspace that holds no plan, or a plan of another shape, writes NaN and
nothing else.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import oracle
import workloads as W
from gpu_helpers import TOL, compare, desc_for, need_gpu

pytestmark = pytest.mark.gpu

SPECS = [
    W.scaled(W.SPECS["gqa_bf16_b32_L32k"]),        # B 4, L 512, 64/8 heads, D 4
    W.scaled(W.SPECS["mla_bf16_b64_bimodal"]),     # B 8, ragged lengths, D 8
    W.scaled(W.SPECS["mla_fp8_b128_bimodal"]),     # B 16, ragged, fp8 + scales
]
# Single-token latent decode with 16 or 32 heads (one zero-padded 64-row group).
FEW_HEADS = [
    replace(W.scaled(W.SPECS["mla_bf16_b64_bimodal"]), name="mla_bf16_16_heads", num_q_heads=16),
    replace(W.scaled(W.SPECS["mla_fp8_b128_bimodal"]), name="mla_fp8_32_heads", num_q_heads=32),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def second_layer(dev):
    """Another layer of the same shape: the query negated (exact) and every
    cache block moved one place along the pool (same lengths and tables, other
    rows under them)."""
    from types import SimpleNamespace

    roll = lambda t: None if t is None else torch.roll(t, 1, dims=0).contiguous()
    return SimpleNamespace(q=(-dev.q).contiguous(), k_cache=roll(dev.k_cache),
                           v_cache=roll(dev.v_cache), kv_scale=roll(dev.kv_scale),
                           block_table=dev.block_table, seq_lens=dev.seq_lens)


def same(a, b):
    """Bit-identical tensors (bf16 compared as raw 16-bit patterns)."""
    if a.dtype == torch.bfloat16:
        return b.dtype == torch.bfloat16 and torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


@pytest.mark.parametrize("spec", SPECS + FEW_HEADS, ids=lambda s: s.name)
def test_partial_runs_on_one_plan_match_unplanned(spec):
    w = W.make(spec)
    dev = W.to_torch(w)
    lay = [dev, second_layer(dev)]
    desc = desc_for(w, dev)
    D = spec.num_shards
    lt, ll = dcp.block_remap(dev.block_table, dev.seq_lens, spec.block_size, D)
    ws_plan = dcp.alloc_workspace(desc, dev.q.device)
    ws_ref = dcp.alloc_workspace(desc, dev.q.device)
    op_ref, lp_ref = oracle.shard_partials(w)
    for r in range(D):
        ltr, llr = lt[r].contiguous(), ll[r].contiguous()
        dcp.decode_partial_plan(desc, llr, ws_plan)
        for i, x in enumerate(lay):
            o, l = dcp.decode_partial_run(desc, x.q, x.k_cache, x.v_cache, x.kv_scale, ltr, ws_plan)
            o_u, l_u = dcp.decode_partial(desc, x.q, x.k_cache, x.v_cache, x.kv_scale, ltr, llr,
                                          workspace=ws_ref)
            torch.cuda.synchronize()
            assert torch.equal(o, o_u) and torch.equal(l, l_u), f"shard {r} layer {i}"
            if i == 0:
                compare(o, l, op_ref[r], lp_ref[r], **TOL[spec.kv_dtype], label=f"shard {r}")


@pytest.mark.parametrize("q_len", [1, 2])
@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_all_shards_runs_on_one_plan_match_unplanned(spec, q_len):
    spec = replace(spec, q_len=q_len)
    w = W.make(spec)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    desc16 = desc_for(w, dev, out_dtype=dcp.BF16)  # same shape, bf16 output
    ws_plan = dcp.alloc_workspace(desc, dev.q.device)
    ws_ref = dcp.alloc_workspace(desc, dev.q.device)
    dcp.decode_all_shards_plan(desc, dev.seq_lens, ws_plan)
    o_ref, lse_ref = oracle.decode_reference(w)
    for i, x in enumerate([dev, second_layer(dev)]):
        for d in (desc, desc16):
            o, l = dcp.decode_all_shards_run(d, x.q, x.k_cache, x.v_cache, x.kv_scale,
                                             x.block_table, ws_plan)
            o_u, l_u = dcp.decode_all_shards(d, x.q, x.k_cache, x.v_cache, x.kv_scale,
                                             x.block_table, x.seq_lens, workspace=ws_ref)
            torch.cuda.synchronize()
            assert same(o, o_u) and torch.equal(l, l_u), f"layer {i} out dtype {d.out_dtype}"
            if i == 0 and d is desc:
                compare(o, l, o_ref, lse_ref, **TOL[spec.kv_dtype], label=spec.name)


def test_run_uses_the_planned_lengths():
    spec = W.scaled(W.SPECS["mla_bf16_b64_bimodal"])
    w = W.make(spec)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    ws = dcp.alloc_workspace(desc, dev.q.device)
    lens = dev.seq_lens.clone()
    dcp.decode_all_shards_plan(desc, lens, ws)
    lens.copy_(torch.div(lens, 3, rounding_mode="floor"))  # the caller's array changes
    o, l = dcp.decode_all_shards_run(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                     dev.block_table, ws)
    o_u, l_u = dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                     dev.block_table, dev.seq_lens)
    torch.cuda.synchronize()
    assert torch.equal(o, o_u) and torch.equal(l, l_u)


def test_run_without_a_matching_plan_writes_nan():
    spec = W.scaled(W.SPECS["mla_bf16_b64_bimodal"])
    w = W.make(spec)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    dv = dev.q.device
    # A workspace that was never planned.
    ws = torch.zeros(dcp.workspace_size(desc), dtype=torch.uint8, device=dv)
    o, l = dcp.decode_all_shards_run(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                     dev.block_table, ws)
    o16, _ = dcp.decode_all_shards_run(desc_for(w, dev, out_dtype=dcp.BF16), dev.q, dev.k_cache,
                                       dev.v_cache, dev.kv_scale, dev.block_table, ws,
                                       want_lse=False)
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and torch.isnan(l).all() and torch.isnan(o16.float()).all()
    # A plan of one shard's partial, then a run of the fused call on it.
    lt, ll = dcp.block_remap(dev.block_table, dev.seq_lens, spec.block_size, spec.num_shards)
    dcp.decode_partial_plan(desc, ll[0].contiguous(), ws)
    o, l = dcp.decode_all_shards_run(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                     dev.block_table, ws)
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and torch.isnan(l).all()
    # A plan for the whole batch, then a run of a descriptor with one sequence
    # fewer (the first B - 1 rows of the same tensors).
    dcp.decode_all_shards_plan(desc, dev.seq_lens, ws)
    small = desc_for(w, dev)
    small.batch = spec.batch - 1
    o, l = dcp.decode_all_shards_run(small, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                     dev.block_table, ws)
    torch.cuda.synchronize()
    assert o.shape[0] == spec.batch - 1
    assert torch.isnan(o).all() and torch.isnan(l).all()
    # The same workspace planned again for the run's shape works as usual.
    dcp.decode_all_shards_plan(small, dev.seq_lens[: spec.batch - 1].contiguous(), ws)
    o, l = dcp.decode_all_shards_run(small, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                     dev.block_table, ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_reference(w)
    rows = np.arange(spec.batch - 1)
    compare(o, l, o_ref[rows], lse_ref[rows], **TOL["bf16"], label="replanned")


@pytest.mark.parametrize("spec", [W.scaled(W.SPECS["mla_bf16_b64_bimodal"], 16, 128),
                                  W.scaled(W.SPECS["gqa_bf16_b32_L32k"], 8, 64),
                                  FEW_HEADS[1]],
                         ids=lambda s: s.name)
def test_run_captured_in_a_graph_follows_each_new_plan(spec):
    """The run alone captured in a HIP graph, the plan made eagerly before each
    replay: every replay computes what the unplanned call computes for the
    lengths of the latest plan and the query in the buffer at replay time, so
    one captured graph serves decode steps whose lengths change."""
    w = W.make(spec)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    ws = dcp.alloc_workspace(desc, "cuda")
    rows = spec.q_len * spec.num_q_heads
    out = torch.empty((spec.batch, rows, spec.v_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((spec.batch, rows), dtype=torch.float32, device="cuda")
    q = dev.q.clone()

    def run():
        dcp.decode_all_shards_run(desc, q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                  dev.block_table, ws, out=out, lse_out=lse)

    dcp.decode_all_shards_plan(desc, dev.seq_lens, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    lens_steps = [dev.seq_lens, torch.clamp(dev.seq_lens - 7, min=0),
                  torch.div(dev.seq_lens, 2, rounding_mode="floor")]
    for i, lens in enumerate(lens_steps):
        lens = lens.to(torch.int32).contiguous()
        q.copy_(dev.q if i % 2 == 0 else -dev.q)
        dcp.decode_all_shards_plan(desc, lens, ws)
        out.fill_(float("nan"))
        graph.replay()
        o_ref, l_ref = dcp.decode_all_shards(desc, q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                             dev.block_table, lens)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), f"step {i}"
