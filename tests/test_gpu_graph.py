"""The fused path inside a captured HIP graph (the library enqueues only
kernels, no memsets or allocations), and the timed entry point."""
import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import workloads as W
from gpu_helpers import desc_for, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("spec", [W.scaled(W.SPECS["mla_bf16_b64_bimodal"], 16, 128),
                                  W.scaled(W.SPECS["mla_fp8_b128_bimodal"], 16, 128),
                                  W.scaled(W.SPECS["gqa_bf16_b32_L32k"], 8, 64)],
                         ids=lambda s: s.name)
def test_graph_replays_match_eager(spec):
    w = W.make(spec)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    ws = dcp.alloc_workspace(desc, "cuda")
    rows = spec.q_len * spec.num_q_heads
    out = torch.empty((spec.batch, rows, spec.v_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((spec.batch, rows), dtype=torch.float32, device="cuda")

    def call():
        dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                              dev.block_table, dev.seq_lens, workspace=ws, out=out, lse_out=lse)

    call()
    torch.cuda.synchronize()
    o_ref, l_ref = out.clone(), lse.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xAB)  # stale workspace contents must not matter
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), f"replay {i}"
        assert torch.equal(lse, l_ref), f"replay {i}"
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref)


def test_timed_entry_point_matches_and_times_the_kernel():
    spec = W.scaled(W.SPECS["mla_bf16_b64_bimodal"], 8, 16)
    w = W.make(spec)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    ws = dcp.alloc_workspace(desc, "cuda")
    o1, l1 = dcp.decode_all_shards(desc, dev.q, dev.k_cache, None, None, dev.block_table,
                                   dev.seq_lens, workspace=ws)
    ev = (dcp.HipEvent(), dcp.HipEvent())
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    o2, l2 = dcp.decode_all_shards(desc, dev.q, dev.k_cache, None, None, dev.block_table,
                                   dev.seq_lens, workspace=ws, attn_events=ev)
    stop.record()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    kernel_ms = ev[0].elapsed_ms(ev[1])
    assert 0.0 < kernel_ms <= start.elapsed_time(stop) * 1.05 + 0.05
