"""Edge cases on the GPU: empty and ragged sequences, tiny and odd block sizes,
shard counts above the block count, other head counts, and unusable block ids."""
import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import oracle
import workloads as W
from gpu_helpers import TOL, compare, desc_for, need_gpu, run_all_shards, run_per_shard

pytestmark = pytest.mark.gpu

EDGE_LENS = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 129, 1000]

CASES = [
    # kind, kv dtype, block size, shards, Hq, Hkv, qk_dim
    ("mla", "bf16", 64, 8, 64, 1, 576),
    ("mla", "fp8", 64, 8, 64, 1, 576),
    ("mla", "bf16", 16, 4, 64, 1, 576),
    ("mla", "fp8", 32, 3, 32, 1, 576),
    ("mla", "bf16", 128, 2, 128, 1, 576),
    ("mla", "bf16", 1, 8, 16, 1, 576),
    ("mla", "fp8", 48, 5, 64, 1, 576),
    ("mla", "fp8", 32, 3, 64, 1, 576),
    ("mla", "fp8", 128, 2, 128, 1, 576),
    ("gqa", "bf16", 16, 4, 64, 8, 128),
    ("gqa", "bf16", 16, 3, 16, 1, 64),
    ("gqa", "bf16", 8, 2, 32, 2, 128),
    ("gqa", "bf16", 5, 7, 12, 4, 64),
    ("gqa", "f32", 16, 2, 4, 1, 64),
    ("gqa", "f32", 5, 3, 8, 2, 128),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _workload(kind, dtype, bs, d, hq, hkv, dim, lens, seed=11):
    return W.custom(kind, lens, num_q_heads=hq, num_kv_heads=hkv, qk_dim=dim,
                    v_dim=512 if kind == "mla" else dim, block_size=bs, num_shards=d,
                    kv_dtype=dtype, seed=seed)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_edge_lengths(case):
    w = _workload(*case, EDGE_LENS)
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse, dev, _ = run_all_shards(w)
    compare(o, lse, o_ref, lse_ref, **TOL[case[1]], label="all shards")
    op, lp, _, _ = run_per_shard(w, dev)
    opr, lpr = oracle.shard_partials(w)
    for r in range(case[3]):
        compare(op[r], lp[r], opr[r], lpr[r], **TOL[case[1]], label=f"shard {r}")


def test_all_sequences_empty():
    w = _workload("mla", "bf16", 64, 8, 64, 1, 576, [0, 0, 0])
    o, lse, _, _ = run_all_shards(w)
    assert float(o.abs().max()) == 0.0 and bool((lse == -np.inf).all())


@pytest.mark.parametrize("kind,dtype", [("mla", "bf16"), ("mla", "fp8"), ("gqa", "bf16"),
                                        ("gqa", "f32")])
def test_unusable_block_ids_are_skipped(kind, dtype):
    dim = 576 if kind == "mla" else 128
    bs = 64 if kind == "mla" else 16
    w = _workload(kind, dtype, bs, 4, 64 if kind == "mla" else 16, 1 if kind == "mla" else 2,
                  dim, [5 * bs + 7, 3 * bs, 2 * bs + 1])
    bad = {0: [1, 4], 1: [2], 2: [0]}
    for b, blocks in bad.items():
        for j in blocks:
            w.block_table[b, j] = -7 if j % 2 else w.num_blocks + 3
    o_ref = np.zeros((3, w.spec.num_q_heads, w.spec.v_dim))
    lse_ref = np.zeros((3, w.spec.num_q_heads))
    for b in range(3):
        pos = [t for t in range(int(w.seq_lens[b])) if t // bs not in bad[b]]
        k, v = oracle.sequence_kv(w, b, np.array(pos))
        o_ref[b], lse_ref[b] = oracle.attend(oracle.query(w, b), k, v, w.spec.softmax_scale)
    o, lse, _, _ = run_all_shards(w)
    compare(o, lse, o_ref, lse_ref, **TOL[dtype], label="skipped ids")


@pytest.mark.parametrize("kind,dtype,bs,hq,hkv,dim", [
    ("mla", "bf16", 64, 64, 1, 576),
    ("mla", "fp8", 64, 64, 1, 576),
    ("mla", "fp8", 64, 32, 1, 576),
    ("gqa", "bf16", 16, 64, 8, 128),
])
def test_sharp_softmax(kind, dtype, bs, hq, hkv, dim):
    """A large softmax scale spreads the scores over tens of log2 units, so a
    head's running maximum rises (and its accumulators are rescaled) many
    times within a shard's range, and most probabilities underflow."""
    w = W.custom(kind, [3000, 777, 4096], num_q_heads=hq, num_kv_heads=hkv, qk_dim=dim,
                 v_dim=512 if kind == "mla" else dim, block_size=bs, num_shards=4,
                 kv_dtype=dtype, softmax_scale=0.5, seed=5)
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse, _, _ = run_all_shards(w)
    compare(o, lse, o_ref, lse_ref, **TOL[dtype], label="sharp softmax")


@pytest.mark.parametrize("kind,dtype", [("mla", "bf16"), ("mla", "fp8"), ("gqa", "bf16")])
def test_device_lengths_are_clamped(kind, dtype):
    """Device-resident lengths are not validated: a negative length reads as 0 and a
    length past the table's reach reads as the table width times the block size."""
    dim = 576 if kind == "mla" else 128
    bs = 64 if kind == "mla" else 16
    hq, hkv = (64, 1) if kind == "mla" else (16, 2)
    lens = [3 * bs + 5, 2 * bs, 1]
    w = _workload(kind, dtype, bs, 4, hq, hkv, dim, lens)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    mb = w.block_table.shape[1]
    o_ref, lse_ref = oracle.decode_reference(w)
    bad = torch.tensor([-5, 10 ** 6, 1], dtype=torch.int32, device="cuda")
    o, lse = dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                   dev.block_table, bad)
    torch.cuda.synchronize()
    # Sequence 0 reads as empty. Sequence 1 reads as mb * bs tokens, but its row
    # maps only its own blocks (the rest are -1, skipped): the result is its
    # attention over those, the same as for its true length.
    assert mb * bs > 2 * bs
    o_ref[0], lse_ref[0] = 0.0, -np.inf
    compare(o, lse, o_ref, lse_ref, **TOL[dtype], label="clamped lengths")


def test_empty_cache_pool():
    """num_cache_blocks = 0 with null cache pointers: every sequence is empty."""
    w = _workload("mla", "bf16", 64, 8, 64, 1, 576, [100, 7])
    dev = W.to_torch(w)
    empty = torch.empty((0, 64, 576), dtype=torch.bfloat16, device="cuda")
    desc = dcp.make_desc(dcp.KV_LATENT, dev.q, empty, dev.block_table, num_shards=8, v_dim=512,
                         max_seq_len=100)
    o, lse = dcp.decode_all_shards(desc, dev.q, None, None, None, dev.block_table, dev.seq_lens)
    torch.cuda.synchronize()
    assert float(o.abs().max()) == 0.0 and bool((lse == -np.inf).all())


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("hq", [16, 32])
def test_latent_few_heads_padded_group(dtype, hq):
    """Single-token latent decode with 16 or 32 query heads runs as one 64-row
    head group padded with zero queries: the results of the real heads match
    the oracle, and nothing is written past the workspace (a guard zone after
    it keeps its fill)."""
    lens = [0, 1, 63, 64, 65, 1000, 4097, 9000, 2, 300]
    w = _workload("mla", dtype, 64, 4, hq, 1, 576, lens, seed=17)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    n = dcp.workspace_size(desc)
    guard = 1 << 20
    buf = torch.full((n + guard,), 0x5A, dtype=torch.uint8, device=dev.q.device)
    o, lse = dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                   dev.block_table, dev.seq_lens, workspace=buf[:n])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_reference(w)
    compare(o, lse, o_ref, lse_ref, **TOL[dtype], label=f"all shards {hq} heads")
    assert bool((buf[n:] == 0x5A).all()), "write past the workspace"
    lt, ll = dcp.block_remap(dev.block_table, dev.seq_lens, 64, 4)
    opr, lpr = oracle.shard_partials(w)
    for r in range(4):
        o_r, l_r = dcp.decode_partial(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                      lt[r].contiguous(), ll[r].contiguous(), workspace=buf[:n])
        torch.cuda.synchronize()
        compare(o_r, l_r, opr[r], lpr[r], **TOL[dtype], label=f"shard {r} {hq} heads")
    assert bool((buf[n:] == 0x5A).all()), "write past the workspace"


def _scale_bf16_bits(x, k):
    """bf16 bit patterns times 2^k, exactly (the exponent field moved by k);
    zeros stay zero."""
    e = ((x >> 7) & 0xFF).astype(np.int32)
    assert e.max() + k < 255 and (e[e != 0].min() + k) > 0
    y = x.astype(np.int32)
    y[e != 0] += k << 7
    return y.astype(np.uint16)


@pytest.mark.parametrize("shift", [60, -60])
def test_latent_piece_rows_far_outside_fp16_range(shift):
    """A latent cache 2^shift times a normal draw, read by a query 2^-shift
    times one: the scores, the softmax and the LSE are those of the unscaled
    draw, and the outputs 2^shift times theirs, far outside fp16's range. The
    fp16 partial rows of split sequences carry a power-of-two scale per
    128-column slice, so the outputs match the oracle in relative terms."""
    from dataclasses import replace

    lens = [5000, 3000, 64, 1, 9000, 700]
    w = _workload("mla", "bf16", 64, 4, 64, 1, 576, lens, seed=21)
    w = replace(w, k_cache=_scale_bf16_bits(w.k_cache, shift), q=_scale_bf16_bits(w.q, -shift))
    o_ref, lse_ref = oracle.decode_reference(w)
    f = 2.0 ** -shift
    o, lse, dev, _ = run_all_shards(w)
    compare(o * f, lse, o_ref * f, lse_ref, **TOL["bf16"], label=f"all shards, 2^{shift}")
    op, lp, _, _ = run_per_shard(w, dev)
    opr, lpr = oracle.shard_partials(w)
    for r in range(4):
        compare(op[r] * f, lp[r], opr[r] * f, lpr[r], **TOL["bf16"], label=f"shard {r}, 2^{shift}")


@pytest.mark.parametrize("bs", [8224, 16384])
def test_latent_blocks_above_8192_tokens(bs):
    """Blocks of more than 8192 tokens (the producer/consumer kernel's window
    holds at most one such block, so these go to the general latent kernel):
    several blocks per sequence, a partial last block and an empty sequence."""
    lens = [20000, bs + 1, 1, 0, 40000]
    w = _workload("mla", "bf16", bs, 3, 64, 1, 576, lens, seed=23)
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse, dev, _ = run_all_shards(w)
    compare(o, lse, o_ref, lse_ref, **TOL["bf16"], label=f"all shards, bs {bs}")
    op, lp, _, _ = run_per_shard(w, dev)
    opr, lpr = oracle.shard_partials(w)
    for r in range(3):
        compare(op[r], lp[r], opr[r], lpr[r], **TOL["bf16"], label=f"shard {r}, bs {bs}")
