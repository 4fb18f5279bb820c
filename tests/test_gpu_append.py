"""KV append (dcp_kv_append) and the incremental table update (dcp_block_remap_update)
against the oracle: bit-exact cache contents, scales and tables."""
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


CASES = [
    # kind, cache dtype, new-row dtype, block size, shards, Hq, Hkv, qk_dim, v_dim
    ("gqa", "f32", "f32", 16, 3, 8, 2, 128, 128),
    ("gqa", "bf16", "bf16", 16, 4, 64, 8, 128, 128),
    ("gqa", "bf16", "bf16", 5, 2, 12, 4, 64, 64),
    ("mla", "bf16", "bf16", 64, 8, 64, 1, 576, 512),
    ("mla", "fp8", "bf16", 64, 8, 64, 1, 576, 512),
    ("mla", "fp8", "f32", 32, 3, 64, 1, 576, 512),
]
LENS = [1, 15, 16, 17, 64, 65, 200, 511, 512, 1000]


def _workload(case, lens, seed=3):
    kind, kvd, _, bs, d, hq, hkv, dqk, dv = case
    return W.custom(kind, lens, num_q_heads=hq, num_kv_heads=hkv, qk_dim=dqk, v_dim=dv,
                    block_size=bs, num_shards=d, kv_dtype=kvd, seed=seed)


def _new_rows(case, n, seed, spread=(0.01, 30.0)):
    """Host rows for n new tokens: (k_new, v_new) in stored form and as device tensors.
    Each token's rows are normal values times a per-token factor drawn from ``spread``."""
    kind, kvd, newd, _, _, _, hkv, dqk, dv = case
    rng = np.random.default_rng(seed)
    kshape = (n, hkv, dqk) if kind == "gqa" else (n, dqk)
    k = (rng.standard_normal(kshape) * rng.uniform(*spread, (n,) + (1,) * (len(kshape) - 1)))
    k = k.astype(np.float32)
    v = rng.standard_normal((n, hkv, dv)).astype(np.float32) if kind == "gqa" else None

    def host(x):
        return None if x is None else (W.encode_bf16(x) if newd == "bf16" else x)

    def dev(x):
        if x is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.view(torch.int16).view(torch.bfloat16) if x.dtype == np.uint16 else t).cuda()

    kh, vh = host(k), host(v)
    return kh, vh, dev(kh), dev(vh)


def _cache_np(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _check_caches(w, dev, k_ref, v_ref, s_ref):
    torch.cuda.synchronize()
    assert np.array_equal(_cache_np(dev.k_cache), k_ref)
    if v_ref is not None:
        assert np.array_equal(_cache_np(dev.v_cache), v_ref)
    if s_ref is not None:
        assert np.array_equal(_cache_np(dev.kv_scale).view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:5])))
def test_append_global_table_bit_exact(case):
    """Every sequence gains one token at position L - 1 (the slot its table already maps)."""
    w = _workload(case, LENS)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    n = len(LENS)
    kh, vh, kd, vd = _new_rows(case, n, 11)
    pos = np.array(LENS, dtype=np.int32) - 1
    k_ref, v_ref, s_ref = oracle.kv_append(w.k_cache, w.v_cache, w.kv_scale, w.block_table, pos, kh,
                                           vh, kv_dtype=case[1], block_size=case[3])
    dcp.kv_append(desc, torch.from_numpy(pos).cuda(), kd, vd, dev.block_table, dev.k_cache,
                  dev.v_cache, dev.kv_scale)
    _check_caches(w, dev, k_ref, v_ref, s_ref)


@pytest.mark.parametrize("case", CASES[1::2], ids=lambda c: "-".join(map(str, c[:5])))
def test_append_per_shard_tables(case):
    """Each shard writes only the tokens whose block it owns, through its local table; the
    union over shards equals one write through the global table."""
    w = _workload(case, LENS)
    dev = W.to_torch(w)
    d = case[4]
    desc = desc_for(w, dev)
    lt, _ = dcp.block_remap(dev.block_table, dev.seq_lens, case[3], d)
    kh, vh, kd, vd = _new_rows(case, len(LENS), 12)
    pos = np.array(LENS, dtype=np.int32) - 1
    local, _ = oracle.remap_block_table(w.block_table, w.seq_lens, case[3], d)
    k_ref, v_ref, s_ref = w.k_cache, w.v_cache, w.kv_scale
    for r in range(d):
        dcp.kv_append(desc, torch.from_numpy(pos).cuda(), kd, vd, lt[r].contiguous(), dev.k_cache,
                      dev.v_cache, dev.kv_scale, shard=r)
        k_ref, v_ref, s_ref = oracle.kv_append(k_ref, v_ref, s_ref, local[r], pos, kh, vh,
                                               kv_dtype=case[1], block_size=case[3],
                                               num_shards=d, shard=r)
        _check_caches(w, dev, k_ref, v_ref, s_ref)
    k_all, v_all, s_all = oracle.kv_append(w.k_cache, w.v_cache, w.kv_scale, w.block_table, pos,
                                           kh, vh, kv_dtype=case[1], block_size=case[3])
    assert np.array_equal(k_ref, k_all)


def test_append_token_map_and_skips():
    """Several tokens per sequence through token_seq; skipped tokens write nothing."""
    case = CASES[4]
    w = _workload(case, [300, 129, 64])
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    seq = np.array([0, 0, 0, 1, 2, 2, 1, 0, 5, -1, 1], dtype=np.int32)
    pos = np.array([297, 298, 299, 128, 62, 63, -4, 10**6, 3, 3, 0], dtype=np.int32)
    kh, _, kd, _ = _new_rows(case, len(pos), 13)
    k_ref, _, s_ref = oracle.kv_append(w.k_cache, None, w.kv_scale, w.block_table, pos, kh, None,
                                       kv_dtype="fp8", block_size=case[3], token_seq=seq)
    w.block_table[1, 0] = w.num_blocks + 5  # an unusable entry: token (1, 0) is skipped
    k_ref2, _, s_ref2 = oracle.kv_append(w.k_cache, None, w.kv_scale, w.block_table, pos, kh, None,
                                         kv_dtype="fp8", block_size=case[3], token_seq=seq)
    assert not np.array_equal(k_ref, k_ref2)
    dev.block_table[1, 0] = w.num_blocks + 5
    dcp.kv_append(desc, torch.from_numpy(pos).cuda(), kd, None, dev.block_table, dev.k_cache,
                  None, dev.kv_scale, token_seq=torch.from_numpy(seq).cuda())
    _check_caches(w, dev, k_ref2, None, s_ref2)


def test_fp8_encoding_ties_subnormals_and_zero_rows():
    """Rows with amax exactly 448 (scale 1, x * 448 / amax == x): midpoints between codes
    must round to the even code, subnormals and signed zeros must match the oracle."""
    case = ("mla", "fp8", "f32", 16, 1, 16, 1, 576, 512)
    w = _workload(case, [16] * 6)
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    codes = np.array([c for c in range(128) if c != 0x7F], dtype=np.uint8)
    vals = np.sort(oracle.e4m3_to_f64(codes))
    mids = 0.5 * (vals[1:] + vals[:-1])
    row = np.concatenate([[448.0], mids, -mids, vals, -vals, [-0.0, 0.0, 2.0 ** -12, -(2.0 ** -12)]])
    rows = np.zeros((6, 576), dtype=np.float32)
    rows[0, : len(row)] = row[:576]
    rows[1] = np.linspace(-3, 3, 576, dtype=np.float32)
    rows[2] = 0.0                      # all-zero token
    rows[3, 7] = 1e-38                 # 448 / amax overflows float32
    rows[4] = -rows[1] * 1e-30         # tiny but usable
    rows[5] = np.random.default_rng(9).standard_normal(576).astype(np.float32) * 1e4
    assert np.all(np.float32(448.0) / np.max(np.abs(rows[0])) == 1.0)
    pos = np.arange(6, dtype=np.int32) * 0 + 5
    k_ref, _, s_ref = oracle.kv_append(w.k_cache, None, w.kv_scale, w.block_table, pos, rows, None,
                                       kv_dtype="fp8", block_size=16)
    dcp.kv_append(desc, torch.from_numpy(pos).cuda(), torch.from_numpy(rows).cuda(), None,
                  dev.block_table, dev.k_cache, None, dev.kv_scale)
    _check_caches(w, dev, k_ref, None, s_ref)


@pytest.mark.parametrize("case", [CASES[3], CASES[4], CASES[1]], ids=lambda c: c[0] + c[1])
def test_decode_after_append_matches_oracle(case):
    """A decode step: append the new token at position L, then attend over L + 1 tokens."""
    lens = [0, 31, 64, 700, 2047]
    cap = [x + 1 for x in lens]
    w = _workload(case, cap, seed=5)
    dev = W.to_torch(w)
    kh, vh, kd, vd = _new_rows(case, len(lens), 14, spread=(0.5, 2.0))
    pos = np.array(lens, dtype=np.int32)
    desc = desc_for(w, dev)
    dcp.kv_append(desc, torch.from_numpy(pos).cuda(), kd, vd, dev.block_table, dev.k_cache,
                  dev.v_cache, dev.kv_scale)
    k2, v2, s2 = oracle.kv_append(w.k_cache, w.v_cache, w.kv_scale, w.block_table, pos, kh, vh,
                                  kv_dtype=case[1], block_size=case[3])
    w.k_cache, w.v_cache, w.kv_scale = k2, v2, s2
    o_ref, lse_ref = oracle.decode_reference(w)
    o, lse = dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                   dev.block_table, dev.seq_lens)
    compare(o, lse, o_ref, lse_ref, **TOL[case[1]], label="decode after append")


@pytest.mark.parametrize("d", [1, 2, 3, 8])
def test_remap_update_chain_equals_full_remap(d):
    """Decode steps grow every sequence by one token (crossing block boundaries), then a
    multi-token step, a shrink and an empty sequence; after each incremental update the
    tables equal a full remap of the new lengths."""
    bs, B = 4, 5
    rng = np.random.default_rng(21)
    lens = np.array([0, 3, 4, 9, 30], dtype=np.int32)
    mb = 16
    table = rng.permutation(1000)[: B * mb].reshape(B, mb).astype(np.int32)
    t = torch.from_numpy(table).cuda()
    cur = torch.from_numpy(lens).cuda()
    lt, ll = dcp.block_remap(t, cur, bs, d)
    steps = [lens + k for k in range(1, 10)]
    steps.append(steps[-1] + np.array([1, 13, 0, 5, 2], dtype=np.int32))
    steps.append(steps[-1] - np.array([0, 9, 3, 11, 20], dtype=np.int32))
    steps.append(np.array([0, 0, 64, 1, 70], dtype=np.int32))  # 70 clamps to mb * bs
    for new in steps:
        new_t = torch.from_numpy(np.ascontiguousarray(new, dtype=np.int32)).cuda()
        dcp.block_remap_update(t, cur, new_t, bs, d, lt, ll)
        torch.cuda.synchronize()
        rt, rl = oracle.remap_block_table(table, new, bs, d)
        assert np.array_equal(lt.cpu().numpy(), rt), new
        assert np.array_equal(ll.cpu().numpy(), rl), new
        cur = new_t


def test_append_argument_errors():
    case = CASES[4]
    w = _workload(case, [10])
    dev = W.to_torch(w)
    desc = desc_for(w, dev)
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    k16 = torch.zeros((1, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dcp.DcpValueError):  # shard out of range
        dcp.kv_append(desc, pos, k16, None, dev.block_table, dev.k_cache, None, dev.kv_scale,
                      shard=8)
    with pytest.raises(dcp.DcpValueError):  # fp8 cache without scales
        dcp.kv_append(desc, pos, k16, None, dev.block_table, dev.k_cache, None, None)
    with pytest.raises(dcp.DcpValueError):  # fp8 source rows are not accepted
        dcp.kv_append(desc, pos, torch.zeros((1, 576), dtype=torch.uint8, device="cuda"), None,
                      dev.block_table, dev.k_cache, None, dev.kv_scale)
    with pytest.raises(dcp.DcpValueError):  # row count does not match the positions
        dcp.kv_append(desc, pos, torch.zeros((2, 576), dtype=torch.bfloat16, device="cuda"), None,
                      dev.block_table, dev.k_cache, None, dev.kv_scale)
