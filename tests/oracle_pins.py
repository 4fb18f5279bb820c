"""Checks that pin the CPU oracle to things other than itself.

Each ``check_*`` takes the oracle package as its argument and raises
AssertionError on a mismatch. ``test_oracle.py`` runs them on the oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with one
planted mistake each and requires that some check fails.

Pins used: exhaustive comparison with torch's number-format conversions,
torch's scaled_dot_product_attention in float64, pure-Python brute force on
tiny inputs, closed forms, the merge identities, and the worked examples the
pages print (fixtures under tests/golden/, each carrying its citation).
"""
import json
import math
from pathlib import Path
from types import SimpleNamespace

import numpy as np
import torch

GOLDEN = Path(__file__).parent / "golden"


def _golden(name):
    with open(GOLDEN / name) as f:
        return json.load(f)


# ----------------------------------------------------------------- fake workloads
def fake_workload(kind, seq_lens, *, hq, hkv=1, dqk, dv, bs, kv_dtype="f32", scale=None,
                  seed=0, q_len=1):
    """A small paged workload built here, independent of the workloads module.

    The contiguous K/V (or latent) of each sequence is drawn first and then
    scattered into a shuffled block pool, so a gather mistake cannot cancel.
    Returns (workload, contiguous) where contiguous[b] = (q, K, V) float64.
    """
    rng = np.random.default_rng(seed)
    lens = np.asarray(seq_lens, dtype=np.int32)
    batch = len(lens)
    nb = [-(-int(l) // bs) for l in lens]
    total = sum(nb)
    perm = rng.permutation(max(total, 1))[:total]
    max_blocks = max(1, max(nb) if nb else 1)
    table = np.full((batch, max_blocks), -1, dtype=np.int32)
    width_k = (hkv, dqk) if kind == "gqa" else (dqk,)
    k_pool = rng.standard_normal((max(total, 1), bs) + width_k)
    v_pool = rng.standard_normal((max(total, 1), bs, hkv, dv)) if kind == "gqa" else None
    sigma_pool = rng.uniform(0.5, 2.0, (max(total, 1), bs)) if kv_dtype == "fp8" else None
    if kv_dtype == "bf16":
        k_pool = torch.from_numpy(k_pool.astype(np.float32)).to(torch.bfloat16)
        k_bits = k_pool.view(torch.int16).numpy().view(np.uint16)
        k_val = k_pool.to(torch.float64).numpy()
        if v_pool is not None:
            v_t = torch.from_numpy(v_pool.astype(np.float32)).to(torch.bfloat16)
            v_bits = v_t.view(torch.int16).numpy().view(np.uint16)
            v_val = v_t.to(torch.float64).numpy()
    elif kv_dtype == "fp8":
        k_t = torch.from_numpy(k_pool.astype(np.float32)).to(torch.float8_e4m3fn)
        k_bits = k_t.view(torch.uint8).numpy()
        k_val = k_t.to(torch.float64).numpy() * sigma_pool.astype(np.float32).astype(
            np.float64).reshape(sigma_pool.shape + (1,) * (k_pool.ndim - 2))
        if v_pool is not None:
            v_t = torch.from_numpy(v_pool.astype(np.float32)).to(torch.float8_e4m3fn)
            v_bits = v_t.view(torch.uint8).numpy()
            v_val = v_t.to(torch.float64).numpy() * sigma_pool.astype(np.float32).astype(
                np.float64)[:, :, None, None]
    else:
        k_bits = k_pool.astype(np.float32)
        k_val = k_bits.astype(np.float64)
        if v_pool is not None:
            v_bits = v_pool.astype(np.float32)
            v_val = v_bits.astype(np.float64)
    q32 = rng.standard_normal((batch, q_len * hq, dqk)).astype(np.float32)
    if kv_dtype in ("bf16", "fp8"):
        q_t = torch.from_numpy(q32).to(torch.bfloat16)
        q_store = q_t.view(torch.int16).numpy().view(np.uint16)
        q_val = q_t.to(torch.float64).numpy()
        q_dtype = "bf16"
    else:
        q_store, q_val, q_dtype = q32, q32.astype(np.float64), "f32"
    off = 0
    contiguous = []
    for b in range(batch):
        ids = perm[off:off + nb[b]]
        off += nb[b]
        table[b, :nb[b]] = ids
        L = int(lens[b])
        kc = k_val[ids].reshape((nb[b] * bs,) + k_val.shape[2:])[:L]
        if kind == "gqa":
            vc = v_val[ids].reshape((nb[b] * bs,) + v_val.shape[2:])[:L]
        else:
            kc = kc[:, None, :]
            vc = kc[:, :, :dv]
        contiguous.append((q_val[b], kc, vc))
    spec = SimpleNamespace(kind=kind, batch=batch, num_q_heads=hq, num_kv_heads=hkv,
                           qk_dim=dqk, v_dim=dv, block_size=bs, kv_dtype=kv_dtype,
                           q_dtype=q_dtype,
                           softmax_scale=(1.0 / math.sqrt(dqk)) if scale is None else scale,
                           num_shards=1, q_len=q_len)
    w = SimpleNamespace(spec=spec, seq_lens=lens, block_table=table, q=q_store,
                        k_cache=k_bits, v_cache=(v_bits if kind == "gqa" else None),
                        kv_scale=(sigma_pool.astype(np.float32) if kv_dtype == "fp8" else None))
    return w, contiguous


def sdpa(q, k, v, scale):
    """torch scaled_dot_product_attention (float64, CPU) for one query token.

    q [Hq, d], k [L, Hkv, d], v [L, Hkv, dv]; GQA via torch's enable_gqa
    (query head h reads KV head h // (Hq / Hkv)). Also returns the
    log-sum-exp from torch.logsumexp over the same scaled scores.
    """
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k)).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(np.ascontiguousarray(v)).permute(1, 0, 2)[None].contiguous()
    hq, hkv = q.shape[0], k.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, scale=scale, enable_gqa=(hq != hkv))[0, :, 0, :]
    krep = kt[0].repeat_interleave(hq // hkv, dim=0)  # [Hq, L, d]
    s = scale * torch.bmm(krep, qt[0, :, 0, :, None])[..., 0]
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


def _close(a, b, rtol, atol=0.0):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.allclose(a, b, rtol=rtol, atol=atol, equal_nan=False), \
        float(np.max(np.abs(a - b)))


# ----------------------------------------------------------------- codecs
def check_codec_e4m3(O):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # Format definition spot values: 0x38 = 1.0, 0x7E = 448 (max), 0x01 = 2^-9.
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9
    assert got[0xB8] == -1.0 and nan[0x7F] and nan[0xFF]


def check_codec_bf16(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x3F80] == 1.0 and got[0xC000] == -2.0


# ----------------------------------------------------------------- ownership / remap
def check_ownership_worked_example(O):
    g = _golden("ownership_worked_example.json")
    d = g["num_shards"]
    for r, blocks in g["shard_blocks"].items():
        got = O.shard_blocks(4 * len(blocks), 1, d, int(r))
        assert got == blocks, (r, got)
    for item in g["global_to_local"]:
        assert O.owner_of_block(item["global"], d) == item["shard"]
        assert O.local_index_of_block(item["global"], d) == item["local"]
    # A table whose physical ids equal 1000 + logical index: entry [shard, b, local].
    table = (1000 + np.arange(16, dtype=np.int32))[None, :]
    local, _ = O.remap_block_table(table, np.array([16]), 1, d)
    for item in g["global_to_local"]:
        assert local[item["shard"], 0, item["local"]] == 1000 + item["global"]
    counts = O.local_lengths(g["pool_blocks"], 1, d)
    assert counts == [g["blocks_per_shard"]] * d
    for r, pos in g["positions_one_token_blocks"].items():
        got = list(O.shard_positions(4 * len(pos), 1, d, int(r)))
        assert got == pos, (r, got)


def check_even_split(O):
    g = _golden("even_split.json")
    got = O.local_lengths(g["seq_len"], g["block_size"], g["num_shards"])
    assert got == [g["tokens_per_shard"]] * g["num_shards"], got


def check_remap_ragged(O):
    g = _golden("remap_ragged.json")
    local, lens = O.remap_block_table(np.array([g["block_table"]], dtype=np.int32),
                                      np.array([g["seq_len"]]), g["block_size"], g["num_shards"])
    assert local[:, 0, :].tolist() == g["local_tables"], local[:, 0, :].tolist()
    assert lens[:, 0].tolist() == g["local_lens"], lens[:, 0].tolist()


def _local_len_closed_form(L, bs, d, r):
    nb = -(-L // bs)
    n_r = max(0, -(-(nb - r) // d))
    owner_last = (nb - 1) % d if nb > 0 else -1
    return n_r * bs - (nb * bs - L if owner_last == r else 0)


def check_ownership_bruteforce(O):
    for bs in (1, 2, 3, 16, 64):
        for d in range(1, 10):
            for L in list(range(0, 70)) + [97, 128, 255, 299]:
                nb = O.blocks_of(L, bs)
                seen = []
                for r in range(d):
                    seen.extend(O.shard_blocks(L, bs, d, r))
                assert sorted(seen) == list(range(nb)), (L, bs, d)
                lens = O.local_lengths(L, bs, d)
                assert sum(lens) == L
                for r in range(d):
                    assert lens[r] == _local_len_closed_form(L, bs, d, r), (L, bs, d, r)
                    assert len(O.shard_positions(L, bs, d, r)) == lens[r]
    rng = np.random.default_rng(7)
    for d in (1, 2, 3, 4, 8, 9):
        lens = rng.integers(0, 200, size=5)
        bs = 16
        mb = max(1, -(-int(lens.max()) // bs)) + 2
        table = rng.permutation(10000)[: 5 * mb].reshape(5, mb).astype(np.int32)
        local, llen = O.remap_block_table(table, lens, bs, d)
        assert local.shape == (d, 5, -(-mb // d))
        for b in range(5):
            nb = -(-int(lens[b]) // bs)
            got = sorted(int(x) for x in local[:, b, :].ravel() if x >= 0)
            assert got == sorted(int(x) for x in table[b, :nb])
            for r in range(d):
                for i in range(local.shape[2]):
                    j = r + d * i
                    want = table[b, j] if j < nb else -1
                    assert local[r, b, i] == want
                assert llen[r, b] == _local_len_closed_form(int(lens[b]), bs, d, r)


def check_contiguous_worked_example(O):
    g = _golden("contiguous_split.json")
    L, bs, d = g["seq_len"], g["block_size"], g["num_shards"]
    for r, (lo, hi) in enumerate(g["token_ranges"]):
        pos = O.shard_positions(L, bs, d, r, ownership="contiguous")
        assert len(pos) == hi - lo and int(pos[0]) == lo and int(pos[-1]) == hi - 1, r
        assert bool(np.all(np.diff(pos) == 1)), r
    assert O.local_lengths(L, bs, d, ownership="contiguous") == [hi - lo for lo, hi in
                                                                  g["token_ranges"]]


def check_contiguous_bruteforce(O):
    """Contiguous ownership: shard r owns the r-th run of ceil(nb / D) blocks."""
    for bs in (1, 3, 16):
        for d in range(1, 10):
            for L in list(range(0, 70)) + [97, 255, 299]:
                nb = -(-L // bs)
                c = -(-nb // d) if nb else 0
                owners = []
                for r in range(d):
                    blocks = O.shard_blocks(L, bs, d, r, ownership="contiguous")
                    # The first c blocks go to shard 0, the next c to shard 1, ...
                    want = list(range(min(nb, r * c), min(nb, (r + 1) * c)))
                    assert blocks == want, (L, bs, d, r, blocks)
                    owners.extend([r] * len(blocks))
                    for i, j in enumerate(blocks):
                        assert O.local_index_of_block(j, d, "contiguous", nb) == i
                assert len(owners) == nb
                lens = O.local_lengths(L, bs, d, ownership="contiguous")
                assert sum(lens) == L
                for r in range(d):
                    pos = O.shard_positions(L, bs, d, r, ownership="contiguous")
                    assert len(pos) == lens[r]
                    if len(pos):
                        assert int(pos[0]) == r * c * bs and bool(np.all(np.diff(pos) == 1))
    rng = np.random.default_rng(11)
    for d in (1, 2, 3, 4, 8):
        lens = rng.integers(0, 300, size=4)
        bs = 16
        mb = max(1, -(-int(lens.max()) // bs)) + 1
        table = rng.permutation(10000)[: 4 * mb].reshape(4, mb).astype(np.int32)
        local, llen = O.remap_block_table(table, lens, bs, d, ownership="contiguous")
        for b in range(4):
            nb = -(-int(lens[b]) // bs)
            c = -(-nb // d) if nb else 0
            for r in range(d):
                row = [int(x) for x in local[r, b] if x >= 0]
                assert row == [int(x) for x in table[b, min(nb, r * c):min(nb, (r + 1) * c)]]
                assert all(int(x) == -1 for x in local[r, b, len(row):])
                tok = max(0, min(int(lens[b]), (r + 1) * c * bs) - r * c * bs)
                assert llen[r, b] == tok, (d, b, r)


def check_token_worked_example(O):
    """Token-level interleave against the positions of the practice page's section 3.4."""
    g = _golden("token_interleave.json")
    d, bs, L = g["num_shards"], g["block_size"], g["seq_len"]
    for r, want in g["positions"].items():
        got = [int(x) for x in O.shard_positions(L, bs, d, int(r), ownership="token")]
        assert got == want, (r, got)
        for p in want:
            assert O.owner_of_token(p, d) == int(r)
    for e in g["local_index"]:
        assert O.owner_of_token(e["position"], d) == e["shard"]
        assert O.local_index_of_token(e["position"], d) == e["local"]
    assert O.local_lengths(L, bs, d, ownership="token") == [len(v) for v in g["positions"].values()]


def check_token_bruteforce(O):
    """Token-level interleave: every position owned exactly once, local indices
    counting the shard's tokens in order, and lengths summing to L."""
    for bs in (1, 5, 16, 64):
        for d in range(1, 10):
            for L in list(range(0, 70)) + [97, 128, 255, 299]:
                owned = []
                lens = O.local_lengths(L, bs, d, ownership="token")
                assert sum(lens) == L, (L, bs, d)
                for r in range(d):
                    pos = [int(x) for x in O.shard_positions(L, bs, d, r, ownership="token")]
                    assert len(pos) == lens[r] == len(range(r, L, d)), (L, bs, d, r)
                    for k, p in enumerate(pos):
                        assert O.owner_of_token(p, d) == r
                        assert O.local_index_of_token(p, d) == k
                    assert pos == sorted(pos)
                    owned.extend(pos)
                assert sorted(owned) == list(range(L)), (L, bs, d)
    lens = np.array([0, 1, 7, 8, 9, 100, 257])
    for d in (1, 2, 3, 4, 8):
        tl = O.token_local_lengths(lens, d)
        assert tl.shape == (d, len(lens))
        for b, L in enumerate(lens):
            assert list(tl[:, b]) == [len(range(r, int(L), d)) for r in range(d)]


# ----------------------------------------------------------------- attention
def _brute(q, k, v, scale):
    """Pure-Python loops, math.exp/math.log only."""
    hq, hkv = q.shape[0], k.shape[1]
    L = k.shape[0]
    group = hq // hkv
    out = [[0.0] * v.shape[2] for _ in range(hq)]
    lse = [-math.inf] * hq
    for h in range(hq):
        g = h // group
        s = [scale * sum(float(q[h, i]) * float(k[t, g, i]) for i in range(q.shape[1]))
             for t in range(L)]
        if not s:
            continue
        z = sum(math.exp(x) for x in s)
        lse[h] = math.log(z)
        for c in range(v.shape[2]):
            out[h][c] = sum(math.exp(s[t]) / z * float(v[t, g, c]) for t in range(L))
    return np.array(out), np.array(lse)


def check_attend_bruteforce(O):
    rng = np.random.default_rng(11)
    for L in range(1, 9):
        for hq, hkv in ((4, 2), (2, 2), (3, 1)):
            q = rng.standard_normal((hq, 5))
            k = rng.standard_normal((L, hkv, 5))
            v = rng.standard_normal((L, hkv, 3))
            o, lse = O.attend(q, k, v, 0.7)
            ob, lb = _brute(q, k, v, 0.7)
            _close(o, ob, 1e-12, 1e-13)
            _close(lse, lb, 1e-12, 1e-13)


def check_attend_sdpa(O):
    rng = np.random.default_rng(12)
    for hq, hkv, d, dv, L in ((8, 2, 16, 8, 37), (6, 6, 8, 8, 20), (8, 1, 12, 12, 50),
                              (16, 4, 32, 16, 129)):
        q = rng.standard_normal((hq, d))
        k = rng.standard_normal((L, hkv, d))
        v = rng.standard_normal((L, hkv, dv))
        scale = 1.0 / math.sqrt(d) * 1.3
        o, lse = O.attend(q, k, v, scale)
        os_, ls = sdpa(q, k, v, scale)
        _close(o, os_, 1e-11, 1e-12)
        _close(lse, ls, 1e-12, 1e-12)


def check_closed_forms(O):
    rng = np.random.default_rng(13)
    # q = 0: all scores equal -> LSE = ln L, O = mean of V.
    for L in (1, 5, 64):
        k = rng.standard_normal((L, 2, 6))
        v = rng.standard_normal((L, 2, 4))
        o, lse = O.attend(np.zeros((4, 6)), k, v, 0.5)
        _close(lse, np.full(4, math.log(L)), 1e-15, 1e-15)
        _close(o[:2], np.broadcast_to(v[:, 0].mean(axis=0), (2, 4)), 1e-13, 1e-14)
        _close(o[2:], np.broadcast_to(v[:, 1].mean(axis=0), (2, 4)), 1e-13, 1e-14)
    # L = 1: O = v_0, LSE = s_0.
    q = rng.standard_normal((2, 6))
    k = rng.standard_normal((1, 1, 6))
    v = rng.standard_normal((1, 1, 4))
    o, lse = O.attend(q, k, v, 0.25)
    _close(o, np.broadcast_to(v[0, 0], (2, 4)), 1e-15)
    _close(lse, 0.25 * (q @ k[0, 0]), 1e-15)
    # L = 2: LSE = ln(e^s0 + e^s1), O = softmax-weighted pair.
    k = rng.standard_normal((2, 1, 6))
    v = rng.standard_normal((2, 1, 4))
    o, lse = O.attend(q, k, v, 0.25)
    s = 0.25 * (q @ k[:, 0].T)
    _close(lse, np.log(np.exp(s[:, 0]) + np.exp(s[:, 1])), 1e-14)
    w0 = np.exp(s[:, 0]) / (np.exp(s[:, 0]) + np.exp(s[:, 1]))
    _close(o, w0[:, None] * v[0, 0] + (1 - w0)[:, None] * v[1, 0], 1e-13)
    # One key 50 above the rest: O equals its value to ~e^-50.
    L = 40
    k = np.zeros((L, 1, 6))
    q1 = np.zeros((1, 6))
    q1[0, 0] = 1.0
    k[17, 0, 0] = 50.0
    v = rng.standard_normal((L, 1, 4))
    o, lse = O.attend(q1, k, v, 1.0)
    _close(o[0], v[17, 0], 0, 1e-19)
    # Empty: O = 0, LSE = -inf, no NaN.
    o, lse = O.attend(q, np.zeros((0, 1, 6)), np.zeros((0, 1, 4)), 1.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def check_paged_gqa_sdpa(O):
    for bs, lens, dtype in ((16, [256, 37, 1], "f32"), (3, [10, 0, 17], "f32"),
                            (16, [40, 33], "bf16")):
        w, cont = fake_workload("gqa", lens, hq=8, hkv=2, dqk=16, dv=16, bs=bs, kv_dtype=dtype,
                                seed=bs)
        o, lse = O.decode_reference(w)
        for b, (q, k, v) in enumerate(cont):
            if k.shape[0] == 0:
                assert np.all(o[b] == 0) and np.all(lse[b] == -np.inf)
                continue
            os_, ls = sdpa(q, k, v, w.spec.softmax_scale)
            _close(o[b], os_, 1e-11, 1e-12)
            _close(lse[b], ls, 1e-12, 1e-12)


def check_paged_mla_sdpa(O):
    for dtype in ("bf16", "fp8"):
        w, cont = fake_workload("mla", [70, 129, 5], hq=4, dqk=40, dv=32, bs=8, kv_dtype=dtype,
                                seed=21)
        o, lse = O.decode_reference(w)
        for b, (q, k, v) in enumerate(cont):
            os_, ls = sdpa(q, k, k[:, :, :32], w.spec.softmax_scale)
            _close(o[b], os_, 1e-11, 1e-12)
            _close(lse[b], ls, 1e-12, 1e-12)


def check_fp8_rows(O):
    w, cont = fake_workload("mla", [50, 9], hq=2, dqk=24, dv=16, bs=8, kv_dtype="fp8", seed=5)
    for b, (_, kc, _) in enumerate(cont):
        k, v = O.sequence_kv(w, b)
        _close(k, kc, 0, 0)
        _close(v, kc[:, :, :16], 0, 0)


# ----------------------------------------------------------------- sharding + merge
def _small_cases():
    yield fake_workload("gqa", [0, 1, 15, 16, 17, 100, 203], hq=8, hkv=2, dqk=16, dv=16, bs=16,
                        seed=31)[0]
    yield fake_workload("mla", [3, 64, 65, 300], hq=4, dqk=24, dv=16, bs=8, kv_dtype="bf16",
                        seed=32)[0]
    yield fake_workload("gqa", [7, 29], hq=4, hkv=4, dqk=8, dv=8, bs=1, seed=33)[0]


def check_shard_merge_equals_unsharded(O):
    for w in _small_cases():
        o_ref, lse_ref = O.decode_reference(w)
        for d in range(1, 10):
            op, lp = O.shard_partials(w, d)
            o, lse = O.lse_merge(op, lp)
            _close(o, o_ref, 1e-12, 1e-13)
            _close(lse, lse_ref, 1e-12, 1e-13)
            # The merged result does not depend on which shard owns which token.
            for own in ("contiguous", "token"):
                op2, lp2 = O.shard_partials(w, d, ownership=own)
                o2, lse2 = O.lse_merge(op2, lp2)
                _close(o2, o_ref, 1e-12, 1e-13)
                _close(lse2, lse_ref, 1e-12, 1e-13)
            m, l, ou = O.ml_partials(w, d)
            o2, lse2 = O.ml_merge(m, l, ou)
            _close(o2, o, 1e-12, 1e-13)
            _close(lse2, lse, 1e-12, 1e-13)


def check_merge_invariants(O):
    rng = np.random.default_rng(41)
    p, b, h, dv = 6, 3, 4, 5
    o = rng.standard_normal((p, b, h, dv))
    lse = rng.standard_normal((p, b, h)) * 3
    lse[2, 0, 1] = -np.inf
    base_o, base_l = O.lse_merge(o, lse)
    perm = rng.permutation(p)
    po, pl = O.lse_merge(o[perm], lse[perm])
    _close(po, base_o, 1e-14, 1e-15)
    _close(pl, base_l, 1e-14, 1e-15)
    # An empty partial (LSE = -inf) is the identity, exactly.
    eo = np.concatenate([o, rng.standard_normal((1, b, h, dv))])
    el = np.concatenate([lse, np.full((1, b, h), -np.inf)])
    xo, xl = O.lse_merge(eo, el)
    assert np.array_equal(xo, base_o) and np.array_equal(xl, base_l)
    # Associativity.
    ao, al = O.lse_merge(o[:2], lse[:2])
    co, cl = O.lse_merge(np.concatenate([ao[None], o[2:]]), np.concatenate([al[None], lse[2:]]))
    _close(co, base_o, 1e-13, 1e-14)
    _close(cl, base_l, 1e-13, 1e-14)
    # The merge formula on one element, written out: weights exp(LSE_i)/sum exp(LSE_j).
    wts = np.exp(lse[:, 1, 2]) / np.exp(lse[:, 1, 2]).sum()
    _close(base_o[1, 2], (wts[:, None] * o[:, 1, 2]).sum(axis=0), 1e-13, 1e-14)
    _close(base_l[1, 2], math.log(np.exp(lse[:, 1, 2]).sum()), 1e-14)
    # All partials empty: O = 0, LSE = -inf.
    zo, zl = O.lse_merge(o[:, :1], np.full((p, 1, h), -np.inf))
    assert np.all(zo == 0) and np.all(zl == -np.inf)


# ----------------------------------------------------------------- multi-token decode
def _sdpa_causal(q, k, v, scale, n):
    """torch SDPA (float64) of n query tokens [n, Hq, d] against L positions with the
    bottom-right causal mask built by torch.tril: query t sees p <= t + L - n."""
    L = k.shape[0]
    hq, hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(np.ascontiguousarray(q)).permute(1, 0, 2)[None].contiguous()
    kt = torch.from_numpy(np.ascontiguousarray(k)).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(np.ascontiguousarray(v)).permute(1, 0, 2)[None].contiguous()
    mask = torch.ones((n, L), dtype=torch.bool).tril(diagonal=L - n)
    seen = mask.any(dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=(hq != hkv))[0]  # [Hq, n, dv]
    krep = kt[0].repeat_interleave(hq // hkv, dim=0)  # [Hq, L, d]
    s = scale * torch.matmul(qt[0], krep.transpose(1, 2).contiguous())  # [Hq, n, L]
    s = s.masked_fill(~mask[None], float("-inf"))
    lse = torch.logsumexp(s, dim=-1)  # [Hq, n]
    o = torch.where(seen[None, :, None], o, torch.zeros_like(o))
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


def check_mtp_causal_sdpa(O):
    for kind, dtype, hq, hkv, n in (("mla", "bf16", 4, 1, 3), ("gqa", "f32", 4, 2, 4),
                                    ("mla", "fp8", 2, 1, 2)):
        dqk, dv = (24, 16) if kind == "mla" else (16, 16)
        w, cont = fake_workload(kind, [40, 5, 9, 17], hq=hq, hkv=hkv, dqk=dqk, dv=dv, bs=4,
                                kv_dtype=dtype, seed=41, q_len=n)
        o, lse = O.decode_reference(w)
        for b, (q, k, v) in enumerate(cont):
            os_, ls = _sdpa_causal(q.reshape(n, hq, dqk), k, v, w.spec.softmax_scale, n)
            _close(o[b].reshape(n, hq, dv), os_, 1e-11, 1e-12)
            _close(lse[b].reshape(n, hq), ls, 1e-12, 1e-12)


def check_mtp_closed_form(O):
    """L == q_len: query t sees exactly positions 0..t; query 0 sees one token, so its
    output is that token's value and its LSE is that token's score."""
    w, cont = fake_workload("gqa", [3, 1], hq=2, hkv=1, dqk=8, dv=8, bs=2, seed=43, q_len=3)
    o, lse = O.decode_reference(w)
    q, k, v = cont[0]
    _close(o[0, 0:2], np.repeat(v[0], 2, axis=0), 1e-15, 0)
    _close(lse[0, 0:2], w.spec.softmax_scale * (q[0:2] @ k[0, 0]), 1e-14, 0)
    # Sequence of one cached token with three queries: only query 2 sees it.
    assert np.all(lse[1, 0:4] == -np.inf) and np.all(o[1, 0:4] == 0)
    _close(o[1, 4:6], np.repeat(cont[1][2][0], 2, axis=0), 1e-15, 0)


def check_mtp_shard_merge(O):
    for kind, lens in (("mla", [40, 5, 2, 17, 64]), ("gqa", [33, 8, 1, 20])):
        dqk, dv, hkv = (24, 16, 1) if kind == "mla" else (16, 16, 2)
        w, _ = fake_workload(kind, lens, hq=4, hkv=hkv, dqk=dqk, dv=dv, bs=4,
                             kv_dtype="bf16" if kind == "mla" else "f32", seed=44, q_len=3)
        o_ref, lse_ref = O.decode_reference(w)
        for d in range(1, 7):
            op, lp = O.shard_partials(w, d)
            o, lse = O.lse_merge(op, lp)
            _close(o, o_ref, 1e-12, 1e-13)
            _close(lse, lse_ref, 1e-12, 1e-13)


# ----------------------------------------------------------------- fp8 encode and KV append
def _nearest_code_bruteforce(y, codes, vals):
    """Nearest finite code to y by search; ties to the even code (mantissa bit 0)."""
    a = min(abs(y), 448.0)
    best = None
    for c, v in zip(codes, vals):
        if (c >> 7) or v < 0:
            continue
        dist = abs(v - a)
        if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0):
            best = (dist, c)
    return best[1] | (0x80 if math.copysign(1.0, y) < 0 else 0)


def check_e4m3_encoder(O):
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = [float(x) for x in O.e4m3_to_f64(np.array(codes, dtype=np.uint8))]
    # Every finite code is reproduced from its own value (including -0 -> 0x80).
    got = O.f64_to_e4m3(np.array(vals))
    assert got.tolist() == codes
    # Midpoints between neighbours, values just off them, out-of-range values.
    pos = sorted(set(v for v in vals if v >= 0))
    probes = [0.0, -0.0, 1e-30, -1e-30, 449.0, 463.9, 464.0, 1e6, -1e6, 2.0 ** -10, 2.0 ** -11]
    for lo, hi in zip(pos, pos[1:]):
        mid = 0.5 * (lo + hi)
        probes += [mid, -mid, mid * (1 + 2 ** -30), mid * (1 - 2 ** -30), lo + 0.3 * (hi - lo)]
    rng = np.random.default_rng(3)
    probes += list(rng.standard_normal(300) * np.exp2(rng.integers(-12, 9, 300)))
    got = O.f64_to_e4m3(np.array(probes))
    for y, c in zip(probes, got.tolist()):
        assert c == _nearest_code_bruteforce(y, codes, vals), (y, c)
    # torch's float8_e4m3fn cast (round to nearest even) on clipped random values.
    x = np.clip(rng.standard_normal(20000).astype(np.float32) * 60, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.f64_to_e4m3(x.astype(np.float64)), ref)


def check_quantize_token(O):
    rng = np.random.default_rng(4)
    for n in (1, 7, 64, 576):
        for spread in (1e-3, 1.0, 300.0):
            x = (rng.standard_normal(n) * spread).astype(np.float32)
            codes, sigma = O.quantize_token_e4m3(x)
            amax = float(np.max(np.abs(x)))
            assert sigma.dtype == np.float32 and abs(float(sigma) * 448.0 - amax) <= amax * 2 ** -23
            # The largest magnitude maps to the largest finite code.
            k = int(np.argmax(np.abs(x)))
            assert int(codes[k]) & 0x7F == 0x7E
            # Dequantised values are within half a step of the E4M3 grid:
            # relative 2^-4 for normal codes, absolute sigma * 2^-10 below 2^-6.
            deq = O.e4m3_to_f64(codes) * float(sigma)
            bound = np.maximum(np.abs(x) * 2.0 ** -4, float(sigma) * 2.0 ** -10) * (1 + 1e-6)
            assert np.all(np.abs(deq - x) <= bound), (n, spread)
            assert np.all(np.signbit(O.e4m3_to_f64(codes)) == np.signbit(x))
    codes, sigma = O.quantize_token_e4m3(np.zeros(9, dtype=np.float32))
    assert float(sigma) == 1.0 and not codes.any()
    codes, sigma = O.quantize_token_e4m3(np.array([1e-38, -5e-39], dtype=np.float32))
    assert float(sigma) == 1.0 and not codes.any()


def check_kv_append_bruteforce(O):
    rng = np.random.default_rng(6)
    bs, pool, width = 4, 40, 6
    for d in (1, 2, 3):
        lens = [0, 5, 13, 23]
        table = rng.permutation(pool)[: 4 * width].reshape(4, width).astype(np.int32)
        local, _ = O.remap_block_table(table, np.array([p + 1 for p in lens]), bs, d)
        k = rng.standard_normal((pool, bs, 2, 3)).astype(np.float32)
        v = rng.standard_normal((pool, bs, 2, 5)).astype(np.float32)
        kn = rng.standard_normal((4, 2, 3)).astype(np.float32)
        vn = rng.standard_normal((4, 2, 5)).astype(np.float32)
        for shard in [-1] + list(range(d)):
            tab = table if shard < 0 else local[shard]
            k2, v2, _ = O.kv_append(k, v, None, tab, lens, kn, vn, kv_dtype="f32", block_size=bs,
                                    num_shards=d, shard=shard)
            touched = np.zeros((pool, bs), dtype=bool)
            for b, p in enumerate(lens):
                j = p // bs
                if shard >= 0 and j % d != shard:
                    continue
                phys = table[b, j]
                assert np.array_equal(O.gather_rows(k2, table[b], [p], bs)[0], kn[b])
                assert np.array_equal(O.gather_rows(v2, table[b], [p], bs)[0], vn[b])
                touched[phys, p % bs] = True
            assert np.array_equal(k2[~touched], k[~touched])
            assert np.array_equal(v2[~touched], v[~touched])
            want = sum(1 for p in lens if shard < 0 or (p // bs) % d == shard)
            assert touched.sum() == want
    # fp8 latent rows: codes and sigma land in the slot of each position.
    lat = np.zeros((pool, bs, 8), dtype=np.uint8)
    sc = np.full((pool, bs), -1.0, dtype=np.float32)
    xn = rng.standard_normal((3, 8)).astype(np.float32)
    table = rng.permutation(pool)[:15].reshape(3, 5).astype(np.int32)
    pos = [3, 4, 17]
    lat2, _, sc2 = O.kv_append(lat, None, sc, table, pos, xn, None, kv_dtype="fp8", block_size=bs)
    for b, p in enumerate(pos):
        phys, slot = table[b, p // bs], p % bs
        deq = O.e4m3_to_f64(lat2[phys, slot]) * float(sc2[phys, slot])
        assert np.all(np.abs(deq - xn[b]) <= np.abs(xn[b]) * 2.0 ** -4 + float(sc2[phys, slot]) * 2.0 ** -10)
    assert int((sc2 != -1.0).sum()) == 3


ALL_CHECKS = [
    check_codec_e4m3,
    check_codec_bf16,
    check_ownership_worked_example,
    check_even_split,
    check_remap_ragged,
    check_ownership_bruteforce,
    check_contiguous_worked_example,
    check_contiguous_bruteforce,
    check_token_worked_example,
    check_token_bruteforce,
    check_attend_bruteforce,
    check_attend_sdpa,
    check_closed_forms,
    check_paged_gqa_sdpa,
    check_paged_mla_sdpa,
    check_fp8_rows,
    check_shard_merge_equals_unsharded,
    check_merge_invariants,
    check_mtp_causal_sdpa,
    check_mtp_closed_form,
    check_mtp_shard_merge,
    check_e4m3_encoder,
    check_quantize_token,
    check_kv_append_bruteforce,
]
