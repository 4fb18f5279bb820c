"""Single-token decode attention, sharded partials and LSE merge, in float64.

Test infrastructure: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use this module.

Definitions followed (page titles, then the passage):
  * "Efficient Decode Context Parallelism with vLLM for Long Context
    Workloads", A2: each shard attends the full single-token query against
    its local KV slice and emits a local output and its log-sum-exp (LSE);
    the summary section gives the merge
        O = sum_i exp(LSE_i) / sum_j exp(LSE_j) * O_i .
  * Same page, A2: GQA shares one KV head across its group of query heads
    ("tensor broadcast"); MLA keeps one latent row per token shared by all
    query heads (one effective KV head).
  * "vLLM长序列推理优化：DCP切分KV Cache原理与实战", section 2.3: per shard
    m_i = max S_i, l_i = sum exp(S_i - m_i), O_i = exp(S_i - m_i) V_i; then
    m = max m_i, l = sum_i l_i exp(m_i - m), O = sum_i O_i exp(m_i - m) / l.
  * Same page, section 3.4: the cache holds keys after the rotary embedding
    is applied, so single-token decode needs no positions and no mask: all
    seq_len cached tokens are visible.
  * Multi-token decode (MTP / speculative drafts; named as DCP future work on
    the DCP blog page, A5, future work): a sequence carries q_len query tokens, the last
    q_len cached positions L - q_len .. L - 1. The pages give no masking
    rule; the reading used here is the usual causal one: query t (at position
    L - q_len + t) sees the positions p <= L - q_len + t. Under DCP a shard
    sees only its own blocks, so it needs the global position of each local
    token (block j of the sequence holds positions j*bs .. j*bs + bs - 1).

Readings where the pages are silent: scores are softmax_scale * q.k with the
scale a runtime argument; LSE is the natural log over the scaled scores;
partial outputs are normalised (O_i = sum_t softmax_t v_t); query head h
uses KV head h // (Hq / Hkv); an empty token set gives O = 0, LSE = -inf and
merge weight 0. In the absorbed-MLA form the score is taken over all
qk_dim latent columns and the value is the first v_dim columns.
"""
import numpy as np

from .codecs import bf16_to_f64, e4m3_to_f64
from .paged import gather_rows, owner_of_block, owner_of_token, blocks_of, tokens_in_block


def attend(q, k, v, scale):
    """Softmax attention of one query token per head.

    q [Hq, dqk], k [L, Hkv, dqk], v [L, Hkv, dv]  (float64)
    Returns O [Hq, dv] (normalised) and LSE [Hq] = ln sum_t exp(s_t).
    The max-shifted form below is the same quantity: exp(s - m) / sum exp(s - m)
    equals exp(s) / sum exp(s) for any common m.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq = q.shape[0]
    n, hkv = k.shape[0], k.shape[1]
    dv = v.shape[2]
    group = hq // hkv
    out = np.zeros((hq, dv))
    lse = np.full(hq, -np.inf)
    if n == 0:
        return out, lse
    for g in range(hkv):
        heads = slice(g * group, (g + 1) * group)
        s = scale * (q[heads] @ k[:, g, :].T)  # [group, L]
        m = s.max(axis=1, keepdims=True)
        lse_g = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
        p = np.exp(s - lse_g[:, None])
        out[heads] = p @ v[:, g, :]
        lse[heads] = lse_g
    return out, lse


def _decode(values, dtype):
    if dtype == "f32":
        return np.asarray(values, dtype=np.float64)
    if dtype == "bf16":
        return bf16_to_f64(values)
    if dtype == "fp8":
        return e4m3_to_f64(values)
    raise ValueError(dtype)


def query(w, b):
    """Queries of sequence b as float64 [q_len * Hq, qk_dim], token-major."""
    return _decode(w.q[b], w.spec.q_dtype)


def query_positions(w, b):
    """Positions of the q_len query tokens of sequence b: L - q_len + t."""
    n = w.spec.q_len
    return [int(w.seq_lens[b]) - n + t for t in range(n)]


def sequence_kv(w, b, positions=None):
    """De-paged K and V of sequence b at the given token positions, float64.

    GQA: K [n, Hkv, qk_dim] and V [n, Hkv, v_dim] from their own caches.
    MLA: K [n, 1, qk_dim] is the latent row and V [n, 1, v_dim] its first
    v_dim columns. fp8 rows are decode(code) times the token's scale.
    """
    spec = w.spec
    bs = spec.block_size
    if positions is None:
        positions = np.arange(int(w.seq_lens[b]))
    row = w.block_table[b]
    k = _decode(gather_rows(w.k_cache, row, positions, bs), spec.kv_dtype)
    if spec.kv_dtype == "fp8":
        sigma = gather_rows(w.kv_scale, row, positions, bs).astype(np.float64)
        k = k * sigma.reshape((-1,) + (1,) * (k.ndim - 1))
    if spec.kind == "gqa":
        v = _decode(gather_rows(w.v_cache, row, positions, bs), spec.kv_dtype)
        if spec.kv_dtype == "fp8":
            v = v * sigma.reshape((-1,) + (1,) * (v.ndim - 1))
        return k, v
    k = k[:, None, :]
    return k, k[:, :, : spec.v_dim]


def decode_reference(w, batch_indices=None):
    """Unsharded attention for every (b, t, h): O [B, q_len * Hq, v_dim],
    LSE [B, q_len * Hq]; query t sees the positions up to its own.

    Rows of sequences not in ``batch_indices`` are left as NaN.
    """
    spec = w.spec
    hq, n = spec.num_q_heads, spec.q_len
    bsel = range(spec.batch) if batch_indices is None else batch_indices
    out = np.full((spec.batch, n * hq, spec.v_dim), np.nan)
    lse = np.full((spec.batch, n * hq), np.nan)
    for b in bsel:
        k, v = sequence_kv(w, b)  # row i holds position i
        q = query(w, b)
        for t, p in enumerate(query_positions(w, b)):
            rows = slice(t * hq, (t + 1) * hq)
            seen = max(0, p + 1)
            out[b, rows], lse[b, rows] = attend(q[rows], k[:seen], v[:seen], spec.softmax_scale)
    return out, lse


def shard_positions(seq_len, block_size, num_shards, shard, ownership="interleaved"):
    """Token positions held by ``shard``: the tokens of its owned blocks (or,
    under token-level interleave, the tokens it owns one by one)."""
    if ownership == "token":
        return np.asarray([t for t in range(int(seq_len)) if owner_of_token(t, num_shards) == shard],
                          dtype=np.int64)
    pos = []
    nb = blocks_of(seq_len, block_size)
    for j in range(nb):
        if owner_of_block(j, num_shards, ownership, nb) == shard:
            start = j * block_size
            pos.extend(range(start, start + tokens_in_block(j, seq_len, block_size)))
    return np.asarray(pos, dtype=np.int64)


def shard_partials(w, num_shards=None, batch_indices=None, ownership="interleaved",
                   q_pos=None):
    """Per-shard partial (O_r, LSE_r): [D, B, q_len * Hq, v_dim] and [D, B, q_len * Hq].

    Query t of sequence b sees the shard's positions p <= q_pos[b] + t
    (default q_pos[b] = L_b - q_len, the last q_len cached positions).
    """
    spec = w.spec
    hq, n = spec.num_q_heads, spec.q_len
    d = spec.num_shards if num_shards is None else num_shards
    bsel = range(spec.batch) if batch_indices is None else batch_indices
    out = np.full((d, spec.batch, n * hq, spec.v_dim), np.nan)
    lse = np.full((d, spec.batch, n * hq), np.nan)
    for b in bsel:
        q = query(w, b)
        qp = query_positions(w, b) if q_pos is None else [int(q_pos[b]) + t for t in range(n)]
        for r in range(d):
            pos = shard_positions(int(w.seq_lens[b]), spec.block_size, d, r, ownership)
            k, v = sequence_kv(w, b, pos)
            for t, p in enumerate(qp):
                rows = slice(t * hq, (t + 1) * hq)
                keep = pos <= p
                out[r, b, rows], lse[r, b, rows] = attend(q[rows], k[keep], v[keep],
                                                          spec.softmax_scale)
    return out, lse


def lse_merge(o_parts, lse_parts):
    """Merge P partials: O = sum_i exp(LSE_i) / sum_j exp(LSE_j) * O_i.

    o_parts [P, ..., dv], lse_parts [P, ...]. Returns (O, LSE) with
    LSE = ln sum_j exp(LSE_j). The common factor exp(-max_j LSE_j) is taken
    out of numerator and denominator (it cancels). Partials with LSE = -inf
    get weight 0; if all are -inf the result is O = 0, LSE = -inf.
    """
    o = np.asarray(o_parts, dtype=np.float64)
    lse = np.asarray(lse_parts, dtype=np.float64)
    top = lse.max(axis=0)
    live = np.isfinite(top)
    shift = np.where(live, top, 0.0)
    e = np.exp(lse - shift)  # exp(-inf) = 0
    denom = e.sum(axis=0)
    weight = e / np.where(live, denom, 1.0)
    merged = (weight[..., None] * o).sum(axis=0)
    merged = np.where(live[..., None], merged, 0.0)
    lse_out = np.where(live, shift + np.log(np.where(live, denom, 1.0)), -np.inf)
    return merged, lse_out


def ml_partials(w, num_shards=None, batch_indices=None):
    """Per-shard (m_i, l_i, unnormalised O_i), section 2.3 of the DCP practice page.

    m [D, B, Hq], l [D, B, Hq], O [D, B, Hq, v_dim]; an empty shard has
    m = -inf, l = 0, O = 0.
    """
    spec = w.spec
    if spec.q_len != 1:
        raise ValueError("the (m, l) form here covers single-token decode")
    d = spec.num_shards if num_shards is None else num_shards
    bsel = range(spec.batch) if batch_indices is None else batch_indices
    hq, hkv = spec.num_q_heads, spec.num_kv_heads
    group = hq // hkv
    m = np.full((d, spec.batch, hq), -np.inf)
    l = np.zeros((d, spec.batch, hq))
    o = np.zeros((d, spec.batch, hq, spec.v_dim))
    for b in bsel:
        q = query(w, b)
        for r in range(d):
            pos = shard_positions(int(w.seq_lens[b]), spec.block_size, d, r)
            if len(pos) == 0:
                continue
            k, v = sequence_kv(w, b, pos)
            for h in range(hq):
                g = h // group
                s = spec.softmax_scale * (k[:, g, :] @ q[h])
                m[r, b, h] = s.max()
                e = np.exp(s - m[r, b, h])
                l[r, b, h] = e.sum()
                o[r, b, h] = e @ v[:, g, :]
    return m, l, o


def ml_merge(m, l, o):
    """Global m = max m_i, l = sum l_i exp(m_i - m), O = sum O_i exp(m_i - m) / l.

    Returns (O, LSE = m + ln l); with no tokens at all, O = 0 and LSE = -inf.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    top = m.max(axis=0)
    live = np.isfinite(top)
    shift = np.where(live, top, 0.0)
    factor = np.exp(m - shift)
    total = (l * factor).sum(axis=0)
    safe = np.where(live, total, 1.0)
    merged = (o * factor[..., None]).sum(axis=0) / safe[..., None]
    merged = np.where(live[..., None], merged, 0.0)
    lse = np.where(live, shift + np.log(safe), -np.inf)
    return merged, lse
