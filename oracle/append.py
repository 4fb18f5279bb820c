"""KV append into the owning shard, and fp8 quantisation on write (test infrastructure).

A decode step writes the new token's cached row (K/V, or the latent row)
before attending. The token at position p of a sequence lies in logical
block j = p // bs at slot p % bs; with interleaved ownership that block is
held by shard j % D at local index j // D ("vLLM长序列推理优化：DCP切分KV Cache原理与实战",
sections 2.2 and 3.2; section 3.4 places the write after the rotary embedding,
so the row is stored as given).

fp8 caches ("FP8 KV Cache", same page, section 7) hold OCP E4M3 codes with one
float32 scale per token. The pages give no quantisation rule; the reading used
here: the scale is sigma = amax / 448 (amax the token's largest magnitude, so
that value maps to the largest finite code), each value is stored as the
nearest code of x * (448 / amax), both computed in float32. A token whose
amax is 0, or so small that 448 / amax overflows float32, is stored as all
zero codes with sigma = 1.
"""
import numpy as np

from .codecs import E4M3_MAX, bf16_to_f64, f64_to_e4m3


def quantize_token_e4m3(x):
    """One token's values (float32) -> (uint8 codes, float32 sigma)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.float32(E4M3_MAX) / amax
    if amax == 0 or not np.isfinite(inv):
        return np.zeros(x32.shape, dtype=np.uint8), np.float32(1.0)
    sigma = amax / np.float32(E4M3_MAX)
    y = x32 * inv  # float32 products
    return f64_to_e4m3(y.astype(np.float64)), np.float32(sigma)


def append_slot(position, block_size, num_shards, shard, table_row):
    """Physical (block, slot) that receives the token at ``position``, or None.

    shard < 0: ``table_row`` is the sequence's global table row and the token
    goes to logical block position // bs. shard >= 0: ``table_row`` is that
    shard's local row; the token is written only if the shard owns the block
    (block % D == shard), at local index block // D.
    """
    if position < 0:
        return None
    j = position // block_size
    if shard >= 0:
        if j % num_shards != shard:
            return None
        j = j // num_shards
    if j >= len(table_row):
        return None
    return int(table_row[j]), position % block_size


def kv_append(k_cache, v_cache, kv_scale, block_table, positions, k_new, v_new, *, kv_dtype,
              block_size, num_shards=1, shard=-1, token_seq=None):
    """Copies of (k_cache, v_cache, kv_scale) after writing every new token.

    Caches are indexed [physical block, slot, ...] in their stored form
    (float32, bf16 bit patterns as uint16, or E4M3 codes as uint8). Token i
    belongs to sequence token_seq[i] (default i) and has its rows in
    k_new[i] / v_new[i]: stored form for float32 and bf16 caches, float32 or
    bf16 bit patterns for fp8 caches (which hold one latent row, no v).
    Tokens with a negative position, a sequence outside the table, a block
    past the table's width or a physical id outside the pool are skipped.
    """
    k = np.array(k_cache, copy=True)
    v = None if v_cache is None else np.array(v_cache, copy=True)
    sc = None if kv_scale is None else np.array(kv_scale, copy=True)
    table = np.asarray(block_table)
    pool = k.shape[0]
    for i in range(len(positions)):
        s = i if token_seq is None else int(token_seq[i])
        if s < 0 or s >= table.shape[0]:
            continue
        where = append_slot(int(positions[i]), block_size, num_shards, shard, table[s])
        if where is None or not 0 <= where[0] < pool:
            continue
        phys, slot = where
        if kv_dtype == "fp8":
            row = np.asarray(k_new[i])
            x = bf16_to_f64(row) if row.dtype == np.uint16 else row.astype(np.float64)
            codes, sigma = quantize_token_e4m3(x.astype(np.float32))
            k[phys, slot] = codes
            sc[phys, slot] = sigma
        else:
            k[phys, slot] = k_new[i]
            if v is not None:
                v[phys, slot] = v_new[i]
    return k, v, sc
