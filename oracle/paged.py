"""Paged-cache bookkeeping: block ownership, remap and gathers (test infrastructure).

Source: "vLLM长序列推理优化：DCP切分KV Cache原理与实战".
  * Section 2.2: with D shards, shard i owns the blocks whose index satisfies
    block_idx % D == i (interleaved, not contiguous).
  * Section 3.2: the block table keeps global logical indices and is remapped
    to local indices per shard; global block 4 is local block 1 on shard 0
    because shard 0 holds global blocks 0, 4, 8, ... with local indices
    counting from 0.
The block index that is interleaved is the *logical* index of a block within
its sequence (position t lives in logical block t // block_size at slot
t % block_size). The last block of a sequence may be partly filled; it
belongs to the shard that owns its index like any other block.

Contiguous ownership, the alternative the pages also describe ("Efficient
Decode Context Parallelism with vLLM for Long Context Workloads", section A2,
and the vLLM blog post it summarises: a 200K-token request over 4 GPUs, GPU 0
holding tokens 0-50K, GPU 1 50K-100K, and so on). At block granularity this
reads: the nb blocks of a sequence form D consecutive chunks of
c = ceil(nb / D) blocks, shard r owning blocks [r c, (r + 1) c) (the last
chunks may be short or empty), with local index j - r c.

Token-level interleave, the finer granularity section 2.2 of the practice
page sets beside block-level splitting; its section 3.4 gives the example
"rank 0 holds positions 0, 4, 8, ..., rank 1 holds 1, 5, 9, ..." at D = 4.
Reading: the token at position t belongs to shard t mod D, at local index
t // D, whatever the block size.
"""
import numpy as np


OWNERSHIPS = ("interleaved", "contiguous", "token")


def blocks_of(seq_len: int, block_size: int) -> int:
    """Number of logical blocks a sequence of seq_len tokens occupies."""
    return -(-int(seq_len) // int(block_size))


def chunk_of(nb: int, num_shards: int) -> int:
    """Blocks per shard under contiguous ownership: ceil(nb / D)."""
    return -(-int(nb) // int(num_shards))


def owner_of_block(j: int, num_shards: int, ownership: str = "interleaved", nb: int = 0) -> int:
    """Shard owning logical block j: j % D (section 2.2), or, contiguous,
    j // ceil(nb / D) for a sequence of nb blocks."""
    if ownership == "interleaved":
        return j % num_shards
    if ownership == "contiguous":
        return j // chunk_of(nb, num_shards)
    raise ValueError(ownership)


def local_index_of_block(j: int, num_shards: int, ownership: str = "interleaved", nb: int = 0) -> int:
    """Position of logical block j in its owner's local table (section 3.2)."""
    if ownership == "interleaved":
        return j // num_shards
    if ownership == "contiguous":
        return j - owner_of_block(j, num_shards, ownership, nb) * chunk_of(nb, num_shards)
    raise ValueError(ownership)


def owner_of_token(t: int, num_shards: int) -> int:
    """Token-level interleave: the token at position t lives on shard t mod D."""
    return t % num_shards


def local_index_of_token(t: int, num_shards: int) -> int:
    """Token-level interleave: its index among that shard's tokens."""
    return t // num_shards


def tokens_in_block(j: int, seq_len: int, block_size: int) -> int:
    """Valid tokens in logical block j of a sequence of seq_len tokens."""
    return max(0, min(block_size, seq_len - j * block_size))


def shard_blocks(seq_len: int, block_size: int, num_shards: int, shard: int,
                 ownership: str = "interleaved") -> list:
    """Logical blocks of one sequence that ``shard`` owns, in local order."""
    nb = blocks_of(seq_len, block_size)
    return [j for j in range(nb) if owner_of_block(j, num_shards, ownership, nb) == shard]


def local_lengths(seq_len: int, block_size: int, num_shards: int,
                  ownership: str = "interleaved") -> list:
    """Tokens each shard holds for one sequence, by counting its blocks (or,
    under token-level interleave, its tokens)."""
    out = [0] * num_shards
    if ownership == "token":
        for t in range(int(seq_len)):
            out[owner_of_token(t, num_shards)] += 1
        return out
    nb = blocks_of(seq_len, block_size)
    for j in range(nb):
        out[owner_of_block(j, num_shards, ownership, nb)] += tokens_in_block(j, seq_len, block_size)
    return out


def remap_block_table(block_table, seq_lens, block_size: int, num_shards: int,
                      ownership: str = "interleaved"):
    """Global block table -> per-shard local tables (section 3.2).

    block_table: int32 [B, max_blocks] of physical block ids (logical j -> id).
    Returns (local_table int32 [D, B, ceil(max_blocks / D)] padded with -1,
             local_lens  int32 [D, B]).
    Entry [r, b, i] is the physical id of the logical block j that shard r
    owns at local index i (interleaved: j % D == r and j // D == i).
    """
    table = np.asarray(block_table)
    lens = np.asarray(seq_lens)
    batch, max_blocks = table.shape
    width = -(-max_blocks // num_shards)
    local = np.full((num_shards, batch, width), -1, dtype=np.int32)
    local_len = np.zeros((num_shards, batch), dtype=np.int32)
    for b in range(batch):
        n = min(blocks_of(lens[b], block_size), max_blocks)
        for j in range(n):
            r = owner_of_block(j, num_shards, ownership, n)
            i = local_index_of_block(j, num_shards, ownership, n)
            local[r, b, i] = table[b, j]
            local_len[r, b] += tokens_in_block(j, int(lens[b]), block_size)
    return local, local_len


def token_local_lengths(seq_lens, num_shards: int):
    """Token-level interleave: int32 [D, B], the tokens shard r holds of
    sequence b. Every block carries tokens of several shards, so the global
    block table serves every shard and there is no local table."""
    lens = np.asarray(seq_lens)
    out = np.zeros((num_shards, len(lens)), dtype=np.int32)
    for b, L in enumerate(lens):
        out[:, b] = local_lengths(int(L), 1, num_shards, ownership="token")
    return out


def gather_rows(cache, table_row, positions, block_size: int):
    """Rows cache[table_row[t // bs], t % bs] for every token position t.

    ``cache`` is indexed [physical block, slot, ...]; the result keeps the
    trailing dimensions and lists rows in the order of ``positions``.
    """
    pos = np.asarray(positions, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[pos // block_size]
    return cache[phys, pos % block_size]
