"""CPU oracle for sharded paged decode attention (test infrastructure).

This package is test infrastructure only. It is imported by the tests, by
``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``; the
library and its Python binding never import or call it.

It computes, in float64 with NumPy, exactly what the pages define:

* interleaved block ownership (block j belongs to shard j mod D) and the
  global-to-local block-table remap -- "vLLM长序列推理优化：DCP切分KV Cache原理与实战",
  sections 2.2 and 3.2; contiguous ownership (each shard one consecutive
  chunk of a sequence) -- "Efficient Decode Context Parallelism with vLLM for
  Long Context Workloads", section A2; token-level interleave (the token at
  position t on shard t mod D) -- "vLLM长序列推理优化", sections 2.2 and 3.4;
* single-token softmax attention over a paged cache, unsharded, with GQA
  head sharing and absorbed-MLA latent rows -- "Efficient Decode Context
  Parallelism with vLLM for Long Context Workloads", section A2 (Compute step);
* per-shard partial outputs with their log-sum-exp and the LSE merge
  O = sum_i exp(LSE_i) / sum_j exp(LSE_j) * O_i -- same page, summary
  section (merge equation) and A2 (AllGather + ReduceScatter step);
* the equivalent (m, l) max/sum rescale merge -- "vLLM长序列推理优化", section 2.3;
* multi-token (MTP / draft) decode: q_len query tokens per sequence at the
  last q_len positions, each seeing the positions up to its own (a reading;
  the DCP blog page lists MTP as future work in A5);
* the KV append of a decode step into the block (and shard) owning the new
  position, with E4M3 quantisation on write for fp8 caches -- "vLLM长序列推理优化",
  sections 2.2, 3.2, 3.4 and 7 (the quantisation rule is a reading).

No blocking, fusion or reordering is added beyond those definitions. Every
function is pinned by the CPU tests to closed forms, brute force, library
routines or the pages' worked examples; none is marked "parity unpinned".
"""
from .codecs import E4M3_MAX, bf16_to_f64, e4m3_to_f64, f64_to_e4m3
from .append import append_slot, kv_append, quantize_token_e4m3
from .paged import (
    OWNERSHIPS,
    blocks_of,
    chunk_of,
    gather_rows,
    local_lengths,
    owner_of_block,
    local_index_of_block,
    owner_of_token,
    local_index_of_token,
    remap_block_table,
    shard_blocks,
    token_local_lengths,
    tokens_in_block,
)
from .attention import (
    attend,
    decode_reference,
    lse_merge,
    ml_merge,
    ml_partials,
    query,
    query_positions,
    sequence_kv,
    shard_partials,
    shard_positions,
)

__all__ = [
    "E4M3_MAX",
    "f64_to_e4m3",
    "append_slot",
    "kv_append",
    "quantize_token_e4m3",
    "OWNERSHIPS",
    "chunk_of",
    "bf16_to_f64",
    "e4m3_to_f64",
    "blocks_of",
    "gather_rows",
    "local_lengths",
    "owner_of_block",
    "local_index_of_block",
    "owner_of_token",
    "local_index_of_token",
    "remap_block_table",
    "shard_blocks",
    "token_local_lengths",
    "tokens_in_block",
    "attend",
    "decode_reference",
    "lse_merge",
    "ml_merge",
    "ml_partials",
    "query",
    "query_positions",
    "sequence_kv",
    "shard_partials",
    "shard_positions",
]
