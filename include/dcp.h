/*
 * dcp.h -- C ABI of libdcp: sharded paged decode attention for AMD MI355X (gfx950).
 *
 * Decode Context Parallelism shards a sequence's paged KV cache along the
 * sequence: logical block j of a sequence belongs to shard j % D
 * ("vLLM长序列推理优化：DCP切分KV Cache原理与实战", section 2.2). Each shard
 * attends the full single-token query against its own blocks and produces a
 * partial output O_i with its log-sum-exp LSE_i; the partials are combined as
 *     O = sum_i exp(LSE_i) / sum_j exp(LSE_j) * O_i
 * ("Efficient Decode Context Parallelism with vLLM for Long Context
 * Workloads", summary section, merge equation, and section A2). On one GPU the
 * D shards are D interleaved block subsets of one cache.
 *
 * Conventions for every entry point
 *  - Pointers named *_table, *_lens, q, k_cache, v_cache, kv_scale, out,
 *    o_*, lse_* and workspace are DEVICE pointers; descriptors and scalars are
 *    host values. The caller owns and allocates every buffer; the library
 *    never allocates, frees or keeps pointers after the enqueued work ends.
 *  - Every call only enqueues work on `stream` (0 = the default stream) and
 *    returns without synchronising, so calls can be captured in a HIP graph.
 *    The library keeps no mutable global state and is thread-safe, except
 *    for the static device scratch array of dcp_decode_all_shards_noalloc
 *    (one per GPU, shared by that entry point's calls). A workspace holds
 *    what the caller last planned into it (the *_plan entry points) until the
 *    next call on it.
 *  - Host-visible arguments are validated before anything is enqueued; on an
 *    error nothing is enqueued and the call returns a non-zero status.
 *    DCP_ERR_HIP reports a launch error from the HIP runtime.
 *  - Device-resident integers (block tables, lengths) are not validated.
 *    Lengths are clamped to the table width times the block size; a table
 *    entry outside [0, num_cache_blocks) is skipped (its tokens contribute
 *    nothing), so no out-of-range cache address is ever formed. A pool of
 *    num_cache_blocks = 0 is allowed (cache pointers may then be NULL) and
 *    makes every sequence empty.
 *  - seq_len counts every cached token of the sequence, including the one just
 *    written; decode attends to all of them with no mask, since keys are
 *    cached after the rotary embedding ("vLLM长序列推理优化", section 3.4).
 *  - An empty token set (seq_len 0, or a shard that owns no block) yields
 *    O = 0 and LSE = -inf; such a partial has weight 0 in every merge.
 *  - LSE values are natural logarithms of sum_t exp(softmax_scale * q.k_t).
 *  - All layouts are row-major with the last dimension contiguous.
 */
#ifndef DCP_H_
#define DCP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DCP_OK = 0,
  DCP_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad stride or alignment */
  DCP_ERR_UNSUPPORTED = 2, /* a valid combination the library has no kernel for */
  DCP_ERR_WORKSPACE = 3,   /* workspace missing or smaller than dcp_workspace_size() */
  DCP_ERR_HIP = 4          /* the HIP runtime rejected a launch */
} dcp_status_t;

typedef enum { DCP_F32 = 0, DCP_BF16 = 1, DCP_FP8_E4M3 = 2 } dcp_dtype_t;

typedef enum {
  /* Grouped-query attention: separate K and V caches [num_cache_blocks,
   * block_size, num_kv_heads, dim]; query head h reads KV head
   * h / (num_q_heads / num_kv_heads) ("tensor broadcast" of the shared head). */
  DCP_KV_SEPARATE = 0,
  /* Absorbed multi-head latent attention: one latent row of qk_dim values per
   * token [num_cache_blocks, block_size, qk_dim], shared by every query head;
   * scores use all qk_dim columns and the value is the first v_dim columns. */
  DCP_KV_LATENT = 1
} dcp_kv_kind_t;

/* Shape and types of one decode-attention layer call. Fields and arguments
 * that take one of the enumerations above are int32_t holding its value, so
 * that any value a caller stores is well defined to read (out-of-range values
 * are rejected with DCP_ERR_INVALID_ARG). */
typedef struct {
  uint32_t struct_size;      /* sizeof(dcp_attn_desc_t), for ABI versioning */
  int32_t batch;             /* B, sequences (one query token each) */
  int32_t num_q_heads;       /* Hq */
  int32_t num_kv_heads;      /* Hkv; must be 1 for DCP_KV_LATENT */
  int32_t qk_dim;            /* width of q and k (the latent width for MLA) */
  int32_t v_dim;             /* width of v and of the output */
  int32_t block_size;        /* tokens per cache block */
  int32_t max_blocks_per_seq;/* width of the global block table */
  int32_t num_shards;        /* D >= 1 */
  int32_t max_seq_len;       /* host upper bound of any seq_len (sizes the workspace) */
  int32_t num_cache_blocks;  /* physical blocks in the cache pool (>= 0) */
  int32_t kv_kind;           /* a dcp_kv_kind_t */
  int32_t q_dtype;           /* a dcp_dtype_t: DCP_F32 or DCP_BF16 */
  int32_t kv_dtype;          /* a dcp_dtype_t: DCP_F32, DCP_BF16 or DCP_FP8_E4M3 (latent only) */
  int32_t out_dtype;         /* a dcp_dtype_t, the final output of dcp_decode_all_shards:
                              * DCP_F32 or DCP_BF16 */
  float softmax_scale;       /* score = softmax_scale * q . k */
  int64_t kv_block_stride;   /* elements between cache blocks */
  int64_t kv_token_stride;   /* elements between tokens of a block */
  int64_t kv_head_stride;    /* elements between KV heads of a token (0 for latent) */
  int32_t q_len;             /* query tokens per sequence (0 or 1: single-token decode).
                              * q_len > 1 is multi-token (draft / MTP) decode: the
                              * queries are the last q_len cached positions of their
                              * sequence and query t sees the positions up to its own.
                              * q, out and partials then hold q_len * num_q_heads rows
                              * per sequence, token-major (row t * num_q_heads + h).
                              * A descriptor whose struct_size ends before this field
                              * is read as q_len = 1. At most 64. */
} dcp_attn_desc_t;

/* Smallest struct_size accepted: descriptors from before the q_len field. */
#define DCP_ATTN_DESC_MIN_SIZE offsetof(dcp_attn_desc_t, q_len)

/* Shapes and types the library has kernels for:
 *   DCP_KV_SEPARATE: q_dtype == kv_dtype in {F32, BF16}; qk_dim == v_dim in
 *     {64, 128}; num_q_heads % num_kv_heads == 0.
 *   DCP_KV_LATENT: q BF16; kv BF16, or FP8_E4M3 with kv_scale; qk_dim 576,
 *     v_dim 512; q_len * num_q_heads 16, 32 or a multiple of 64 up to 256
 *     (with q_len > 1, num_q_heads a multiple of 16). With an
 *     FP8 cache both products run on fp16 MFMAs; each head's query and each
 *     tile's probability-times-scale weights are brought into fp16's range by
 *     exact powers of two, so the query may hold any finite values and the
 *     token scales any finite non-negative values up to 2^64 (nonzero scales
 *     below 2^-64 keep less than fp16 precision in their weights). Where a
 *     sequence is split between work groups, the latent kernels hand their
 *     partial outputs to the merge as fp16, each 128-column slice scaled by a
 *     power of two (at most 2^-11 of the slice's largest magnitude per value);
 *     the merge and every output stay fp32.
 * Cache rows (the qk_dim / v_dim values of one token and head) must start on
 * a 16-byte boundary. */

/* Global block table -> per-shard local tables.
 * "vLLM长序列推理优化", sections 2.2 and 3.2: shard r keeps the blocks j with
 * j % D == r, and global block j is local block j / D there.
 *   block_table       [batch, max_blocks] int32, physical id of logical block j
 *   seq_lens          [batch] int32
 *   local_block_table [num_shards, batch, ceil(max_blocks / num_shards)] int32 (out);
 *                     entry [r, b, i] = block_table[b, r + D*i] for every owned
 *                     block, -1 elsewhere
 *   local_seq_lens    [num_shards, batch] int32 (out): tokens shard r holds of
 *                     sequence b (the last block may be partly filled)
 * Bit-exact integer work. */
dcp_status_t dcp_block_remap(const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                             int32_t max_blocks, int32_t block_size, int32_t num_shards,
                             int32_t* local_block_table, int32_t* local_seq_lens,
                             hipStream_t stream);

/* Which shard owns which logical block of a sequence.
 *   DCP_OWN_INTERLEAVED: block j on shard j % D at local index j / D
 *     ("vLLM长序列推理优化", section 2.2); the layout every decode entry point
 *     that takes a global table assumes.
 *   DCP_OWN_CONTIGUOUS: a sequence of nb blocks is cut into D runs of
 *     c = ceil(nb / D) blocks; block j on shard j / c at local index j % c
 *     (the 200K-token split over four GPUs, 0-50K on the first, in section A2
 *     of "Efficient Decode Context Parallelism with vLLM for Long Context
 *     Workloads"). The runs depend on the sequence's current length. */
typedef enum { DCP_OWN_INTERLEAVED = 0, DCP_OWN_CONTIGUOUS = 1 } dcp_ownership_t;

/* dcp_block_remap under a chosen ownership. Same arguments and output layout;
 * entry [r, b, i] is the physical id of the i-th block shard r owns of
 * sequence b. Any other ownership value is DCP_ERR_INVALID_ARG.
 * dcp_block_remap is this call with DCP_OWN_INTERLEAVED. */
dcp_status_t dcp_block_remap_ex(const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                                int32_t max_blocks, int32_t block_size, int32_t num_shards,
                                int32_t ownership /* a dcp_ownership_t */, int32_t* local_block_table,
                                int32_t* local_seq_lens, hipStream_t stream);

/* Incremental form of dcp_block_remap (interleaved ownership) for a decode
 * step: only the blocks a sequence gained or lost are remapped, as in
 * "vLLM长序列推理优化", section 6.2.
 *   local_block_table, local_seq_lens hold dcp_block_remap's output for
 *   old_seq_lens on entry and for seq_lens on return, provided block_table
 *   entries below min(old, new) block counts did not change.
 *   Entries of blocks [nb(old), nb(new)) are written from block_table; if
 *   a sequence shrank, entries of blocks [nb(new), nb(old)) become -1. Every
 *   local_seq_lens entry is recomputed. Other arguments as in dcp_block_remap.
 * Cost O(batch * num_shards + changed blocks). Bit-exact integer work. */
dcp_status_t dcp_block_remap_update(const int32_t* block_table, const int32_t* old_seq_lens,
                                    const int32_t* seq_lens, int32_t batch, int32_t max_blocks,
                                    int32_t block_size, int32_t num_shards,
                                    int32_t* local_block_table, int32_t* local_seq_lens,
                                    hipStream_t stream);

/* KV write of a decode step: stores each new token's cached row(s) in the
 * block that owns its position (sections 2.2, 3.2 and 3.4 of
 * "vLLM长序列推理优化"; keys arrive after the rotary embedding and are
 * stored as given).
 *   num_tokens  tokens to write (0 is a no-op)
 *   token_seq   [num_tokens] int32 sequence (block-table row) of each token,
 *               or NULL for token i in sequence i
 *   positions   [num_tokens] int32 position p of each token in its sequence;
 *               it goes to logical block p / block_size, slot p % block_size
 *   k_new       DCP_KV_SEPARATE: [num_tokens, num_kv_heads, qk_dim];
 *               DCP_KV_LATENT: [num_tokens, qk_dim] (16-byte aligned)
 *   v_new       [num_tokens, num_kv_heads, v_dim] for DCP_KV_SEPARATE, else ignored
 *   new_dtype   element type of k_new / v_new: desc->kv_dtype for F32 and
 *               BF16 caches (a copy); BF16 or F32 for an FP8_E4M3 cache
 *   shard       -1: block_table is the global table [batch, max_blocks_per_seq];
 *               r in [0, num_shards): block_table is shard r's local table
 *               [batch, ceil(max_blocks_per_seq / num_shards)] and only tokens
 *               whose block j satisfies j % num_shards == r are written (at
 *               local index j / num_shards), the others are skipped
 *   k_cache, v_cache, kv_scale  the cache as described by desc (written)
 * FP8 caches: per token, sigma = amax / 448 with amax the row's largest
 * magnitude, and each code is the nearest E4M3 value (ties to even) of
 * x * (448 / amax), both quotients rounded once in fp32; a row with amax 0
 * (or 448 / amax beyond fp32) is stored as zero codes with sigma = 1. Inputs
 * must be finite; rows with amax above 448 * 2^64 get a scale beyond the
 * range fp8 decoding supports. The pages name an FP8 KV cache (section 7)
 * without a rule; this one is a reading.
 * Tokens with a negative position, a sequence outside [0, batch), a block
 * past the table width or a table entry outside [0, num_cache_blocks) are
 * skipped. Two tokens for the same slot in one call race. */
dcp_status_t dcp_kv_append(const dcp_attn_desc_t* desc, int32_t num_tokens,
                           const int32_t* token_seq, const int32_t* positions, const void* k_new,
                           const void* v_new, int32_t new_dtype /* a dcp_dtype_t */, int32_t shard,
                           const int32_t* block_table, void* k_cache, void* v_cache,
                           float* kv_scale, hipStream_t stream);

/* Bytes of device workspace dcp_decode_partial and dcp_decode_all_shards need
 * for this descriptor (the larger of the two), or 0 if the descriptor is
 * invalid or unsupported. The workspace holds split partials and a small
 * work plan; it need not be initialised and may be reused between calls that
 * are ordered on one stream. */
size_t dcp_workspace_size(const dcp_attn_desc_t* desc);

/* One shard's partial attention (the "Compute" step of section A2 of the
 * DCP blog summary): attends every query head to the tokens of one shard.
 *   q                 [batch, num_q_heads, qk_dim] (q_dtype)
 *   k_cache, v_cache  cache pools as described by desc (v_cache NULL for latent)
 *   kv_scale          [num_cache_blocks, block_size] fp32 per-token scale for FP8, else NULL
 *   local_block_table [batch, ceil(max_blocks_per_seq / num_shards)] int32, this
 *                     shard's rows of dcp_block_remap's output
 *   local_seq_lens    [batch] int32, this shard's token counts
 *   o_partial         [batch, num_q_heads, v_dim] fp32 (out), normalised output
 *   lse_partial       [batch, num_q_heads] fp32 (out)
 * desc->num_shards only sizes the local table width here. desc->q_len must be
 * at most 1 (multi-token decode needs global positions: dcp_decode_partial_mtp). */
dcp_status_t dcp_decode_partial(const dcp_attn_desc_t* desc, const void* q, const void* k_cache,
                                const void* v_cache, const float* kv_scale,
                                const int32_t* local_block_table, const int32_t* local_seq_lens,
                                float* o_partial, float* lse_partial, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* One shard's partial for multi-token (draft / MTP) decode, which the DCP
 * blog page lists as future work (section A5). Query t of sequence b sits at
 * global position q_pos[b] + t and sees the positions p <= q_pos[b] + t
 * among this shard's tokens. Local block i of this shard is global block
 * shard + num_shards * i (interleaved ownership, "vLLM长序列推理优化" §2.2),
 * which gives each local token its global position.
 *   shard       this shard's index in [0, num_shards)
 *   q_pos       [batch] int32 (device): position of query 0 of each sequence
 *               (normally L_b - q_len, L_b the global length including the
 *               q_len new tokens)
 *   q           [batch, q_len, num_q_heads, qk_dim]
 *   o_partial   [batch, q_len, num_q_heads, v_dim] fp32 (out)
 *   lse_partial [batch, q_len, num_q_heads] fp32 (out); a query that sees no
 *               token of this shard gets O = 0, LSE = -inf
 * Other arguments as in dcp_decode_partial. With q_len 1 the result is that
 * of dcp_decode_partial restricted to positions <= q_pos[b]. */
dcp_status_t dcp_decode_partial_mtp(const dcp_attn_desc_t* desc, int32_t shard,
                                    const int32_t* q_pos, const void* q, const void* k_cache,
                                    const void* v_cache, const float* kv_scale,
                                    const int32_t* local_block_table,
                                    const int32_t* local_seq_lens, float* o_partial,
                                    float* lse_partial, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* One shard's partial under token-level interleave, the finer split that
 * "vLLM长序列推理优化" sets beside block-level ownership (section 2.2; its
 * section 3.4 lists rank 0 holding positions 0, 4, 8, ... at D = 4): the token
 * at position t belongs to shard t % num_shards. Every block then holds tokens
 * of every shard, so the shard reads the global table directly: within each
 * block its tokens are the slots shard, shard + D, ... (block_size must be a
 * multiple of num_shards, else DCP_ERR_UNSUPPORTED). Merging the D partials
 * with dcp_lse_merge gives the unsharded result, as under block ownership.
 *   shard       this shard's index in [0, num_shards)
 *   block_table [batch, max_blocks_per_seq] int32 (global)
 *   seq_lens    [batch] int32 (global lengths; the shard holds
 *               ceil((L - shard) / num_shards) tokens of a sequence of L)
 *   o_partial   [batch, num_q_heads, v_dim] fp32 (out)
 *   lse_partial [batch, num_q_heads] fp32 (out); a shard holding no token of
 *               a sequence gives O = 0, LSE = -inf
 * desc->q_len must be at most 1. The workspace is sized by
 * dcp_workspace_size(desc). Other arguments as in dcp_decode_partial. */
dcp_status_t dcp_decode_partial_token(const dcp_attn_desc_t* desc, int32_t shard, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const float* kv_scale, const int32_t* block_table,
                                      const int32_t* seq_lens, float* o_partial,
                                      float* lse_partial, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* LSE merge of num_partials partial results (summary section of the DCP blog
 * page, merge equation; the reweighting inside cp_lse_ag_out_rs of section A2):
 *   o_partials   [num_partials, batch, num_heads, v_dim] fp32
 *   lse_partials [num_partials, batch, num_heads] fp32 (-inf marks an empty partial;
 *                its o_partials rows are never read)
 *   out          [batch, num_heads, v_dim] of out_dtype (DCP_F32 or DCP_BF16)
 *   lse_out      [batch, num_heads] fp32, ln sum_i exp(LSE_i), or NULL */
dcp_status_t dcp_lse_merge(const float* o_partials, const float* lse_partials,
                           int32_t num_partials, int32_t batch, int32_t num_heads, int32_t v_dim,
                           void* out, int32_t out_dtype /* a dcp_dtype_t */, float* lse_out, hipStream_t stream);

/* All D shards of one layer on one GPU, fused: ownership j % D is applied on
 * the fly to the global block table, every shard's blocks are attended in
 * parallel splits, and one LSE merge over all shards and splits produces the
 * unsharded result (the whole AllGather-Q / Compute / AllGather+ReduceScatter
 * round of section A2, with the collectives replaced by on-device data).
 *   block_table [batch, max_blocks_per_seq] int32 (global), seq_lens [batch] int32
 *   out         [batch, q_len, num_q_heads, v_dim] of desc->out_dtype
 *   lse_out     [batch, q_len, num_q_heads] fp32 or NULL
 * With desc->q_len > 1 the queries are the last q_len positions of each
 * sequence (query t at seq_len - q_len + t) and each sees the positions up to
 * its own.
 * Other arguments as in dcp_decode_partial. */
dcp_status_t dcp_decode_all_shards(const dcp_attn_desc_t* desc, const void* q, const void* k_cache,
                                   const void* v_cache, const float* kv_scale,
                                   const int32_t* block_table, const int32_t* seq_lens, void* out,
                                   float* lse_out, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* dcp_decode_all_shards with timing hooks for profilers and benchmarks: the
 * same work, plus `attn_begin` / `attn_end` (events created by the caller)
 * that the attention kernel's dispatch itself records at the kernel's start
 * and end (hipExtLaunchKernel), so hipEventElapsedTime gives that kernel's
 * duration alone and no marker is queued between the kernels. Either event
 * may be NULL. */
dcp_status_t dcp_decode_all_shards_timed(const dcp_attn_desc_t* desc, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const float* kv_scale, const int32_t* block_table,
                                         const int32_t* seq_lens, void* out, float* lse_out,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream, hipEvent_t attn_begin,
                                         hipEvent_t attn_end);

/* Plan once, run per layer. A call of dcp_decode_partial or
 * dcp_decode_all_shards first plans its work (a small kernel that splits the
 * shards' blocks into equal ranges, one per work group, from the sequence
 * lengths) and then runs attention and merge. The plan depends only on the
 * descriptor's shape fields and the lengths, which every layer of a decode
 * step shares, so a model computes it once per step and runs each layer on it
 * -- as "vLLM长序列推理优化" (section 6.2) has the block-table remap computed
 * once and reused until the tables change.
 *
 * dcp_decode_partial_plan / dcp_decode_all_shards_plan write the plan for
 * `desc` and the given lengths into `workspace` (sized by
 * dcp_workspace_size(desc)), together with a copy of the lengths.
 * dcp_decode_partial_run / dcp_decode_all_shards_run then compute exactly what
 * dcp_decode_partial / dcp_decode_all_shards would for those lengths (bit for
 * bit), reading the block table, query and cache as they are at run time;
 * their other arguments are those of the unplanned calls, without the
 * lengths. Any number of runs, with any queries and caches of the same shape,
 * may follow one plan on the same workspace, in stream order.
 *
 * Ownership: the workspace holds the plan until the next plan or unplanned
 * call on it. Errors: the host checks are those of the unplanned calls. The
 * workspace records the shape its plan was made for (batch, heads, query
 * rows, v_dim, block size, table width, shard count); a run whose descriptor
 * differs in any of them, or a run on a workspace that holds no plan, reads
 * none of it and writes NaN to every output (and LSE) value instead. A run
 * after the caller changed the lengths without planning again uses the
 * planned lengths. */
dcp_status_t dcp_decode_partial_plan(const dcp_attn_desc_t* desc, const int32_t* local_seq_lens,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);
dcp_status_t dcp_decode_partial_run(const dcp_attn_desc_t* desc, const void* q, const void* k_cache,
                                    const void* v_cache, const float* kv_scale,
                                    const int32_t* local_block_table, float* o_partial,
                                    float* lse_partial, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);
dcp_status_t dcp_decode_all_shards_plan(const dcp_attn_desc_t* desc, const int32_t* seq_lens,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);
dcp_status_t dcp_decode_all_shards_run(const dcp_attn_desc_t* desc, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const float* kv_scale, const int32_t* block_table,
                                       void* out, float* lse_out, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* Bytes of the device scratch array behind dcp_decode_all_shards_noalloc. */
#define DCP_NOALLOC_SCRATCH_BYTES (64u << 20)

/* dcp_decode_all_shards for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops that must not allocate, harnesses
 * that forbid it. Same computation and arguments without the workspace; the
 * work plan and split partials go to a static device array of
 * DCP_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends (its address is resolved once per device, on the
 * first call there). The call itself allocates nothing.
 * Returns DCP_ERR_WORKSPACE when the descriptor needs more scratch than that
 * (the need is at most dcp_workspace_size(desc); the batch-64 and batch-128
 * absorbed-MLA shapes with 64 heads need about 42 and 50 MiB).
 * Every call on one GPU shares that GPU's array: calls ordered on one stream
 * are safe, calls that may overlap (other streams, other threads) race. */
dcp_status_t dcp_decode_all_shards_noalloc(const dcp_attn_desc_t* desc, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const float* kv_scale, const int32_t* block_table,
                                           const int32_t* seq_lens, void* out, float* lse_out,
                                           hipStream_t stream);

/* Static text for a status code. */
const char* dcp_status_str(int32_t status /* a dcp_status_t */);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t dcp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DCP_H_ */
