// C ABI of libdcp (declared in include/dcp.h): argument validation, workspace
// carving and the launch sequence plan -> attention -> merge on one stream.
#include <math.h>

#include <mutex>

#include "dcp_internal.hpp"

using namespace dcp;

namespace {

constexpr int32_t kVersion = 100;  // 0.1.0

// Scratch of dcp_decode_all_shards_noalloc: one static device array per GPU.
// Host code refers to it only through the device address that
// hipGetSymbolAddress returns with that GPU current (the array's name in host
// code is a host-side stand-in, not a device address), resolved once per
// device and kept here.
__device__ __align__(256) char noalloc_scratch[DCP_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the GPU that runs `stream`.
dcp_status_t noalloc_scratch_ptr(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return DCP_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DCP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return DCP_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return DCP_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return DCP_ERR_HIP;
    if (e != hipSuccess || !p) return DCP_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DCP_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elt_bytes(int32_t t) { return t == DCP_F32 ? 4 : (t == DCP_BF16 ? 2 : 1); }

bool valid_dtype(int t) { return t == DCP_F32 || t == DCP_BF16 || t == DCP_FP8_E4M3; }

// Shape and type checks shared by every attention entry point.
dcp_status_t check_desc(const dcp_attn_desc_t* d) {
  if (!d || d->struct_size < DCP_ATTN_DESC_MIN_SIZE) return DCP_ERR_INVALID_ARG;
  if (d->struct_size >= sizeof(dcp_attn_desc_t) && (d->q_len < 0 || d->q_len > 64))
    return DCP_ERR_INVALID_ARG;
  if (d->batch < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->qk_dim < 1 ||
      d->v_dim < 1 || d->block_size < 1 || d->max_blocks_per_seq < 1 || d->num_shards < 1 ||
      d->max_seq_len < 0 || d->num_cache_blocks < 0)
    return DCP_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return DCP_ERR_INVALID_ARG;
  if (!valid_dtype(d->q_dtype) || !valid_dtype(d->kv_dtype) || !valid_dtype(d->out_dtype))
    return DCP_ERR_INVALID_ARG;
  if (d->kv_kind != DCP_KV_SEPARATE && d->kv_kind != DCP_KV_LATENT) return DCP_ERR_INVALID_ARG;
  if (d->kv_kind == DCP_KV_LATENT && (d->num_kv_heads != 1 || d->v_dim > d->qk_dim))
    return DCP_ERR_INVALID_ARG;
  if (!isfinite(d->softmax_scale)) return DCP_ERR_INVALID_ARG;
  const long long cap = static_cast<long long>(d->max_blocks_per_seq) * d->block_size;
  if (d->max_seq_len > cap) return DCP_ERR_INVALID_ARG;
  if (static_cast<long long>(d->batch) * d->max_blocks_per_seq >= (1ll << 31) ||
      static_cast<long long>(d->batch) * d->num_shards >= (1ll << 24) || cap >= (1ll << 31))
    return DCP_ERR_INVALID_ARG;
  const int e = elt_bytes(d->kv_dtype);
  if (d->kv_token_stride <= 0 || d->kv_block_stride <= 0 || d->kv_head_stride < 0)
    return DCP_ERR_INVALID_ARG;
  if ((d->kv_token_stride * e) % 16 || (d->kv_block_stride * e) % 16 ||
      (d->kv_head_stride * e) % 16)
    return DCP_ERR_INVALID_ARG;
  if (d->out_dtype == DCP_FP8_E4M3) return DCP_ERR_UNSUPPORTED;
  if (d->kv_kind == DCP_KV_LATENT ? !mla_supported(d) : !gqa_supported(d))
    return DCP_ERR_UNSUPPORTED;
  return DCP_OK;
}

int groups_for(const dcp_attn_desc_t* d) {
  return d->kv_kind == DCP_KV_LATENT ? mla_groups() : gqa_groups(d);
}

dcp_status_t check_tensors(const dcp_attn_desc_t* d, const void* q, const void* k,
                           const void* v, const float* scale) {
  if (!q) return DCP_ERR_INVALID_ARG;
  // An empty cache pool may come with null cache pointers; it is never read.
  const bool pool = d->num_cache_blocks > 0;
  if (pool && !k) return DCP_ERR_INVALID_ARG;
  if (pool && d->kv_kind == DCP_KV_SEPARATE && !v) return DCP_ERR_INVALID_ARG;
  if (pool && d->kv_dtype == DCP_FP8_E4M3 && !scale) return DCP_ERR_INVALID_ARG;
  if (!aligned(q, 16) || (k && !aligned(k, 16)) || (v && !aligned(v, 16))) return DCP_ERR_INVALID_ARG;
  if (scale && !aligned(scale, 4)) return DCP_ERR_INVALID_ARG;
  return DCP_OK;
}

// What a call runs: the plan and the kernels that read it (one call), the plan
// alone, or the kernels alone on a workspace planned before.
enum class Phase { kAll, kPlan, kRun };

// scale_ts: token stride of the fp8 scales (a token-interleave view's shard
// count; else 1), scale_bs: their block stride in tokens (0: the block size).
// The attention and merge kernels read the lengths the plan counted (its copy
// in the workspace), never map.lens: a kRun call passes map.lens = null.
dcp_status_t run_attention(const dcp_attn_desc_t* d, const void* q, const void* k, const void* v,
                           const float* kv_scale, const SegMap& map, int S, const Causal& cz,
                           void* out, dcp_dtype_t out_dtype, float* lse_out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream,
                           hipEvent_t attn_begin = nullptr, hipEvent_t attn_end = nullptr,
                           int scale_ts = 1, int scale_bs = 0, Phase phase = Phase::kAll) {
  const int G = groups_for(d);
  const int rows = desc_rows(d);
  const bool seq_pieces = d->kv_kind == DCP_KV_LATENT && mla_sequence_pieces(d, scale_ts);
  const size_t need = workspace_bytes_for(S, G, d->batch, rows, d->v_dim, seq_pieces);
  SegMap m = map;
  // No cache blocks: every block id is unusable, so every sequence is empty.
  if (d->num_cache_blocks == 0) m.width = 0;
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return DCP_ERR_WORKSPACE;
  WorkspaceView ws = carve_workspace(workspace, S, G, d->batch, rows, d->v_dim, seq_pieces);
  // Fixed work per piece of a segment, in blocks (about 128 tokens' worth).
  const int seg_cost = (128 + d->block_size - 1) / d->block_size;
  const PlanSig sig{kPlanMagic, S, G, d->batch, rows, seq_pieces ? 1 : 0,
                    m.D, m.bs, m.width, m.tok_r, m.tok_D, d->v_dim};
  if (phase != Phase::kRun &&
      launch_plan(m, S, G, seg_cost, rows, seq_pieces, sig, ws, stream) != hipSuccess)
    return DCP_ERR_HIP;
  if (phase == Phase::kPlan) return DCP_OK;
  m.lens = ws.lens;  // the lengths the plan counted
  AttnLaunch L{d,  q,  k,  v, kv_scale, m, S, ws, cz, scale_bs > 0 ? scale_bs : d->block_size,
               scale_ts, sig, attn_begin, attn_end};
  hipError_t err = d->kv_kind == DCP_KV_LATENT ? launch_mla(L, stream) : launch_gqa(L, stream);
  if (err != hipSuccess) return DCP_ERR_HIP;
  if (launch_merge_pieces(m, ws, sig, G, rows, d->v_dim, out, out_dtype, lse_out, stream) !=
      hipSuccess)
    return DCP_ERR_HIP;
  return DCP_OK;
}

// Segment maps: one shard's local table (one segment per sequence), and the
// global table of all shards (segment s = sequence s / D, shard s % D).
SegMap local_map(const dcp_attn_desc_t* d, const int32_t* table, const int32_t* lens) {
  SegMap map;
  map.table = table;
  map.lens = lens;
  map.width = (d->max_blocks_per_seq + d->num_shards - 1) / d->num_shards;
  map.D = 1;
  map.bs = d->block_size;
  map.batch = d->batch;
  map.tok_r = 0;
  map.tok_D = 1;
  return map;
}
SegMap global_map(const dcp_attn_desc_t* d, const int32_t* table, const int32_t* lens) {
  SegMap map;
  map.table = table;
  map.lens = lens;
  map.width = d->max_blocks_per_seq;
  map.D = d->num_shards;
  map.bs = d->block_size;
  map.batch = d->batch;
  map.tok_r = 0;
  map.tok_D = 1;
  return map;
}

// One shard's partial over its local table. q_pos null: single-token decode
// (no mask); else the causal multi-token form with global positions
// shard + D * (local block) .
dcp_status_t shard_partial(const dcp_attn_desc_t* d, int shard, const int32_t* q_pos,
                           const void* q, const void* k_cache, const void* v_cache,
                           const float* kv_scale, const int32_t* local_block_table,
                           const int32_t* local_seq_lens, float* o_partial, float* lse_partial,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dcp_status_t st;
  if ((st = check_tensors(d, q, k_cache, v_cache, kv_scale)) != DCP_OK) return st;
  if (!local_block_table || !local_seq_lens || !o_partial || !lse_partial)
    return DCP_ERR_INVALID_ARG;
  if (!aligned(o_partial, 16)) return DCP_ERR_INVALID_ARG;
  if (d->batch == 0) return DCP_OK;
  const SegMap map = local_map(d, local_block_table, local_seq_lens);
  Causal cz{q_pos, q_pos ? desc_q_len(d) : 1, d->num_q_heads, shard, d->num_shards};
  return run_attention(d, q, k_cache, v_cache, kv_scale, map, d->batch, cz, o_partial, DCP_F32,
                       lse_partial, workspace, workspace_bytes, stream);
}

}  // namespace

extern "C" {

const char* dcp_status_str(int32_t s) {
  switch (s) {
    case DCP_OK: return "ok";
    case DCP_ERR_INVALID_ARG: return "invalid argument";
    case DCP_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
    case DCP_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case DCP_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t dcp_version(void) { return kVersion; }

size_t dcp_workspace_size(const dcp_attn_desc_t* d) {
  if (check_desc(d) != DCP_OK) return 0;
  const int G = groups_for(d);
  const int S_all = d->batch * d->num_shards;
  const bool sp = d->kv_kind == DCP_KV_LATENT && mla_sequence_pieces(d);
  const size_t a = workspace_bytes_for(S_all, G, d->batch, desc_rows(d), d->v_dim, sp);
  const size_t b = workspace_bytes_for(d->batch, G, d->batch, desc_rows(d), d->v_dim, sp);
  return a > b ? a : b;
}

dcp_status_t dcp_block_remap_ex(const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                                int32_t max_blocks, int32_t block_size, int32_t num_shards,
                                int32_t ownership, int32_t* local_block_table,
                                int32_t* local_seq_lens, hipStream_t stream) {
  if (!block_table || !seq_lens || !local_block_table || !local_seq_lens) return DCP_ERR_INVALID_ARG;
  if (batch < 1 || max_blocks < 1 || block_size < 1 || num_shards < 1) return DCP_ERR_INVALID_ARG;
  if (ownership != DCP_OWN_INTERLEAVED && ownership != DCP_OWN_CONTIGUOUS) return DCP_ERR_INVALID_ARG;
  const long long width = (max_blocks + num_shards - 1) / num_shards;
  if (static_cast<long long>(batch) * max_blocks >= (1ll << 31) ||
      width * batch * num_shards >= (1ll << 31) ||
      static_cast<long long>(max_blocks) * block_size >= (1ll << 31))
    return DCP_ERR_INVALID_ARG;
  if (launch_remap(block_table, seq_lens, batch, max_blocks, block_size, num_shards,
                   ownership == DCP_OWN_CONTIGUOUS, local_block_table, local_seq_lens,
                   stream) != hipSuccess)
    return DCP_ERR_HIP;
  return DCP_OK;
}

dcp_status_t dcp_block_remap(const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                             int32_t max_blocks, int32_t block_size, int32_t num_shards,
                             int32_t* local_block_table, int32_t* local_seq_lens,
                             hipStream_t stream) {
  return dcp_block_remap_ex(block_table, seq_lens, batch, max_blocks, block_size, num_shards,
                            DCP_OWN_INTERLEAVED, local_block_table, local_seq_lens, stream);
}

dcp_status_t dcp_block_remap_update(const int32_t* block_table, const int32_t* old_seq_lens,
                                    const int32_t* seq_lens, int32_t batch, int32_t max_blocks,
                                    int32_t block_size, int32_t num_shards,
                                    int32_t* local_block_table, int32_t* local_seq_lens,
                                    hipStream_t stream) {
  if (!block_table || !old_seq_lens || !seq_lens || !local_block_table || !local_seq_lens)
    return DCP_ERR_INVALID_ARG;
  if (batch < 1 || max_blocks < 1 || block_size < 1 || num_shards < 1) return DCP_ERR_INVALID_ARG;
  const long long width = (max_blocks + num_shards - 1) / num_shards;
  if (static_cast<long long>(batch) * max_blocks >= (1ll << 31) ||
      width * batch * num_shards >= (1ll << 31) ||
      static_cast<long long>(max_blocks) * block_size >= (1ll << 31))
    return DCP_ERR_INVALID_ARG;
  if (launch_remap_update(block_table, old_seq_lens, seq_lens, batch, max_blocks, block_size,
                          num_shards, local_block_table, local_seq_lens, stream) != hipSuccess)
    return DCP_ERR_HIP;
  return DCP_OK;
}

dcp_status_t dcp_kv_append(const dcp_attn_desc_t* d, int32_t num_tokens, const int32_t* token_seq,
                           const int32_t* positions, const void* k_new, const void* v_new,
                           int32_t new_dtype, int32_t shard, const int32_t* block_table,
                           void* k_cache, void* v_cache, float* kv_scale, hipStream_t stream) {
  const dcp_status_t st = check_desc(d);
  if (st != DCP_OK) return st;
  if (num_tokens < 0 || shard < -1 || shard >= d->num_shards) return DCP_ERR_INVALID_ARG;
  if (!valid_dtype(new_dtype)) return DCP_ERR_INVALID_ARG;
  if (d->kv_dtype == DCP_FP8_E4M3 ? (new_dtype != DCP_BF16 && new_dtype != DCP_F32)
                                  : new_dtype != d->kv_dtype)
    return DCP_ERR_UNSUPPORTED;
  if (num_tokens == 0 || d->batch == 0 || d->num_cache_blocks == 0) return DCP_OK;
  if (!positions || !block_table || !k_new || !k_cache) return DCP_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(k_cache, 16)) return DCP_ERR_INVALID_ARG;
  if (d->kv_kind == DCP_KV_SEPARATE &&
      (!v_new || !v_cache || !aligned(v_new, 16) || !aligned(v_cache, 16)))
    return DCP_ERR_INVALID_ARG;
  if (d->kv_dtype == DCP_FP8_E4M3 && (!kv_scale || !aligned(kv_scale, 4)))
    return DCP_ERR_INVALID_ARG;
  if (launch_kv_append(d, num_tokens, token_seq, positions, k_new, v_new,
                       static_cast<dcp_dtype_t>(new_dtype), shard,
                       block_table, k_cache, v_cache, kv_scale, stream) != hipSuccess)
    return DCP_ERR_HIP;
  return DCP_OK;
}

dcp_status_t dcp_decode_partial(const dcp_attn_desc_t* d, const void* q, const void* k_cache,
                                const void* v_cache, const float* kv_scale,
                                const int32_t* local_block_table, const int32_t* local_seq_lens,
                                float* o_partial, float* lse_partial, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  dcp_status_t st = check_desc(d);
  if (st != DCP_OK) return st;
  if (desc_q_len(d) > 1) return DCP_ERR_INVALID_ARG;
  return shard_partial(d, 0, nullptr, q, k_cache, v_cache, kv_scale, local_block_table,
                       local_seq_lens, o_partial, lse_partial, workspace, workspace_bytes, stream);
}

dcp_status_t dcp_decode_partial_mtp(const dcp_attn_desc_t* d, int32_t shard, const int32_t* q_pos,
                                    const void* q, const void* k_cache, const void* v_cache,
                                    const float* kv_scale, const int32_t* local_block_table,
                                    const int32_t* local_seq_lens, float* o_partial,
                                    float* lse_partial, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  dcp_status_t st = check_desc(d);
  if (st != DCP_OK) return st;
  if (shard < 0 || shard >= d->num_shards || !q_pos) return DCP_ERR_INVALID_ARG;
  return shard_partial(d, shard, q_pos, q, k_cache, v_cache, kv_scale, local_block_table,
                       local_seq_lens, o_partial, lse_partial, workspace, workspace_bytes, stream);
}

dcp_status_t dcp_decode_partial_token(const dcp_attn_desc_t* d, int32_t shard, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const float* kv_scale, const int32_t* block_table,
                                      const int32_t* seq_lens, float* o_partial,
                                      float* lse_partial, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  dcp_status_t st = check_desc(d);
  if (st != DCP_OK) return st;
  if (desc_q_len(d) > 1 || shard < 0 || shard >= d->num_shards) return DCP_ERR_INVALID_ARG;
  if ((st = check_tensors(d, q, k_cache, v_cache, kv_scale)) != DCP_OK) return st;
  if (!block_table || !seq_lens || !o_partial || !lse_partial) return DCP_ERR_INVALID_ARG;
  if (!aligned(o_partial, 16)) return DCP_ERR_INVALID_ARG;
  const int D = d->num_shards;
  if (d->block_size % D) return DCP_ERR_UNSUPPORTED;
  if (d->batch == 0) return DCP_OK;
  // Shard r's view of the cache: every global block holds bs / D of its tokens,
  // at slots r, r + D, ..., i.e. a cache of blocks of bs / D tokens whose rows
  // start r tokens in and lie D token strides apart.
  dcp_attn_desc_t v = *d;
  v.block_size = d->block_size / D;
  v.kv_token_stride = d->kv_token_stride * D;
  v.num_shards = 1;
  v.max_seq_len = (d->max_seq_len + D - 1) / D;
  const size_t shift = static_cast<size_t>(shard) * d->kv_token_stride * elt_bytes(d->kv_dtype);
  const bool pool = d->num_cache_blocks > 0;
  const void* k = pool ? static_cast<const char*>(k_cache) + shift : k_cache;
  const void* vc = pool && v_cache ? static_cast<const char*>(v_cache) + shift : v_cache;
  const float* sc = pool && kv_scale ? kv_scale + shard : kv_scale;
  SegMap map;
  map.table = block_table;
  map.lens = seq_lens;
  map.width = d->max_blocks_per_seq;
  map.D = 1;
  map.bs = v.block_size;
  map.batch = d->batch;
  map.tok_r = shard;
  map.tok_D = D;
  const Causal cz{nullptr, 1, d->num_q_heads, 0, 1};
  return run_attention(&v, q, k, vc, sc, map, d->batch, cz, o_partial, DCP_F32, lse_partial,
                       workspace, workspace_bytes, stream, nullptr, nullptr, D, d->block_size);
}

dcp_status_t dcp_lse_merge(const float* o_partials, const float* lse_partials,
                           int32_t num_partials, int32_t batch, int32_t num_heads, int32_t v_dim,
                           void* out, int32_t out_dtype, float* lse_out, hipStream_t stream) {
  if (!o_partials || !lse_partials || !out) return DCP_ERR_INVALID_ARG;
  if (num_partials < 1 || batch < 1 || num_heads < 1 || v_dim < 4) return DCP_ERR_INVALID_ARG;
  if (out_dtype != DCP_F32 && out_dtype != DCP_BF16) return DCP_ERR_INVALID_ARG;
  if (static_cast<long long>(num_partials) * batch * num_heads * v_dim >= (1ll << 40))
    return DCP_ERR_INVALID_ARG;
  if (v_dim % 4 || v_dim > 1024) return DCP_ERR_UNSUPPORTED;
  if (!aligned(o_partials, 16) || !aligned(out, out_dtype == DCP_F32 ? 16 : 8))
    return DCP_ERR_INVALID_ARG;
  if (launch_merge_partials(o_partials, lse_partials, num_partials, batch, num_heads, v_dim, out,
                            static_cast<dcp_dtype_t>(out_dtype), lse_out, stream) != hipSuccess)
    return DCP_ERR_HIP;
  return DCP_OK;
}

dcp_status_t dcp_decode_all_shards(const dcp_attn_desc_t* d, const void* q, const void* k_cache,
                                   const void* v_cache, const float* kv_scale,
                                   const int32_t* block_table, const int32_t* seq_lens, void* out,
                                   float* lse_out, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return dcp_decode_all_shards_timed(d, q, k_cache, v_cache, kv_scale, block_table, seq_lens, out,
                                     lse_out, workspace, workspace_bytes, stream, nullptr, nullptr);
}

dcp_status_t dcp_decode_all_shards_noalloc(const dcp_attn_desc_t* d, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const float* kv_scale, const int32_t* block_table,
                                           const int32_t* seq_lens, void* out, float* lse_out,
                                           hipStream_t stream) {
  dcp_status_t st = check_desc(d);
  if (st != DCP_OK) return st;
  const bool sp = d->kv_kind == DCP_KV_LATENT && mla_sequence_pieces(d);
  const size_t need = workspace_bytes_for(d->batch * d->num_shards, groups_for(d), d->batch,
                                          desc_rows(d), d->v_dim, sp);
  if (need > DCP_NOALLOC_SCRATCH_BYTES) return DCP_ERR_WORKSPACE;
  void* scratch = nullptr;
  if ((st = noalloc_scratch_ptr(stream, &scratch)) != DCP_OK) return st;
  return dcp_decode_all_shards_timed(d, q, k_cache, v_cache, kv_scale, block_table, seq_lens, out,
                                     lse_out, scratch, DCP_NOALLOC_SCRATCH_BYTES, stream, nullptr,
                                     nullptr);
}

dcp_status_t dcp_decode_all_shards_timed(const dcp_attn_desc_t* d, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const float* kv_scale, const int32_t* block_table,
                                         const int32_t* seq_lens, void* out, float* lse_out,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream, hipEvent_t attn_begin,
                                         hipEvent_t attn_end) {
  dcp_status_t st = check_desc(d);
  if (st != DCP_OK) return st;
  if ((st = check_tensors(d, q, k_cache, v_cache, kv_scale)) != DCP_OK) return st;
  if (!block_table || !seq_lens || !out) return DCP_ERR_INVALID_ARG;
  if (!aligned(out, d->out_dtype == DCP_F32 ? 16 : 8)) return DCP_ERR_INVALID_ARG;
  if (d->batch == 0) return DCP_OK;
  const SegMap map = global_map(d, block_table, seq_lens);
  const Causal cz{nullptr, desc_q_len(d), d->num_q_heads, 0, 1};
  return run_attention(d, q, k_cache, v_cache, kv_scale, map, d->batch * d->num_shards, cz, out,
                       static_cast<dcp_dtype_t>(d->out_dtype), lse_out, workspace, workspace_bytes,
                       stream, attn_begin, attn_end);
}

dcp_status_t dcp_decode_partial_plan(const dcp_attn_desc_t* d, const int32_t* local_seq_lens,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const dcp_status_t st = check_desc(d);
  if (st != DCP_OK) return st;
  if (desc_q_len(d) > 1 || !local_seq_lens) return DCP_ERR_INVALID_ARG;
  if (d->batch == 0) return DCP_OK;
  const Causal cz{nullptr, 1, d->num_q_heads, 0, d->num_shards};
  return run_attention(d, nullptr, nullptr, nullptr, nullptr, local_map(d, nullptr, local_seq_lens),
                       d->batch, cz, nullptr, DCP_F32, nullptr, workspace, workspace_bytes, stream,
                       nullptr, nullptr, 1, 0, Phase::kPlan);
}

dcp_status_t dcp_decode_partial_run(const dcp_attn_desc_t* d, const void* q, const void* k_cache,
                                    const void* v_cache, const float* kv_scale,
                                    const int32_t* local_block_table, float* o_partial,
                                    float* lse_partial, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  dcp_status_t st = check_desc(d);
  if (st != DCP_OK) return st;
  if (desc_q_len(d) > 1) return DCP_ERR_INVALID_ARG;
  if ((st = check_tensors(d, q, k_cache, v_cache, kv_scale)) != DCP_OK) return st;
  if (!local_block_table || !o_partial || !lse_partial) return DCP_ERR_INVALID_ARG;
  if (!aligned(o_partial, 16)) return DCP_ERR_INVALID_ARG;
  if (d->batch == 0) return DCP_OK;
  const Causal cz{nullptr, 1, d->num_q_heads, 0, d->num_shards};
  return run_attention(d, q, k_cache, v_cache, kv_scale, local_map(d, local_block_table, nullptr),
                       d->batch, cz, o_partial, DCP_F32, lse_partial, workspace, workspace_bytes,
                       stream, nullptr, nullptr, 1, 0, Phase::kRun);
}

dcp_status_t dcp_decode_all_shards_plan(const dcp_attn_desc_t* d, const int32_t* seq_lens,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  const dcp_status_t st = check_desc(d);
  if (st != DCP_OK) return st;
  if (!seq_lens) return DCP_ERR_INVALID_ARG;
  if (d->batch == 0) return DCP_OK;
  const Causal cz{nullptr, desc_q_len(d), d->num_q_heads, 0, 1};
  return run_attention(d, nullptr, nullptr, nullptr, nullptr, global_map(d, nullptr, seq_lens),
                       d->batch * d->num_shards, cz, nullptr, DCP_F32, nullptr, workspace,
                       workspace_bytes, stream, nullptr, nullptr, 1, 0, Phase::kPlan);
}

dcp_status_t dcp_decode_all_shards_run(const dcp_attn_desc_t* d, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const float* kv_scale, const int32_t* block_table,
                                       void* out, float* lse_out, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  dcp_status_t st = check_desc(d);
  if (st != DCP_OK) return st;
  if ((st = check_tensors(d, q, k_cache, v_cache, kv_scale)) != DCP_OK) return st;
  if (!block_table || !out) return DCP_ERR_INVALID_ARG;
  if (!aligned(out, d->out_dtype == DCP_F32 ? 16 : 8)) return DCP_ERR_INVALID_ARG;
  if (d->batch == 0) return DCP_OK;
  const Causal cz{nullptr, desc_q_len(d), d->num_q_heads, 0, 1};
  return run_attention(d, q, k_cache, v_cache, kv_scale, global_map(d, block_table, nullptr),
                       d->batch * d->num_shards, cz, out, static_cast<dcp_dtype_t>(d->out_dtype),
                       lse_out, workspace, workspace_bytes, stream, nullptr, nullptr, 1, 0,
                       Phase::kRun);
}

}  // extern "C"
