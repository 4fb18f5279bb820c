// Per-step cache maintenance (gfx950): the KV write of a decode step into the
// block and shard that own the new position, with E4M3 quantisation for fp8
// latent caches, and the incremental local-table update for blocks a
// sequence gained or lost.
//
// Ownership: the token at position p lies in logical block j = p / bs, slot
// p % bs; shard j % D holds that block at local index j / D
// ("vLLM长序列推理优化：DCP切分KV Cache原理与实战", sections 2.2 and 3.2). Keys
// are stored after the rotary embedding (same page, section 3.4), so rows are
// written as given. The incremental table update maps only the blocks added
// since the last call (same page, section 6.2).
//
// fp8 rows: one float32 scale sigma = amax / 448 per token, amax being the
// row's largest magnitude, and codes = nearest E4M3 (ties to even) of
// x * (448 / amax), both quotients rounded once in float32. A row with
// amax == 0, or with 448 / amax beyond float32, is stored as zero codes with
// sigma = 1. The pages only name the FP8 KV cache (section 7); the rule is a
// reading.
#include "dcp_internal.hpp"

namespace dcp {
namespace {

constexpr float kE4m3Max = 448.0f;

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* token_seq;  // nullptr: token i belongs to sequence i
  const int32_t* positions;
  const int32_t* table;
  int32_t width;  // table row width
  int32_t batch;
  int32_t bs;
  int32_t D;
  int32_t shard;  // -1: global table; else local table of this shard
  int32_t pool;   // physical blocks in the cache
  void* k_cache;
  void* v_cache;
  float* kv_scale;
  int64_t block_stride;  // elements
  int64_t token_stride;
  int64_t head_stride;
  int32_t heads;  // rows per token (1 for latent)
  int32_t k_dim;
  int32_t v_dim;
};

// Physical block and slot receiving token i; false if it is skipped.
__device__ __forceinline__ bool append_target(const AppendArgs& a, int i, int& phys, int& slot) {
  const int s = a.token_seq ? a.token_seq[i] : i;
  if (s < 0 || s >= a.batch) return false;
  const int p = a.positions[i];
  if (p < 0) return false;
  int j = p / a.bs;
  if (a.shard >= 0) {
    if (j % a.D != a.shard) return false;
    j /= a.D;
  }
  if (j >= a.width) return false;
  phys = a.table[static_cast<size_t>(s) * a.width + j];
  if (phys < 0 || phys >= a.pool) return false;
  slot = p - (p / a.bs) * a.bs;
  return true;
}

// Rows of ELT bytes per element, copied as 16-byte vectors (row widths and
// strides are multiples of 16 bytes). One wave per token.
template <int ELT>
__global__ __launch_bounds__(64) void append_copy_kernel(AppendArgs a) {
  const int i = blockIdx.x;
  int phys, slot;
  if (!append_target(a, i, phys, slot)) return;
  const long long base = static_cast<long long>(phys) * a.block_stride +
                         static_cast<long long>(slot) * a.token_stride;
  const int kvec = a.k_dim * ELT / 16;
  const i32x4* ksrc = reinterpret_cast<const i32x4*>(a.k_new) +
                      static_cast<long long>(i) * a.heads * kvec;
  char* kdst = static_cast<char*>(a.k_cache) + base * ELT;
  for (int t = threadIdx.x; t < a.heads * kvec; t += 64) {
    const int h = t / kvec, c = t - h * kvec;
    reinterpret_cast<i32x4*>(kdst + a.head_stride * h * ELT)[c] = ksrc[t];
  }
  if (!a.v_cache) return;
  const int vvec = a.v_dim * ELT / 16;
  const i32x4* vsrc = reinterpret_cast<const i32x4*>(a.v_new) +
                      static_cast<long long>(i) * a.heads * vvec;
  char* vdst = static_cast<char*>(a.v_cache) + base * ELT;
  for (int t = threadIdx.x; t < a.heads * vvec; t += 64) {
    const int h = t / vvec, c = t - h * vvec;
    reinterpret_cast<i32x4*>(vdst + a.head_stride * h * ELT)[c] = vsrc[t];
  }
}

template <bool SRC_BF16>
__device__ __forceinline__ float load_src(const void* p, long long e) {
  if constexpr (SRC_BF16)
    return static_cast<float>(static_cast<const __bf16*>(p)[e]);
  else
    return static_cast<const float*>(p)[e];
}

// One latent row per token, quantised to E4M3 codes plus its scale. One wave
// per token; lane l handles elements l, l + 64, ...
template <bool SRC_BF16>
__global__ __launch_bounds__(64) void append_fp8_kernel(AppendArgs a) {
  const int i = blockIdx.x;
  int phys, slot;
  if (!append_target(a, i, phys, slot)) return;
  const int lane = threadIdx.x;
  const long long src0 = static_cast<long long>(i) * a.k_dim;
  float amax = 0.0f;
  for (int e = lane; e < a.k_dim; e += 64) amax = fmaxf(amax, fabsf(load_src<SRC_BF16>(a.k_new, src0 + e)));
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float inv = kE4m3Max / amax;
  const bool zero = !(amax > 0.0f) || __builtin_isinf(inv);
  const float sigma = zero ? 1.0f : amax / kE4m3Max;
  uint8_t* dst = static_cast<uint8_t*>(a.k_cache) + static_cast<long long>(phys) * a.block_stride +
                 static_cast<long long>(slot) * a.token_stride;
  for (int e = lane; e < a.k_dim; e += 64) {
    float y = zero ? 0.0f : load_src<SRC_BF16>(a.k_new, src0 + e) * inv;
    y = fminf(fmaxf(y, -kE4m3Max), kE4m3Max);
    // Hardware conversion: round to nearest even into OCP E4M3.
    dst[e] = static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFF);
  }
  if (lane == 0) a.kv_scale[static_cast<long long>(phys) * a.bs + slot] = sigma;
}

// Local tables after sequence b went from old_lens[b] to lens[b] tokens:
// entries of the blocks in between are written (or cleared to -1 if the
// sequence shrank) and every shard's token count is recomputed. One wave per
// sequence.
__global__ __launch_bounds__(64) void remap_update_kernel(const int32_t* __restrict__ table,
                                                          const int32_t* __restrict__ old_lens,
                                                          const int32_t* __restrict__ lens, int B,
                                                          int max_blocks, int bs, int D, int width,
                                                          int32_t* __restrict__ local_table,
                                                          int32_t* __restrict__ local_lens) {
  const int b = blockIdx.x;
  const long long cap = static_cast<long long>(max_blocks) * bs;
  long long Lo = old_lens[b], Ln = lens[b];
  Lo = Lo < 0 ? 0 : (Lo > cap ? cap : Lo);
  Ln = Ln < 0 ? 0 : (Ln > cap ? cap : Ln);
  const int nbo = static_cast<int>((Lo + bs - 1) / bs);
  const int nbn = static_cast<int>((Ln + bs - 1) / bs);
  const int lo = nbo < nbn ? nbo : nbn;
  const int hi = nbo < nbn ? nbn : nbo;
  for (int j = lo + static_cast<int>(threadIdx.x); j < hi; j += 64) {
    const int r = j % D, li = j / D;
    local_table[(static_cast<size_t>(r) * B + b) * width + li] =
        j < nbn ? table[static_cast<size_t>(b) * max_blocks + j] : -1;
  }
  for (int r = threadIdx.x; r < D; r += 64) {
    const int n_r = nbn > r ? (nbn - r + D - 1) / D : 0;
    const int tail = (nbn > 0 && (nbn - 1) % D == r)
                         ? static_cast<int>(static_cast<long long>(nbn) * bs - Ln)
                         : 0;
    local_lens[static_cast<size_t>(r) * B + b] = n_r * bs - tail;
  }
}

}  // namespace

hipError_t launch_kv_append(const dcp_attn_desc_t* d, int n_tokens, const int32_t* token_seq,
                            const int32_t* positions, const void* k_new, const void* v_new,
                            dcp_dtype_t new_dtype, int shard, const int32_t* table, void* k_cache,
                            void* v_cache, float* kv_scale, hipStream_t stream) {
  AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.token_seq = token_seq;
  a.positions = positions;
  a.table = table;
  a.width = shard < 0 ? d->max_blocks_per_seq
                      : (d->max_blocks_per_seq + d->num_shards - 1) / d->num_shards;
  a.batch = d->batch;
  a.bs = d->block_size;
  a.D = d->num_shards;
  a.shard = shard;
  a.pool = d->num_cache_blocks;
  a.k_cache = k_cache;
  a.v_cache = d->kv_kind == DCP_KV_SEPARATE ? v_cache : nullptr;
  a.kv_scale = kv_scale;
  a.block_stride = d->kv_block_stride;
  a.token_stride = d->kv_token_stride;
  a.head_stride = d->kv_head_stride;
  a.heads = d->kv_kind == DCP_KV_SEPARATE ? d->num_kv_heads : 1;
  a.k_dim = d->qk_dim;
  a.v_dim = d->v_dim;
  const dim3 grid(static_cast<unsigned>(n_tokens)), block(64);
  if (d->kv_dtype == DCP_FP8_E4M3) {
    if (new_dtype == DCP_BF16)
      hipLaunchKernelGGL(append_fp8_kernel<true>, grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL(append_fp8_kernel<false>, grid, block, 0, stream, a);
  } else if (d->kv_dtype == DCP_BF16) {
    hipLaunchKernelGGL(append_copy_kernel<2>, grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL(append_copy_kernel<4>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_remap_update(const int32_t* table, const int32_t* old_lens, const int32_t* lens,
                               int B, int max_blocks, int bs, int D, int32_t* local_table,
                               int32_t* local_lens, hipStream_t stream) {
  const int width = (max_blocks + D - 1) / D;
  hipLaunchKernelGGL(remap_update_kernel, dim3(static_cast<unsigned>(B)), dim3(64), 0, stream,
                     table, old_lens, lens, B, max_blocks, bs, D, width, local_table, local_lens);
  return hipGetLastError();
}

}  // namespace dcp
