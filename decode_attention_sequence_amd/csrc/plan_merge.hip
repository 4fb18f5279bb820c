// Work planning, LSE merge and block-table remap kernels (gfx950).
//
// Merge: "Efficient Decode Context Parallelism with vLLM for Long Context
// Workloads", summary section (merge equation) and A2: the partial outputs
// are reweighted by exp(LSE_i) / sum_j exp(LSE_j) and summed. Here the common
// factor exp(-max_j LSE_j) is divided out of both sums so every weight is at
// most 1, and partials with LSE = -inf (no tokens) are skipped entirely.
//
// Remap: "vLLM长序列推理优化：DCP切分KV Cache原理与实战", sections 2.2 and 3.2:
// shard r keeps global blocks j with j % D == r; global block j is local
// block j / D on that shard.
#include "dcp_internal.hpp"

namespace dcp {

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t workspace_bytes_for(int S, int G, int Hq, int v_dim) {
  size_t slots = static_cast<size_t>(S) + static_cast<size_t>(G) - 1;
  size_t off = align_up(sizeof(PlanHeader) + sizeof(int32_t) * (static_cast<size_t>(S) + 1), 256);
  off += align_up(slots * Hq * sizeof(float), 256);
  off += slots * Hq * v_dim * sizeof(float);
  return off;
}

WorkspaceView carve_workspace(void* ws, int S, int G, int Hq, int v_dim) {
  WorkspaceView v;
  char* base = static_cast<char*>(ws);
  v.num_slots = S + G - 1;
  v.header = reinterpret_cast<PlanHeader*>(base);
  v.seg_off = reinterpret_cast<int32_t*>(base + sizeof(PlanHeader));
  size_t off = align_up(sizeof(PlanHeader) + sizeof(int32_t) * (static_cast<size_t>(S) + 1), 256);
  v.lse = reinterpret_cast<float*>(base + off);
  off += align_up(static_cast<size_t>(v.num_slots) * Hq * sizeof(float), 256);
  v.o = reinterpret_cast<float*>(base + off);
  return v;
}

// ------------------------------------------------------------------ planning
__global__ __launch_bounds__(1024) void plan_kernel(SegMap m, int S, int G, PlanHeader* hdr,
                                                    int32_t* seg_off) {
  __shared__ int sums[1024];
  const int t = threadIdx.x;
  const int per = (S + 1023) / 1024;
  const int s0 = t * per;
  const int s1 = min(S, s0 + per);
  int local = 0;
  for (int s = s0; s < s1; ++s) local += segment_blocks(m, s);
  sums[t] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int v = t >= off ? sums[t - off] : 0;
    __syncthreads();
    sums[t] += v;
    __syncthreads();
  }
  int run = sums[t] - local;
  for (int s = s0; s < s1; ++s) {
    run += segment_blocks(m, s);
    seg_off[s + 1] = run;
  }
  if (t == 0) seg_off[0] = 0;
  if (t < 4) hdr->zero[t] = 0;
  if (t == 1023) {
    int total = sums[1023];
    hdr->total = total;
    hdr->chunk = max(1, (total + G - 1) / G);
  }
}

hipError_t launch_plan(const SegMap& m, int S, int G, WorkspaceView ws, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, m, S, G, ws.header, ws.seg_off);
  return hipGetLastError();
}

// ------------------------------------------------------------------ merge
// Slot sources: which stored partial rows feed output row b.
struct PieceSource {
  const int32_t* seg_off;
  const PlanHeader* hdr;
  int D;
  template <class F>
  __device__ __forceinline__ void for_each(int b, F&& f) const {
    const int chunk = hdr->chunk;
    for (int s = b * D; s < (b + 1) * D; ++s) {
      int a = seg_off[s], e = seg_off[s + 1];
      if (a >= e) continue;
      for (int g = a / chunk, g1 = (e - 1) / chunk; g <= g1; ++g) f(s + g);
    }
  }
};

struct PartialSource {
  int P, B;
  template <class F>
  __device__ __forceinline__ void for_each(int b, F&& f) const {
    for (int p = 0; p < P; ++p) f(p * B + b);
  }
};

// One thread per 4 output values; blockDim.x = heads_per_block * (v_dim / 4).
template <class Src>
__global__ __launch_bounds__(256) void merge_kernel(Src src, const float* __restrict__ o_rows,
                                                    const float* __restrict__ lse_rows, int H,
                                                    int v_dim, void* out, int out_bf16,
                                                    float* lse_out) {
  const int tph = v_dim >> 2;
  const int b = blockIdx.x;
  const int h = blockIdx.y * (blockDim.x / tph) + threadIdx.x / tph;
  const int v4 = threadIdx.x % tph;
  if (h >= H) return;
  float top = -INFINITY;
  src.for_each(b, [&](int row) {
    float l = lse_rows[static_cast<size_t>(row) * H + h];
    top = l > top ? l : top;
  });
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (top != -INFINITY) {
    src.for_each(b, [&](int row) {
      float l = lse_rows[static_cast<size_t>(row) * H + h];
      if (l == -INFINITY) return;
      float w = fast_exp2((l - top) * kLog2e);
      const f32x4 o = *reinterpret_cast<const f32x4*>(
          o_rows + (static_cast<size_t>(row) * H + h) * v_dim + 4 * v4);
      wsum += w;
      acc += w * o;
    });
    acc *= 1.0f / wsum;
  }
  const size_t oidx = (static_cast<size_t>(b) * H + h) * v_dim + 4 * v4;
  if (out_bf16) {
    uint16_t* o16 = static_cast<uint16_t*>(out) + oidx;
    uint32_t lo = f32_to_bf16_bits(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[1])) << 16);
    uint32_t hi = f32_to_bf16_bits(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[3])) << 16);
    *reinterpret_cast<i32x2*>(o16) = i32x2{static_cast<int>(lo), static_cast<int>(hi)};
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + oidx) = acc;
  }
  if (lse_out && v4 == 0) {
    lse_out[static_cast<size_t>(b) * H + h] =
        top == -INFINITY ? -INFINITY : top + fast_log2(wsum) * kLn2;
  }
}

static dim3 merge_block(int v_dim) {
  int tph = v_dim / 4;
  int hpb = tph >= 256 ? 1 : 256 / tph;
  return dim3(hpb * tph);
}

hipError_t launch_merge_pieces(const SegMap& m, const WorkspaceView& ws, int G, int Hq, int v_dim,
                               void* out, dcp_dtype_t out_dtype, float* lse_out,
                               hipStream_t stream) {
  (void)G;
  PieceSource src{ws.seg_off, ws.header, m.D};
  dim3 block = merge_block(v_dim);
  int hpb = block.x / (v_dim / 4);
  dim3 grid(m.batch, (Hq + hpb - 1) / hpb);
  hipLaunchKernelGGL(merge_kernel<PieceSource>, grid, block, 0, stream, src, ws.o, ws.lse, Hq,
                     v_dim, out, out_dtype == DCP_BF16 ? 1 : 0, lse_out);
  return hipGetLastError();
}

hipError_t launch_merge_partials(const float* o, const float* lse, int P, int B, int H, int v_dim,
                                 void* out, dcp_dtype_t out_dtype, float* lse_out,
                                 hipStream_t stream) {
  PartialSource src{P, B};
  dim3 block = merge_block(v_dim);
  int hpb = block.x / (v_dim / 4);
  dim3 grid(B, (H + hpb - 1) / hpb);
  hipLaunchKernelGGL(merge_kernel<PartialSource>, grid, block, 0, stream, src, o, lse, H, v_dim,
                     out, out_dtype == DCP_BF16 ? 1 : 0, lse_out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ remap
// One thread per local-table entry [r, b, i]; entries with i == 0 also write
// the shard's token count for sequence b.
__global__ __launch_bounds__(256) void remap_kernel(const int32_t* __restrict__ table,
                                                    const int32_t* __restrict__ lens, int B,
                                                    int max_blocks, int bs, int D, int width,
                                                    int32_t* __restrict__ local_table,
                                                    int32_t* __restrict__ local_lens) {
  const long long total = static_cast<long long>(D) * B * width;
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int i = static_cast<int>(idx % width);
  const int b = static_cast<int>((idx / width) % B);
  const int r = static_cast<int>(idx / (static_cast<long long>(width) * B));
  long long L = lens[b];
  const long long cap = static_cast<long long>(max_blocks) * bs;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int nb = static_cast<int>((L + bs - 1) / bs);
  const int j = r + D * i;
  local_table[idx] = j < nb ? table[static_cast<size_t>(b) * max_blocks + j] : -1;
  if (i == 0) {
    const int n_r = nb > r ? (nb - r + D - 1) / D : 0;
    const int tail = (nb > 0 && (nb - 1) % D == r) ? static_cast<int>(static_cast<long long>(nb) * bs - L) : 0;
    local_lens[static_cast<size_t>(r) * B + b] = n_r * bs - tail;
  }
}

hipError_t launch_remap(const int32_t* table, const int32_t* lens, int B, int max_blocks, int bs,
                        int D, int32_t* local_table, int32_t* local_lens, hipStream_t stream) {
  const int width = (max_blocks + D - 1) / D;
  const long long total = static_cast<long long>(D) * B * width;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(remap_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream,
                     table, lens, B, max_blocks, bs, D, width, local_table, local_lens);
  return hipGetLastError();
}

}  // namespace dcp
