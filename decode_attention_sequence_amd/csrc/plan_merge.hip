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

static inline size_t plan_bytes(int S, int G, int B) {
  return sizeof(PlanHeader) + sizeof(int32_t) * (2 * (static_cast<size_t>(S) + 1) +
                                                 2 * (static_cast<size_t>(G) + 1) +
                                                 3 * static_cast<size_t>(B));
}

static inline int slot_count(int S, int G, int B, bool seq_pieces) {
  return (seq_pieces ? B : S) + G - 1;
}

size_t workspace_bytes_for(int S, int G, int B, int Hq, int v_dim, bool seq_pieces) {
  size_t slots = static_cast<size_t>(slot_count(S, G, B, seq_pieces));
  size_t off = align_up(plan_bytes(S, G, B), 256);
  off += align_up(slots * Hq * sizeof(float), 256);
  off += slots * Hq * v_dim * sizeof(float);
  return off;
}

WorkspaceView carve_workspace(void* ws, int S, int G, int B, int Hq, int v_dim, bool seq_pieces) {
  WorkspaceView v;
  char* base = static_cast<char*>(ws);
  v.num_slots = slot_count(S, G, B, seq_pieces);
  v.header = reinterpret_cast<PlanHeader*>(base);
  v.seg_off = reinterpret_cast<int32_t*>(base + sizeof(PlanHeader));
  v.cost_off = v.seg_off + S + 1;
  v.wg_start = v.cost_off + S + 1;
  v.seq_slots = v.wg_start + G + 1;
  v.wg_seg = v.seq_slots + 2 * B;
  v.lens = v.wg_seg + G + 1;
  size_t off = align_up(plan_bytes(S, G, B), 256);
  v.lse = reinterpret_cast<float*>(base + off);
  off += align_up(static_cast<size_t>(v.num_slots) * Hq * sizeof(float), 256);
  v.o = reinterpret_cast<float*>(base + off);
  return v;
}

// ------------------------------------------------------------------ planning
// Stream-K split weighted by cost: a non-empty segment costs its blocks plus
// seg_cost blocks' worth of fixed work (starting a piece, storing its
// partial), so a work group whose range crosses many short segments gets
// fewer blocks. Work group g takes the blocks whose cost positions fall in
// [start(g), start(g + 1)); a segment's overhead units come before its first
// block.
// Range g runs on XCD g / (G / 8) (xcd_logical_group). On MI355X the
// Arrays the plan searches are mirrored in LDS when they fit (flat pointers
// then address LDS), else read from the workspace.
constexpr int kPlanLds = 6144;  // entries per mirrored array

// First cost position of range g (start(G) = total cost): an equal share of
// the cost per range. Below 8 cost units per range the split is in whole
// units, cc = ceil(total / G) per range, which leaves no range without cost
// units before the last block.
__device__ __forceinline__ int split_start(int total_c, int G, int g) {
  if (total_c < 8 * G) {
    const long long cc = max(1, (total_c + G - 1) / G);
    return static_cast<int>(min(static_cast<long long>(g) * cc, static_cast<long long>(total_c)));
  }
  return static_cast<int>(static_cast<long long>(total_c) * g / G);
}

// The range holding cost position y (0 <= y < total_c): the last g in [0, G)
// with split_start(g) <= y, in closed form. Whole units: g * cc <= y. Shares:
// floor(total_c * g / G) <= y exactly when total_c * g < (y + 1) * G.
__device__ __forceinline__ int range_at(int total_c, int G, int y) {
  if (total_c < 8 * G) {
    const int cc = max(1, (total_c + G - 1) / G);
    return min(G - 1, y / cc);
  }
  const long long g = ((static_cast<long long>(y) + 1) * G - 1) / total_c;
  return static_cast<int>(min(static_cast<long long>(G - 1), g));
}

__global__ __launch_bounds__(1024) void plan_kernel(SegMap m, int S, int G, int seg_cost, int Hq,
                                                    int seq_pieces, PlanHeader* hdr, int32_t* seg_off,
                                                    int32_t* cost_off, int32_t* wg_start,
                                                    int32_t* seq_slots, int32_t* wg_seg,
                                                    int32_t* lens, PlanSig sig, float* lse) {
  __shared__ int w_sum[16];
  __shared__ int w_cost[16];
  __shared__ int l_seg[kPlanLds];
  __shared__ int l_cost[kPlanLds];
  __shared__ int l_wg[kPlanLds];
  const bool mirror_s = S + 1 <= kPlanLds;
  const bool mirror_g = G + 1 <= kPlanLds;
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int per = (S + 1023) / 1024;
  const int s0 = min(S, t * per);
  const int s1 = min(S, s0 + per);
  int local = 0, local_c = 0;
  for (int s = s0; s < s1; ++s) {
    const int nb = segment_blocks(m, s);
    local += nb;
    local_c += nb + (nb > 0 ? seg_cost : 0);
  }
  // Prefix sums over the threads' counts: an inclusive scan inside each wave
  // (cross-lane moves, no barrier), then the sixteen wave totals.
  int inc = local, inc_c = local_c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(inc, off), vc = __shfl_up(inc_c, off);
    if (lane >= off) {
      inc += v;
      inc_c += vc;
    }
  }
  if (lane == 63) {
    w_sum[wv] = inc;
    w_cost[wv] = inc_c;
  }
  __syncthreads();
  int run = inc - local, run_c = inc_c - local_c, total = 0, total_c = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int ws = w_sum[i], wc = w_cost[i];
    if (i < wv) {
      run += ws;
      run_c += wc;
    }
    total += ws;
    total_c += wc;
  }
  for (int s = s0; s < s1; ++s) {
    const int nb = segment_blocks(m, s);
    run += nb;
    run_c += nb + (nb > 0 ? seg_cost : 0);
    seg_off[s + 1] = run;
    cost_off[s + 1] = run_c;
    if (mirror_s) {
      l_seg[s + 1] = run;
      l_cost[s + 1] = run_c;
    }
  }
  if (t == 0) {
    seg_off[0] = 0;
    cost_off[0] = 0;
    l_seg[0] = 0;
    l_cost[0] = 0;
  }
  if (t < 4) hdr->zero[t] = 0;
  if (t == 0) {
    hdr->total = total;
    hdr->sig = sig;
  }
  // The lengths this plan counted, for the kernels that run it.
  for (int b = t; b < m.batch; b += 1024) lens[b] = m.lens[b];
  __syncthreads();  // seg_off and cost_off complete
  const int* so = mirror_s ? l_seg : seg_off;
  const int* co = mirror_s ? l_cost : cost_off;
  // (Costs stay below 2^31: they count blocks of int32 table entries plus a
  // few units per segment, so 32-bit arithmetic suffices.)
  for (int g = t; g <= G; g += 1024) {
    const int y = split_start(total_c, G, g);
    // last segment s < S with cost_off[s] <= y
    int lo = 0, hi = S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (co[mid] <= y) lo = mid; else hi = mid;
    }
    int x = total;
    if (S > 0 && y < co[lo + 1]) {
      const long long o = y - co[lo] - seg_cost;  // blocks of segment lo before y
      x = so[lo] + static_cast<int>(max(0ll, o));
    }
    wg_start[g] = g == 0 ? 0 : x;
    if (mirror_g) l_wg[g] = g == 0 ? 0 : x;
    // The segment of the range's first block, so that a work group starts
    // without searching seg_off (ranges past the last block never read it).
    const int x0 = g == 0 ? 0 : x;
    wg_seg[g] = x0 < total ? find_segment(so, S, x0) : 0;
  }
  // The work group of block i of segment s is the range holding its cost
  // position cost_off[s] + seg_cost + i (the same split as above): the last g
  // with start(g) <= that position.
  __syncthreads();  // wg_start complete
  auto range_of = [&](unsigned y) { return range_at(total_c, G, static_cast<int>(y)); };
  if (seq_pieces) {
    // One partial per work group and sequence: sequence b's blocks (contiguous
    // over its segments) lie in work groups g0..g1, whose partials sit in slots
    // b + g0 .. b + g1. A work group in between without blocks leaves its slot
    // unwritten: it gets LSE = -inf (an empty partial).
    const int* wo = mirror_g ? l_wg : wg_start;
    for (int b = t; b < m.batch; b += 1024) {
      int s_first = -1, s_last = -1;
      for (int s = b * m.D; s < (b + 1) * m.D; ++s)
        if (so[s + 1] > so[s]) {
          if (s_first < 0) s_first = s;
          s_last = s;
        }
      int lo = 0, hi = 0;
      if (s_first >= 0) {
        const unsigned y0 = static_cast<unsigned>(co[s_first] + seg_cost);
        const unsigned y1 = static_cast<unsigned>(co[s_last] + seg_cost + (so[s_last + 1] - so[s_last]) - 1);
        const int g0 = range_of(y0);
        const int g1 = range_of(y1);
        lo = b + g0;
        hi = b + g1 + 1;
      }
      seq_slots[2 * b] = lo;
      seq_slots[2 * b + 1] = hi;
    }
    // The gaps, one thread per work group: a work group without blocks lies
    // strictly inside sequence b's range exactly when the blocks just before
    // and just after it (x - 1 and x) both belong to b.
    auto seq_of = [&](int blk) {  // last sequence starting at or before block blk
      int lo = 0, hi = m.batch;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (so[mid * m.D] <= blk) lo = mid; else hi = mid;
      }
      return lo;
    };
    for (int g = t + 1; g < G; g += 1024) {
      const int x = wo[g];
      if (x != wo[g + 1] || x <= 0 || x >= total) continue;
      const int b = seq_of(x - 1);
      if (b == seq_of(x))
        for (int h = 0; h < Hq; ++h) lse[static_cast<size_t>(b + g) * Hq + h] = -INFINITY;
    }
    return;
  }
  // One partial per work group and segment: segment s's pieces sit in slots
  // s + g for the work groups g of its blocks, so b's pieces fill [lo, hi)
  // except for gaps where a work-group boundary falls exactly on a segment
  // boundary. Gap slots get LSE = -inf (an empty partial) so the merge can
  // scan the whole range.
  for (int b = t; b < m.batch; b += 1024) {
    int lo = 0, hi = 0;
    for (int s = b * m.D; s < (b + 1) * m.D; ++s) {
      const int nb = so[s + 1] - so[s];
      if (nb <= 0) continue;
      const unsigned y0 = static_cast<unsigned>(co[s] + seg_cost);
      const int s_lo = s + range_of(y0);
      const int s_hi = s + range_of(y0 + nb - 1) + 1;
      if (hi == 0) lo = s_lo;
      else
        for (int x = hi; x < s_lo; ++x)
          for (int h = 0; h < Hq; ++h) lse[static_cast<size_t>(x) * Hq + h] = -INFINITY;
      hi = s_hi;
    }
    seq_slots[2 * b] = lo;
    seq_slots[2 * b + 1] = hi;
  }
}

hipError_t launch_plan(const SegMap& m, int S, int G, int seg_cost, int Hq, bool seq_pieces,
                       const PlanSig& sig, WorkspaceView ws, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, m, S, G, seg_cost, Hq,
                     seq_pieces ? 1 : 0, ws.header,
                     ws.seg_off, ws.cost_off, ws.wg_start, ws.seq_slots, ws.wg_seg, ws.lens, sig,
                     ws.lse);
  return hipGetLastError();
}

// ------------------------------------------------------------------ merge
// Slot sources: which stored partial rows feed output row b. count(b) slots,
// the i-th at row slot(b, i); a row whose LSE is -inf is empty.
struct PieceSource {
  const int32_t* seq_slots;  // [B][2] contiguous slot range of each sequence
  const PlanHeader* hdr;
  PlanSig sig;
  __device__ __forceinline__ bool valid() const { return plan_matches(sig, hdr); }
  __device__ __forceinline__ int first(int b) const { return seq_slots[2 * b]; }
  __device__ __forceinline__ int count(int b) const { return seq_slots[2 * b + 1] - seq_slots[2 * b]; }
  __device__ __forceinline__ int slot(int b, int i, int first) const { return first + i; }
};

struct PartialSource {
  int P, B;
  __device__ __forceinline__ bool valid() const { return true; }
  __device__ __forceinline__ int first(int) const { return 0; }
  __device__ __forceinline__ int count(int) const { return P; }
  __device__ __forceinline__ int slot(int b, int i, int) const { return i * B + b; }
};

// One thread per 4 output values of one head of one sequence; a work group
// holds kMergeThreads / (v_dim / 4) heads of one sequence, so for the usual
// shapes the whole grid is resident at once. Each thread requests up to
// kMergeRows partial rows (16 bytes of each) and their LSEs together, then
// folds them into its sums with a running maximum (weights exp(LSE_i - max),
// rescaled when the maximum rises): no LDS, no barriers, one memory round
// trip for up to kMergeRows partials. Rows past the count are not loaded; the
// row of an empty partial (LSE = -inf) is dropped by a select, so garbage in
// it never reaches the sum.
// Eight rows keep the kernel at 64 VGPRs, so eight waves fit on every SIMD and
// one round of work groups covers the usual grids (2048 groups of 256 threads);
// sixteen rows took 102 VGPRs and two rounds.
constexpr int kMergeRows = 8;       // partial rows in flight per thread
constexpr int kMergeThreads = 256;  // threads per work group

// Heads per merge work group for a value width (v_dim / 4 threads per head).
__host__ __device__ inline int merge_heads(int v_dim) {
  const int tph = v_dim / 4;
  return tph >= kMergeThreads ? 1 : kMergeThreads / tph;
}

// kF16: each row holds v_dim fp16 values in its first half, every
// kPieceSlice-column slice scaled by a power of two stored after them
// (sequence pieces); the slice's scale weights the row's contribution.
template <class Src, bool kF16>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    Src src, const float* __restrict__ o_rows, const float* __restrict__ lse_rows, int H,
    int v_dim, void* out, int out_bf16, float* lse_out) {
  const int tph = v_dim >> 2;
  const int hpb = merge_heads(v_dim);
  const int hh = threadIdx.x / tph;
  const int v4 = threadIdx.x % tph;
  // Heads vary fastest over the grid: consecutive work groups read rows of
  // different heads rather than of one head (a slot apart).
  const int b = blockIdx.y;
  const int h = blockIdx.x * hpb + hh;
  if (hh >= hpb || h >= H) return;  // (no barriers below)
  const size_t oidx = (static_cast<size_t>(b) * H + h) * v_dim + 4 * v4;
  if (!src.valid()) {
    // The workspace holds no plan of this launch's shape: NaN outputs.
    if (out_bf16)
      *reinterpret_cast<i32x2*>(static_cast<uint16_t*>(out) + oidx) = i32x2{0x7fc07fc0, 0x7fc07fc0};
    else
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + oidx) = f32x4{NAN, NAN, NAN, NAN};
    if (lse_out && v4 == 0) lse_out[static_cast<size_t>(b) * H + h] = NAN;
    return;
  }
  const int n = src.count(b);
  const int f0 = src.first(b);
  const float* orow = o_rows + static_cast<size_t>(h) * v_dim + 4 * v4;
  const float* row = o_rows + static_cast<size_t>(h) * v_dim;
  const uint16_t* orow16 = reinterpret_cast<const uint16_t*>(row) + 4 * v4;
  const float* srow = row + v_dim / 2 + (4 * v4) / kPieceSlice;
  float m = -INFINITY;  // largest LSE so far
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < n; k0 += kMergeRows) {
    f32x4 o[kMergeRows];
    i32x2 o16[kMergeRows];  // (fp16 rows, widened at use)
    float l[kMergeRows];
    float sc[kMergeRows];  // (fp16 rows) the row slice's scale
#pragma unroll
    for (int u = 0; u < kMergeRows; ++u) {
      l[u] = -INFINITY;
      if constexpr (kF16) {
        o16[u] = i32x2{0, 0};
        sc[u] = 1.f;
      } else {
        o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (k0 + u < n) {
        const size_t slot = static_cast<size_t>(src.slot(b, k0 + u, f0));
        l[u] = lse_rows[slot * H + h];
        if constexpr (kF16) {
          o16[u] = *reinterpret_cast<const i32x2*>(orow16 + 2 * slot * H * v_dim);
          sc[u] = srow[slot * H * v_dim];
        } else {
          o[u] = *reinterpret_cast<const f32x4*>(orow + slot * H * v_dim);
        }
      }
    }
    float mr = m;
#pragma unroll
    for (int u = 0; u < kMergeRows; ++u) mr = fmaxf(mr, l[u]);
    if (mr == -INFINITY) continue;  // only empty partials so far
    const float ml = mr * kLog2e;
    if (mr != m) {
      // (Only when the maximum rises: a round of empty partials leaves the sums
      // exactly as they are.)
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(m * kLog2e - ml);
      acc *= alpha;
      wsum *= alpha;
      m = mr;
    }
#pragma unroll
    for (int u = 0; u < kMergeRows; ++u) {
      const bool on = l[u] != -INFINITY;
      const float w = on ? fast_exp2(l[u] * kLog2e - ml) : 0.f;
      wsum += w;
      f32x4 ou;
      if constexpr (kF16) ou = __builtin_convertvector(__builtin_bit_cast(f16x4, o16[u]), f32x4);
      else ou = o[u];
      const float ws = kF16 ? w * sc[u] : w;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += on ? ws * ou[c] : 0.f;
    }
  }
  if (m != -INFINITY) acc *= 1.0f / wsum;
  if (out_bf16) {
    uint16_t* o16 = static_cast<uint16_t*>(out) + oidx;
    uint32_t lo = f32_to_bf16_bits(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[1])) << 16);
    uint32_t hi = f32_to_bf16_bits(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[3])) << 16);
    *reinterpret_cast<i32x2*>(o16) = i32x2{static_cast<int>(lo), static_cast<int>(hi)};
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + oidx) = acc;
  }
  if (lse_out && v4 == 0)
    lse_out[static_cast<size_t>(b) * H + h] = m == -INFINITY ? -INFINITY : m + fast_log2(wsum) * kLn2;
}

hipError_t launch_merge_pieces(const SegMap& m, const WorkspaceView& ws, const PlanSig& sig, int G,
                               int Hq, int v_dim, void* out, dcp_dtype_t out_dtype,
                               float* lse_out, hipStream_t stream) {
  (void)G;
  PieceSource src{ws.seq_slots, ws.header, sig};
  const int hpb = merge_heads(v_dim);
  dim3 grid((Hq + hpb - 1) / hpb, m.batch);
  if (sig.seq_pieces)
    hipLaunchKernelGGL((merge_kernel<PieceSource, true>), grid, dim3(kMergeThreads), 0, stream,
                       src, ws.o, ws.lse, Hq, v_dim, out, out_dtype == DCP_BF16 ? 1 : 0, lse_out);
  else
    hipLaunchKernelGGL((merge_kernel<PieceSource, false>), grid, dim3(kMergeThreads), 0, stream,
                       src, ws.o, ws.lse, Hq, v_dim, out, out_dtype == DCP_BF16 ? 1 : 0, lse_out);
  return hipGetLastError();
}

hipError_t launch_merge_partials(const float* o, const float* lse, int P, int B, int H, int v_dim,
                                 void* out, dcp_dtype_t out_dtype, float* lse_out,
                                 hipStream_t stream) {
  PartialSource src{P, B};
  const int hpb = merge_heads(v_dim);
  dim3 grid((H + hpb - 1) / hpb, B);
  hipLaunchKernelGGL((merge_kernel<PartialSource, false>), grid, dim3(kMergeThreads), 0, stream,
                     src, o, lse, H, v_dim, out, out_dtype == DCP_BF16 ? 1 : 0, lse_out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ remap
// One work group per (shard r, sequence b) row of the local table; its
// threads walk the row's entries i, and thread 0 writes the shard's token
// count for sequence b. Interleaved ownership: entry i of shard r is logical
// block r + D*i. Contiguous ownership (the 200K-token four-way split of the
// DCP blog page, section A2): a sequence of nb blocks is cut into runs of
// c = ceil(nb / D) blocks and entry i of shard r is logical block r*c + i.
__global__ __launch_bounds__(256) void remap_kernel(const int32_t* __restrict__ table,
                                                    const int32_t* __restrict__ lens, int B,
                                                    int max_blocks, int bs, int D, int width,
                                                    int contiguous,
                                                    int32_t* __restrict__ local_table,
                                                    int32_t* __restrict__ local_lens) {
  const int r = blockIdx.x / B;
  const int b = blockIdx.x - r * B;
  long long L = lens[b];
  const long long cap = static_cast<long long>(max_blocks) * bs;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int nb = static_cast<int>((L + bs - 1) / bs);
  const int32_t* trow = table + static_cast<size_t>(b) * max_blocks;
  int32_t* lrow = local_table + static_cast<size_t>(blockIdx.x) * width;
  if (contiguous) {
    const int c = (nb + D - 1) / D;  // c <= width because nb <= max_blocks
    const int j0 = r * c;
    for (int i = threadIdx.x; i < width; i += blockDim.x)
      lrow[i] = (i < c && j0 + i < nb) ? trow[j0 + i] : -1;
    if (threadIdx.x == 0) {
      const long long lo = static_cast<long long>(j0) * bs;
      const long long n = (lo + static_cast<long long>(c) * bs < L ? lo + static_cast<long long>(c) * bs : L) - lo;
      local_lens[blockIdx.x] = static_cast<int32_t>(n > 0 ? n : 0);
    }
    return;
  }
  for (int i = threadIdx.x; i < width; i += blockDim.x) {
    const int j = r + D * i;
    lrow[i] = j < nb ? trow[j] : -1;
  }
  if (threadIdx.x == 0) {
    const int n_r = nb > r ? (nb - r + D - 1) / D : 0;
    const int tail = (nb > 0 && (nb - 1) % D == r) ? static_cast<int>(static_cast<long long>(nb) * bs - L) : 0;
    local_lens[blockIdx.x] = n_r * bs - tail;
  }
}

hipError_t launch_remap(const int32_t* table, const int32_t* lens, int B, int max_blocks, int bs,
                        int D, bool contiguous, int32_t* local_table, int32_t* local_lens,
                        hipStream_t stream) {
  const int width = (max_blocks + D - 1) / D;
  const int threads = width >= 256 ? 256 : (width >= 128 ? 128 : 64);
  hipLaunchKernelGGL(remap_kernel, dim3(static_cast<unsigned>(D) * B), dim3(threads), 0, stream,
                     table, lens, B, max_blocks, bs, D, width, contiguous ? 1 : 0, local_table,
                     local_lens);
  return hipGetLastError();
}

}  // namespace dcp
