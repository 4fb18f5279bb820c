// Grouped-query partial attention over a paged K/V cache (gfx950).
//
// "Efficient Decode Context Parallelism with vLLM for Long Context Workloads",
// A2 (GQA backend): a KV head is shared ("tensor broadcast") by its group of
// query heads; under DCP each shard attends the full query against its own
// blocks of the shared head and returns a partial output with its LSE.
//
// Work: the same stream-K ranges as the latent kernel, times the KV heads and
// their column tiles (grid = ranges x (Hkv x column tiles)). The query rows of
// one KV head are its group's heads for every query token (several tokens in
// multi-token decode), taken 16 at a time. Cache layout
// [block, token, kv_head, dim].
//
// bf16 kernel: one wave per (range, KV head, column tile). 32-token K and V
// tiles are copied HBM -> LDS with 16-byte direct-to-LDS loads (two stages);
// the tile's query rows form the N = 16 side of v_mfma_f32_16x16x32_bf16:
// S^T = K_tile . Q^T, then O^T += V_tile^T . P^T with the transposed V operand
// read by ds_read_b64_tr_b16. A tile with fewer than 16 rows is padded with
// zero queries; padded columns are never stored.
// At 8 flop per cache byte this path is bound by HBM, not by the MFMA pipe.
//
// fp32 kernel: plain VALU, one lane per token for the scores and one lane per
// value column for the weighted sum, over up to 16 query rows per wave.
#include "dcp_internal.hpp"

namespace dcp {
namespace {

constexpr int kT = 32;
// Work groups over all KV heads per launch. A bf16 work group (one wave, two
// stages of 32-token K and V tiles in LDS) holds ~32 KB of LDS, so four fit on
// a CU: 1,024 groups all run at once, in one round. Measured on MI355X at
// 32 sequences x 32K tokens, 8 KV heads of 128: 1,024 groups 0.679 ms against
// 0.688 ms for 2,048 (two rounds, the second 60 % occupied), 0.725 ms for 768
// and 0.98 ms for 1,280 (a fifth group per CU does not fit).
constexpr int kGroupsTotal = 1024;

struct GqaArgs {
  const void* q;          // [B, Hq, d]
  const char* k;          // cache bases
  const char* v;
  SegMap map;
  const PlanHeader* hdr;
  PlanSig sig;              // the plan's expected signature
  const int32_t* wg_start;  // [G + 1] block range of each work group
  const int32_t* wg_seg;    // [G + 1] segment of each range's first block
  const int32_t* seg_off;
  float* ws_o;
  float* ws_lse;
  long long block_stride_b, token_stride_b, head_stride_b;  // bytes
  int S;
  int G;      // ranges (work groups per KV head and column tile)
  int ncb;
  int Hq;     // query rows per sequence (q_len * heads per token)
  int group;  // query heads per KV head
  int cols;   // query rows per KV head: group * q_len, in tiles of 16
  int ctiles;
  float scale_log2;
  Causal cz;
  bool causal;
};

// Column c of a KV head's query rows: token c / group, head c % group of that
// KV head's group; its row in q and in the partials is token * Hq_tok + head.
__device__ __forceinline__ int gqa_row(const GqaArgs& a, int kvh, int c) {
  const int t = c / a.group;
  return t * a.cz.hq + kvh * a.group + (c - t * a.group);
}

// (Through the builtin, so the compiler's own wait insertion sees it; the empty
// asm keeps memory accesses from moving across it.)
__device__ __forceinline__ void wait_vm_all() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
  asm volatile("" ::: "memory");
}

// Row swizzle for rows of R chunks (R = 8 or 16).
template <int R>
__device__ __forceinline__ int swz(int r) {
  if constexpr (R == 16) return r & 15;
  else return (r & 7) ^ ((r >> 3) & 1);
}
template <int R>
__device__ __forceinline__ int chunk_off(int r, int c) {
  return (r * R + (c ^ swz<R>(r))) * 16;
}

template <int DH>
__global__ __launch_bounds__(64) void gqa_bf16_kernel(GqaArgs a) {
  constexpr int R = DH / 8;              // 16-byte chunks per row
  constexpr int kTileB = kT * DH * 2;    // bytes per K (or V) tile
  constexpr int kInst = kT * R / 64;     // wave-wide copies per tile
  constexpr int kKSteps = DH / 32;
  constexpr int kVTiles = DH / 16;
  __shared__ __attribute__((aligned(16))) char smem_raw[2 * 2 * kTileB];
  DCP_LDS char* smem = (DCP_LDS char*)smem_raw;

  const int lane = threadIdx.x;
  const int q4 = lane >> 4, l16 = lane & 15;
  const int kvh = blockIdx.y / a.ctiles;
  const int ct = blockIdx.y - kvh * a.ctiles;
  const int g = xcd_logical_group(blockIdx.x, a.G);
  if (!plan_matches(a.sig, a.hdr)) return;  // no plan of this launch's shape
  int pos = a.wg_start[g];
  const int end = a.wg_start[g + 1];
  if (pos >= end) return;
  int s = a.wg_seg[g];
  const int bs = a.map.bs;
  // This lane's query row: column 16ct + l16 of the KV head's (token, head) rows.
  const int col_q = 16 * ct + l16;
  const bool head_ok = col_q < a.cols;
  const int h = gqa_row(a, kvh, head_ok ? col_q : 0);
  const int t_q = (head_ok ? col_q : 0) / a.group;  // its query token

  int a_off0[kKSteps], a_off1[kKSteps];
#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk) {
    a_off0[kk] = chunk_off<R>(l16, 4 * kk + q4);
    a_off1[kk] = chunk_off<R>(16 + l16, 4 * kk + q4);
  }
  const int t_k = l16 >> 2, t_m = l16 & 3;
  int t_off0[kVTiles], t_off1[kVTiles];
#pragma unroll
  for (int mt = 0; mt < kVTiles; ++mt) {
    const int c = 2 * mt + (t_m >> 1);
    t_off0[mt] = chunk_off<R>(4 * q4 + t_k, c) + 8 * (t_m & 1);
    t_off1[mt] = chunk_off<R>(16 + 4 * q4 + t_k, c) + 8 * (t_m & 1);
  }

  while (pos < end) {
    while (a.seg_off[s + 1] <= pos) ++s;
    const int seg_a = a.seg_off[s];
    const int pe = min(end, a.seg_off[s + 1]);
    const Piece p = make_piece(a.map, s, pos - seg_a, pe - seg_a);
    const int b = p.b;
    const int32_t* trow = a.map.table + static_cast<size_t>(b) * a.map.width;
    const long long qpos0 = a.causal ? first_query_pos(a.cz, a.map, b) : 0;

    bf16x8 qf[kKSteps];
    {
      const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                             (static_cast<size_t>(b) * a.Hq + h) * DH + 8 * q4;
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + 32 * kk);
        if (!head_ok) qf[kk] = bf16x8{};
      }
    }
    f32x4 acc[kVTiles];
#pragma unroll
    for (int mt = 0; mt < kVTiles; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    float l_rnd = 0.f;  // the same sum over the probabilities as rounded to bf16
    const int ntiles = (p.ntok + kT - 1) / kT;

    auto load_id = [&](int tau0) -> int {
      const int tau = tau0 + (lane & 31);
      int id = -1;
      if (lane < 32 && tau < p.ntok) id = trow[piece_col(a.map, p, tau)];
      return id;
    };
    auto row_mask = [&](int tau0, int id) -> unsigned long long {
      return __ballot(lane < 32 && tau0 + lane < p.ntok && id >= 0 && id < a.ncb);
    };
    auto issue_tile = [&](int tau0, int id, unsigned long long vm, int stage) {
      DCP_LDS char* kd = smem + stage * 2 * kTileB;
      DCP_LDS char* vd = kd + kTileB;
#pragma unroll
      for (int ii = 0; ii < kInst; ++ii) {
        const int slot = ii * 64 + lane;
        const int row = slot / R;
        const int pc = slot - row * R;
        const int c = pc ^ swz<R>(row);
        const int rid = __shfl(id, row);
        if ((vm >> row) & 1ull) {
          const long long off = static_cast<long long>(rid) * a.block_stride_b +
                                static_cast<long long>((tau0 + row) % bs) * a.token_stride_b +
                                kvh * a.head_stride_b + 16 * c;
          __builtin_amdgcn_global_load_lds(a.k + off, kd + ii * 1024, 16, 0, kCopyPolicy);
          __builtin_amdgcn_global_load_lds(a.v + off, vd + ii * 1024, 16, 0, kCopyPolicy);
        } else {
          *reinterpret_cast<DCP_LDS i32x4*>(kd + slot * 16) = i32x4{0, 0, 0, 0};
          *reinterpret_cast<DCP_LDS i32x4*>(vd + slot * 16) = i32x4{0, 0, 0, 0};
        }
      }
    };

    int id_cur = load_id(0);
    wait_vm_all();
    unsigned long long vm_cur = row_mask(0, id_cur);
    issue_tile(0, id_cur, vm_cur, 0);
    int id_next = ntiles > 1 ? load_id(kT) : -1;

    for (int k = 0; k < ntiles; ++k) {
      wait_vm_all();
      __builtin_amdgcn_s_barrier();  // single wave: orders LDS use, no other waves
      const unsigned long long vm_k = vm_cur;
      const DCP_LDS char* kt = smem + (k & 1) * 2 * kTileB;
      const DCP_LDS char* vt = kt + kTileB;
      if (k + 1 < ntiles) {
        const int tau1 = (k + 1) * kT;
        vm_cur = row_mask(tau1, id_next);
        issue_tile(tau1, id_next, vm_cur, (k + 1) & 1);
        if (k + 2 < ntiles) id_next = load_id((k + 2) * kT);
      }

      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        const bf16x8 k0 = *reinterpret_cast<const DCP_LDS bf16x8*>(kt + a_off0[kk]);
        const bf16x8 k1 = *reinterpret_cast<const DCP_LDS bf16x8*>(kt + a_off1[kk]);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[kk], s1, 0, 0, 0);
      }
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = 4 * q4 + i, r1 = 16 + 4 * q4 + i;
        x[i] = ((vm_k >> r0) & 1ull) ? s0[i] * a.scale_log2 : -INFINITY;
        x[4 + i] = ((vm_k >> r1) & 1ull) ? s1[i] * a.scale_log2 : -INFINITY;
      }
      if (a.causal) {
        // Multi-token decode: tile row r (lane r < 32 computes its global
        // position) is visible to this lane's query token t_q if it lies at
        // most t_q past the first query's position.
        const int tau = k * kT + (lane & 31);
        const long long e = global_pos(a.cz, piece_col(a.map, p, tau), bs, tau % bs) - qpos0;
        const int ec = static_cast<int>(e < -1 ? -1 : (e > 127 ? 127 : e));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (__shfl(ec, 4 * q4 + i) > t_q) x[i] = -INFINITY;
          if (__shfl(ec, 16 + 4 * q4 + i) > t_q) x[4 + i] = -INFINITY;
        }
      }
      float tmax = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, x[i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = fast_exp2(x[2 * i] - m_use);
        const float p1 = fast_exp2(x[2 * i + 1] - m_use);
        const uint16_t b0 = f32_to_bf16_bits(p0);
        const uint16_t b1 = f32_to_bf16_bits(p1);
        psum += p0 + p1;  // (the LSE's sum keeps the fp32 probabilities)
        pk[i] = static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16);
      }
      l_run = l_run * alpha + psum;
      l_rnd = l_rnd * alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) l_rnd = add_bf16x2(pk[i], l_rnd);
      const i32x4 pki = {static_cast<int>(pk[0]), static_cast<int>(pk[1]), static_cast<int>(pk[2]),
                         static_cast<int>(pk[3])};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pki);
#pragma unroll
      for (int mt = 0; mt < kVTiles; ++mt) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<DCP_LDS s16x4*>(const_cast<DCP_LDS char*>(vt + t_off0[mt])));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<DCP_LDS s16x4*>(const_cast<DCP_LDS char*>(vt + t_off1[mt])));
        const short __attribute__((ext_vector_type(8))) cat = {lo[0], lo[1], lo[2], lo[3],
                                                               hi[0], hi[1], hi[2], hi[3]};
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cat), pb,
                                                         acc[mt] * alpha, 0, 0, 0);
      }
    }

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    // The output is normalised by the sum of the bf16 probabilities its
    // product used; the LSE takes the fp32 sum.
    float l_out = l_rnd + __shfl_xor(l_rnd, 16);
    l_out += __shfl_xor(l_out, 32);
    const float inv = l_out > 0.f ? 1.f / l_out : 0.f;
    const float lse = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
    const size_t slot = static_cast<size_t>(s) + g;
    if (head_ok) {
      float* orow = a.ws_o + (slot * a.Hq + h) * DH + 4 * q4;
#pragma unroll
      for (int mt = 0; mt < kVTiles; ++mt) *reinterpret_cast<f32x4*>(orow + 16 * mt) = acc[mt] * inv;
      if (q4 == 0) a.ws_lse[slot * a.Hq + h] = lse;
    }
    __builtin_amdgcn_s_barrier();
    pos = pe;
  }
}

// fp32: one wave per (range, KV head, column tile). Scores: lane = token of a 64-token
// tile; weighted sum: lane = value column (DH / 64 columns per lane).
template <int DH>
__global__ __launch_bounds__(64) void gqa_f32_kernel(GqaArgs a) {
  constexpr int kTok = 64;
  constexpr int kCols = DH / 64;
  constexpr int kMaxGroup = 16;
  __shared__ float q_lds[kMaxGroup][DH];
  __shared__ float p_lds[kMaxGroup][kTok];
  __shared__ int id_lds[kTok];

  const int lane = threadIdx.x;
  const int kvh = blockIdx.y / a.ctiles;
  const int ct = blockIdx.y - kvh * a.ctiles;
  const int g = xcd_logical_group(blockIdx.x, a.G);
  if (!plan_matches(a.sig, a.hdr)) return;  // no plan of this launch's shape
  int pos = a.wg_start[g];
  const int end = a.wg_start[g + 1];
  if (pos >= end) return;
  int s = a.wg_seg[g];
  const int bs = a.map.bs;
  // Columns j < G of this wave: the KV head's query rows 16ct + j (token, head).
  const int G = min(kMaxGroup, a.cols - 16 * ct);

  while (pos < end) {
    while (a.seg_off[s + 1] <= pos) ++s;
    const int seg_a = a.seg_off[s];
    const int pe = min(end, a.seg_off[s + 1]);
    const Piece p = make_piece(a.map, s, pos - seg_a, pe - seg_a);
    const int b = p.b;
    const int32_t* trow = a.map.table + static_cast<size_t>(b) * a.map.width;
    const float* qb = static_cast<const float*>(a.q) + static_cast<size_t>(b) * a.Hq * DH;
    for (int i = lane; i < G * DH; i += 64)
      q_lds[i / DH][i % DH] = qb[static_cast<size_t>(gqa_row(a, kvh, 16 * ct + i / DH)) * DH + i % DH];
    const long long qpos0 = a.causal ? first_query_pos(a.cz, a.map, b) : 0;
    float m_run[kMaxGroup], l_run[kMaxGroup], acc[kMaxGroup][kCols];
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j) {
      m_run[j] = -INFINITY;
      l_run[j] = 0.f;
#pragma unroll
      for (int c = 0; c < kCols; ++c) acc[j][c] = 0.f;
    }
    __syncthreads();
    for (int tau0 = 0; tau0 < p.ntok; tau0 += kTok) {
      const int tau = tau0 + lane;
      int id = -1;
      if (tau < p.ntok) id = trow[piece_col(a.map, p, tau)];
      const bool ok = tau < p.ntok && id >= 0 && id < a.ncb;
      id_lds[lane] = ok ? id : -1;
      // Multi-token decode: how far this token lies past the first query.
      const long long e = a.causal && ok
                              ? global_pos(a.cz, piece_col(a.map, p, tau), bs, tau % bs) - qpos0
                              : -1;
      const float* krow = ok ? reinterpret_cast<const float*>(
                                   a.k + static_cast<long long>(id) * a.block_stride_b +
                                   static_cast<long long>(tau % bs) * a.token_stride_b +
                                   kvh * a.head_stride_b)
                             : nullptr;
#pragma unroll
      for (int j = 0; j < kMaxGroup; ++j) {
        if (j >= G) continue;
        float dot = 0.f;
        if (ok)
          for (int d = 0; d < DH; ++d) dot = fmaf(q_lds[j][d], krow[d], dot);
        const bool seen = ok && e <= (16 * ct + j) / a.group;
        const float x = seen ? dot * a.scale_log2 : -INFINITY;
        float tmax = x;
        for (int off = 32; off >= 1; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
        const float m_new = fmaxf(m_run[j], tmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[j] - m_use);
        const float pj = fast_exp2(x - m_use);
        float ps = pj;
        for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
        m_run[j] = m_new;
        l_run[j] = l_run[j] * alpha + ps;
#pragma unroll
        for (int c = 0; c < kCols; ++c) acc[j][c] *= alpha;
        p_lds[j][lane] = pj;
      }
      __syncthreads();
      const int ntok = min(kTok, p.ntok - tau0);
      for (int t = 0; t < ntok; ++t) {
        const int tid = id_lds[t];
        if (tid < 0) continue;
        const float* vrow = reinterpret_cast<const float*>(
            a.v + static_cast<long long>(tid) * a.block_stride_b +
            static_cast<long long>((tau0 + t) % bs) * a.token_stride_b + kvh * a.head_stride_b);
        float vv[kCols];
#pragma unroll
        for (int c = 0; c < kCols; ++c) vv[c] = vrow[lane + 64 * c];
#pragma unroll
        for (int j = 0; j < kMaxGroup; ++j) {
          if (j >= G) continue;
          const float pw = p_lds[j][t];
#pragma unroll
          for (int c = 0; c < kCols; ++c) acc[j][c] = fmaf(pw, vv[c], acc[j][c]);
        }
      }
      __syncthreads();
    }
    const size_t slot = static_cast<size_t>(s) + g;
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j) {
      if (j >= G) continue;
      const int h = gqa_row(a, kvh, 16 * ct + j);
      const float inv = l_run[j] > 0.f ? 1.f / l_run[j] : 0.f;
#pragma unroll
      for (int c = 0; c < kCols; ++c) a.ws_o[(slot * a.Hq + h) * DH + lane + 64 * c] = acc[j][c] * inv;
      if (lane == 0)
        a.ws_lse[slot * a.Hq + h] =
            l_run[j] > 0.f ? (m_run[j] + fast_log2(l_run[j])) * kLn2 : -INFINITY;
    }
    __syncthreads();
    pos = pe;
  }
}

}  // namespace

int gqa_groups(const dcp_attn_desc_t* d) {
  int per = kGroupsTotal / (d->num_kv_heads > 0 ? d->num_kv_heads : 1);
  per = per < 8 ? 8 : per;
  return per / 8 * 8;
}

bool gqa_supported(const dcp_attn_desc_t* d) {
  if (d->kv_kind != DCP_KV_SEPARATE) return false;
  if (d->qk_dim != d->v_dim || (d->qk_dim != 64 && d->qk_dim != 128)) return false;
  if (d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0) return false;
  if (d->num_q_heads / d->num_kv_heads > 16) return false;
  if (d->q_dtype != d->kv_dtype) return false;
  return d->kv_dtype == DCP_F32 || d->kv_dtype == DCP_BF16;
}

hipError_t launch_gqa(const AttnLaunch& L, hipStream_t stream) {
  const dcp_attn_desc_t* d = L.desc;
  GqaArgs a;
  a.q = L.q;
  a.k = static_cast<const char*>(L.k_cache);
  a.v = static_cast<const char*>(L.v_cache);
  a.map = L.map;
  a.hdr = L.ws.header;
  a.sig = L.sig;
  a.wg_start = L.ws.wg_start;
  a.wg_seg = L.ws.wg_seg;
  a.seg_off = L.ws.seg_off;
  a.ws_o = L.ws.o;
  a.ws_lse = L.ws.lse;
  const int elt = d->kv_dtype == DCP_F32 ? 4 : 2;
  a.block_stride_b = d->kv_block_stride * elt;
  a.token_stride_b = d->kv_token_stride * elt;
  a.head_stride_b = d->kv_head_stride * elt;
  a.S = L.S;
  a.G = gqa_groups(d);
  a.ncb = d->num_cache_blocks;
  a.Hq = desc_rows(d);
  a.group = d->num_q_heads / d->num_kv_heads;
  a.cols = a.group * desc_q_len(d);
  a.ctiles = (a.cols + 15) / 16;
  a.scale_log2 = d->softmax_scale * kLog2e;
  a.cz = L.cz;
  a.causal = L.cz.q_len > 1 || L.cz.q_pos != nullptr;
  const dim3 grid(a.G, d->num_kv_heads * a.ctiles);
  if (d->kv_dtype == DCP_BF16) {
    if (d->qk_dim == 128)
      hipExtLaunchKernelGGL(gqa_bf16_kernel<128>, grid, dim3(64), 0, stream, L.ev_begin, L.ev_end,
                            0, a);
    else
      hipExtLaunchKernelGGL(gqa_bf16_kernel<64>, grid, dim3(64), 0, stream, L.ev_begin, L.ev_end,
                            0, a);
  } else {
    if (d->qk_dim == 128)
      hipExtLaunchKernelGGL(gqa_f32_kernel<128>, grid, dim3(64), 0, stream, L.ev_begin, L.ev_end,
                            0, a);
    else
      hipExtLaunchKernelGGL(gqa_f32_kernel<64>, grid, dim3(64), 0, stream, L.ev_begin, L.ev_end,
                            0, a);
  }
  return hipGetLastError();
}

}  // namespace dcp
