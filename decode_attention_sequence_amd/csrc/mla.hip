// Absorbed-MLA partial attention over a paged latent cache (gfx950).
//
// "Efficient Decode Context Parallelism with vLLM for Long Context Workloads",
// A2 (MLA backend): the latent KV is one low-rank row per token shared by
// every query head, so the cache has one effective KV head and can be split
// along the sequence as far as the tensor-parallel degree; each shard attends
// the full query against its local latent slice and returns a partial output
// with its log-sum-exp. In the absorbed form used here the query already
// lives in latent space (qk_dim = 576 = 512 latent + 64 rotary columns): the
// score is q . c over all 576 columns and the value is c[0:512].
//
// Kernel design (one work group per CU, one stream-K range of cache blocks
// per work group, up to 64 query heads per work group):
//  * wave w owns query heads 16w .. 16w+15 and keeps their query rows in
//    registers as MFMA B fragments for the whole range;
//  * 32-token latent tiles (36 KB bf16) are copied HBM -> LDS with 16-byte
//    direct-to-LDS loads through a 4-stage ring, so three tiles (108 KB) are
//    in flight per CU while one is consumed; each wave issues a fixed number
//    of copies per tile, so `s_waitcnt vmcnt(n)` names exactly the tiles
//    still in flight. Rows past the end of the range (or with an unusable
//    block id) are copied from a safe address and zero-filled once landed;
//  * S^T[t][h] = C_tile . Q^T with v_mfma_f32_16x16x32_bf16 (A = latent rows
//    from LDS, B = query fragments), so each lane ends up holding one head's
//    scores for 8 tokens -- exactly the B-operand layout of the next product;
//  * online softmax per head in the exp2 domain; the running reference max is
//    only raised (and the accumulator rescaled) when a tile's max exceeds it
//    by more than 8, so probabilities stay <= 256 and rescales are rare;
//  * O^T[v][h] += C_tile^T . P^T with the same MFMA, the transposed A operand
//    read from the same LDS tile by ds_read_b64_tr_b16, so every latent byte
//    is fetched from HBM once and serves both products;
//  * the fp8 variant copies e4m3 codes and one fp32 scale per token, widens
//    the codes to fp16 in LDS (exact) one tile ahead of the MFMAs and runs
//    both products as v_mfma_f32_16x16x32_f16 (query converted bf16 -> fp16);
//    the token scale multiplies the fp32 score and the probability weighting
//    the value, and that product is rounded to fp16 (2^-11 relative), not
//    bf16, so it stays inside the error budget of an 8-bit cache.
#include "dcp_internal.hpp"

namespace dcp {
namespace {

constexpr int kQK = 576;
constexpr int kV = 512;
constexpr int kHeadsPerGroup = 64;         // query heads per work group
constexpr int kT = 32;                     // tokens per tile
constexpr int kRowB = kQK * 2;             // bf16 row bytes (1152)
constexpr int kRowCh = kRowB / 16;         // 16-byte chunks per row (72)
constexpr int kTileB = kT * kRowB;         // 36864
constexpr int kTileCh = kT * kRowCh;       // 2304
constexpr int kDmaInst = kTileCh / 64;     // 36 wave-wide copies per bf16 tile
constexpr int kKSteps = kQK / 32;          // 18
constexpr int kVTiles = kV / 16;           // 32
constexpr int kF8RowB = kQK;               // 576 code bytes per row
constexpr int kF8TileB = kT * kF8RowB;     // 18432
constexpr int kF8RowCh = kF8RowB / 16;     // 36
constexpr int kF8DmaInst = kF8TileB / 1024;  // 18
constexpr int kGroups = 256;               // work groups per head group (one per CU)
constexpr int kStages = 4;                 // copy ring depth
constexpr int kIdWin = 2048;               // block ids staged in LDS at a time
constexpr int kPadB = 1024;                // landing pad for filler copies
constexpr int kScaleB = 256;               // per-wave scale landing area per stage

// LDS layouts.
//   bf16: [kStages tiles][ids][pad]
//   fp8 : [kStages code tiles][2 bf16 tiles][scales: kStages x NW x 256 B][ids][pad]
constexpr int kLdsBf16 = kStages * kTileB + kIdWin * 4 + kPadB;
template <int NW>
constexpr int lds_fp8() { return kStages * kF8TileB + 2 * kTileB + kStages * NW * kScaleB + kIdWin * 4 + kPadB; }

// Row swizzle: logical chunk c of row r sits at (c & ~7) | ((c & 7) ^ swz(r)).
// With 1152-byte rows this keeps both access patterns below free of LDS bank
// conflicts: 16 rows x one 16-byte chunk (MFMA A fragments) and 4 rows x 32
// bytes per 16-lane group (transposed reads).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int chunk_off(int r, int c) {
  return r * kRowB + 16 * ((c & ~7) | ((c & 7) ^ swz(r)));
}

struct MlaArgs {
  const uint16_t* q;      // [B, Hq, 576] bf16 bits
  const char* kv;         // latent cache base
  const char* kv_scale;   // fp8: fp32 [num_cache_blocks, bs]
  SegMap map;
  const PlanHeader* hdr;
  const int32_t* seg_off;
  float* ws_o;
  float* ws_lse;
  long long block_stride_b;  // bytes
  long long token_stride_b;  // bytes
  int S;
  int ncb;
  int Hq;
  float scale_log2;
};

__device__ __forceinline__ bf16x8 lds_read_b128(const DCP_LDS char* p) {
  return *reinterpret_cast<const DCP_LDS bf16x8*>(p);
}

__device__ __forceinline__ s16x4 lds_read_tr(const DCP_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<DCP_LDS s16x4*>(const_cast<DCP_LDS char*>(p)));
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// e4m3 codes -> fp16, exact: every e4m3 value (4 significant bits, |x| <= 448,
// down to 2^-9) is an fp16 normal or subnormal number.
template <bool HI>
__device__ __forceinline__ uint32_t f8x2_to_f16x2(uint32_t codes) {
  f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes), HI);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f[0], f[1]));
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// MFMA element type: bf16 for a bf16 cache; fp16 for an fp8 cache, whose codes
// widen to fp16 exactly and whose probability-times-scale products then keep
// 11 significant bits instead of 8.
template <bool FP8>
struct Elt;
template <>
struct Elt<false> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 mfma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t from_f32(float x) { return f32_to_bf16_bits(x); }
  static __device__ __forceinline__ vec from_bf16(bf16x8 v) { return v; }
};
template <>
struct Elt<true> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 mfma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t from_f32(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  // bf16 -> fp16 (exact inside the fp16 range).
  static __device__ __forceinline__ vec from_bf16(bf16x8 v) {
    vec r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<_Float16>(static_cast<float>(v[i]));
    return r;
  }
};

template <int NW, bool FP8>
struct MlaCfg {
  static constexpr int kInst = FP8 ? kF8DmaInst : kDmaInst;
  static constexpr int kPerWave = (kInst + NW - 1) / NW;        // copies per wave per tile
  static constexpr int kOps = kPerWave + (FP8 ? 1 : 0);          // + the scale copy
  static constexpr int kLds = FP8 ? lds_fp8<NW>() : kLdsBf16;
  static constexpr int kStageB = FP8 ? kF8TileB : kTileB;
  static constexpr int kIdsOff = FP8 ? kStages * kF8TileB + 2 * kTileB + kStages * NW * kScaleB
                                     : kStages * kTileB;
  static constexpr int kPadOff = kIdsOff + kIdWin * 4;
  static constexpr int kBf16Off = kStages * kF8TileB;            // fp8 only
  static constexpr int kScaleOff = kStages * kF8TileB + 2 * kTileB;  // fp8 only
};

// Wait until at most n_after tiles (C::kOps operations each) issued after the
// awaited one are still in flight. The hardware counter saturates at 63, so
// larger counts are clamped, which only waits for more.
template <int NW, bool FP8>
__device__ __forceinline__ void wait_tiles_after(int n_after) {
  using C = MlaCfg<NW, FP8>;
  constexpr int k1 = C::kOps > 63 ? 63 : C::kOps;
  constexpr int k2 = 2 * C::kOps > 63 ? 63 : 2 * C::kOps;
  switch (n_after) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<k1>(); break;
    default: wait_vm<k2>(); break;
  }
}

template <int NW, bool FP8>
__global__ __launch_bounds__(NW * 64) void mla_partial_kernel(MlaArgs a) {
  using C = MlaCfg<NW, FP8>;
  static_assert(kStages == 4, "wait_tiles_after assumes at most two tiles in flight after one");
  __shared__ __attribute__((aligned(16))) char smem_raw[C::kLds];
  DCP_LDS char* smem = (DCP_LDS char*)smem_raw;
  DCP_LDS int* ids = (DCP_LDS int*)(smem + C::kIdsOff);
  DCP_LDS char* pad = smem + C::kPadOff;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int q4 = lane >> 4;
  const int l16 = lane & 15;
  const int g = xcd_logical_group(blockIdx.x, kGroups);
  const int head0 = blockIdx.y * kHeadsPerGroup;
  const int chunk = a.hdr->chunk;
  const int total = a.hdr->total;
  int pos = g * chunk;
  const int end = min(pos + chunk, total);
  if (pos >= end) return;
  int s = find_segment(a.seg_off, a.S, pos);
  const int bs = a.map.bs;
  const int h = head0 + 16 * w + l16;

  // Per-lane constant LDS offsets.
  // A fragment of S^T: rows l16 and 16 + l16, chunk 4kk + q4.
  const int a_even0 = l16 * kRowB + 16 * (q4 ^ swz(l16));
  const int a_odd0 = l16 * kRowB + 16 * ((4 + q4) ^ swz(l16));
  const int a_even1 = (16 + l16) * kRowB + 16 * (q4 ^ swz(16 + l16));
  const int a_odd1 = (16 + l16) * kRowB + 16 * ((4 + q4) ^ swz(16 + l16));
  // Transposed A fragment of O^T: lane (k = l16/4, m = l16%4) points at rows
  // 4q4 + k and 16 + 4q4 + k, bytes 32mt + 8m, i.e. chunk 2mt + m/2.
  const int t_k = l16 >> 2, t_m = l16 & 3;
  const int t_row0 = 4 * q4 + t_k, t_row1 = 16 + 4 * q4 + t_k;
  int t_off0[4], t_off1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 2 * j + (t_m >> 1);  // chunk within an aligned 8-chunk group
    t_off0[j] = t_row0 * kRowB + 16 * (c ^ swz(t_row0)) + 8 * (t_m & 1);
    t_off1[j] = t_row1 * kRowB + 16 * (c ^ swz(t_row1)) + 8 * (t_m & 1);
  }

  while (pos < end) {
    while (a.seg_off[s + 1] <= pos) ++s;
    const int seg_a = a.seg_off[s];
    const int pe = min(end, a.seg_off[s + 1]);
    const Piece p = make_piece(a.map, s, pos - seg_a, pe - seg_a);
    const int32_t* trow = a.map.table + static_cast<size_t>(p.b) * a.map.width;

    // Query fragments (B operand of S^T): head h, columns 32kk + 8q4 .. +7.
    typename Elt<FP8>::vec qf[kKSteps];
    {
      const uint16_t* qrow = a.q + (static_cast<size_t>(p.b) * a.Hq + h) * kQK + 8 * q4;
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk)
        qf[kk] = Elt<FP8>::from_bf16(*reinterpret_cast<const bf16x8*>(qrow + 32 * kk));
    }
    f32x4 acc[kVTiles];
#pragma unroll
    for (int mt = 0; mt < kVTiles; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY;  // reference max (log2 units) the accumulators are scaled to
    float l_run = 0.f;

    // Windows of at most kIdWin blocks share one LDS copy of their block ids.
    for (int wb = p.i0; wb < p.i1; wb += kIdWin) {
      const int we = min(p.i1, wb + kIdWin);
      const int ntok = (we - wb) * bs - (we == p.i1 ? (p.i1 - p.i0) * bs - p.ntok : 0);
      for (int i = threadIdx.x; i < we - wb; i += NW * 64)
        ids[i] = trow[p.r + a.map.D * (wb + i)];
      wait_vm<0>();
      __syncthreads();
      const int ntiles = (ntok + kT - 1) / kT;

      // Copy tile j of this window into ring stage j % kStages. Every wave
      // issues exactly C::kOps vector-memory operations per tile.
      auto issue = [&](int j) {
        const int tau0 = j * kT;
        DCP_LDS char* dst = smem + (j % kStages) * C::kStageB;
#pragma unroll 9
        for (int n = 0; n < C::kPerWave; ++n) {
          const int ii = w + NW * n;
          const char* src;
          DCP_LDS char* ldst;
          if (ii < C::kInst) {
            const int slot = ii * 64 + lane;
            int row, c;
            if constexpr (FP8) {
              row = slot / kF8RowCh;
              c = slot - row * kF8RowCh;
            } else {
              row = slot / kRowCh;
              const int pc = slot - row * kRowCh;
              c = (pc & ~7) | ((pc & 7) ^ swz(row));
            }
            const int tau = tau0 + row;
            int id = tau < ntok ? ids[tau / bs] : -1;
            src = a.kv + 16 * c;  // safe filler address (block 0, token 0)
            if (id >= 0 && id < a.ncb)
              src += static_cast<long long>(id) * a.block_stride_b +
                     static_cast<long long>(tau % bs) * a.token_stride_b;
            ldst = dst + ii * 1024;
          } else {
            src = a.kv;
            ldst = pad;
          }
          __builtin_amdgcn_global_load_lds(src, ldst, 16, 0, 0);
        }
        if constexpr (FP8) {
          const int tau = tau0 + (lane & 31);
          const int id = tau < ntok ? ids[tau / bs] : -1;
          const char* src = a.kv_scale;
          if (id >= 0 && id < a.ncb) src += 4 * (static_cast<long long>(id) * bs + tau % bs);
          __builtin_amdgcn_global_load_lds(
              src, smem + C::kScaleOff + ((j % kStages) * NW + w) * kScaleB, 4, 0, 0);
        }
      };
      // Rows of tile j that hold real tokens with usable block ids.
      auto valid_rows = [&](int j) -> unsigned long long {
        const int tau = j * kT + (lane & 31);
        bool ok = lane < 32 && tau < ntok;
        if (ok) {
          const int id = ids[tau / bs];
          ok = id >= 0 && id < a.ncb;
        }
        return __ballot(ok);
      };
      // fp8 tile j -> the fp16 tile the MFMAs read (buffer j & 1).
      auto widen = [&](int j, unsigned long long vm) {
        const DCP_LDS char* stg = smem + (j % kStages) * kF8TileB;
        DCP_LDS char* dstb = smem + C::kBf16Off + (j & 1) * kTileB;
        for (int u = threadIdx.x; u < kTileCh; u += NW * 64) {
          const int row = u / kRowCh;
          const int c = u - row * kRowCh;
          i32x4 wv = {0, 0, 0, 0};
          if ((vm >> row) & 1ull) {
            const i32x2 codes = *reinterpret_cast<const DCP_LDS i32x2*>(stg + row * kF8RowB + 8 * c);
            wv[0] = static_cast<int>(f8x2_to_f16x2<false>(static_cast<uint32_t>(codes[0])));
            wv[1] = static_cast<int>(f8x2_to_f16x2<true>(static_cast<uint32_t>(codes[0])));
            wv[2] = static_cast<int>(f8x2_to_f16x2<false>(static_cast<uint32_t>(codes[1])));
            wv[3] = static_cast<int>(f8x2_to_f16x2<true>(static_cast<uint32_t>(codes[1])));
          }
          *reinterpret_cast<DCP_LDS i32x4*>(dstb + chunk_off(row, c)) = wv;
        }
      };

      for (int j = 0; j < kStages - 1 && j < ntiles; ++j) issue(j);
      unsigned long long vm_next = 0;
      if constexpr (FP8) {
        // Widen tile 0 before the loop; tile k + 1 is widened while tile k is consumed.
        wait_tiles_after<NW, FP8>(min(kStages - 2, ntiles - 1));
        __syncthreads();
        widen(0, valid_rows(0));
        if (ntiles > 1) vm_next = valid_rows(1);
      }

      for (int k = 0; k < ntiles; ++k) {
        const DCP_LDS char* tile;
        unsigned long long vm_k;
        if constexpr (!FP8) {
          wait_tiles_after<NW, FP8>(min(kStages - 2, ntiles - 1 - k));
          vm_k = valid_rows(k);
          if (vm_k != 0xffffffffull) {
            // Zero the rows that were filled from the safe address, once every
            // wave's copies of this tile have landed.
            __syncthreads();
            DCP_LDS char* st = smem + (k % kStages) * kTileB;
            for (int u = threadIdx.x; u < kTileCh; u += NW * 64)
              if (!((vm_k >> (u / kRowCh)) & 1ull))
                *reinterpret_cast<DCP_LDS i32x4*>(st + 16 * u) = i32x4{0, 0, 0, 0};
          }
          __syncthreads();
          if (k + kStages - 1 < ntiles) issue(k + kStages - 1);
          tile = smem + (k % kStages) * kTileB;
        } else {
          // Tile k is already widened (previous iteration or prologue).
          vm_k = k == 0 ? valid_rows(0) : vm_next;
          if (k + 1 < ntiles) {
            wait_tiles_after<NW, FP8>(min(1, ntiles - 2 - k));
            vm_next = valid_rows(k + 1);
          }
          __syncthreads();
          if (k + kStages - 1 < ntiles) issue(k + kStages - 1);
          if (k + 1 < ntiles) widen(k + 1, vm_next);
          tile = smem + C::kBf16Off + (k & 1) * kTileB;
        }

        // ---- S^T = C_tile . Q^T : two 16-token M tiles, 18 K steps of 32 columns
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
          const int base = 128 * (kk >> 1);
          const auto a0 = __builtin_bit_cast(typename Elt<FP8>::vec,
              lds_read_b128(tile + ((kk & 1) ? a_odd0 : a_even0) + base));
          const auto a1 = __builtin_bit_cast(typename Elt<FP8>::vec,
              lds_read_b128(tile + ((kk & 1) ? a_odd1 : a_even1) + base));
          s0 = Elt<FP8>::mfma(a0, qf[kk], s0);
          s1 = Elt<FP8>::mfma(a1, qf[kk], s1);
        }

        // ---- online softmax for head h over tokens 4q4+i and 16+4q4+i
        float x[8], sig[8];
        const DCP_LDS float* sc =
            (const DCP_LDS float*)(smem + C::kScaleOff + ((k % kStages) * NW + w) * kScaleB);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r0 = 4 * q4 + i, r1 = 16 + 4 * q4 + i;
          sig[i] = FP8 ? sc[r0] : 1.f;
          sig[4 + i] = FP8 ? sc[r1] : 1.f;
          x[i] = ((vm_k >> r0) & 1ull) ? s0[i] * sig[i] * a.scale_log2 : -INFINITY;
          x[4 + i] = ((vm_k >> r1) & 1ull) ? s1[i] * sig[4 + i] * a.scale_log2 : -INFINITY;
        }
        float tmax = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, x[i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        // bf16 cache: probabilities may reach 2^8 before a rescale. fp8 cache:
        // rescale on any increase, so p <= 1 and p * scale stays in fp16 range.
        const bool raise = tmax > m_ref + (FP8 ? 0.f : 8.f);
        float alpha = 1.f;
        if (raise) {
          alpha = fast_exp2(m_ref - tmax);  // 0 on the first tile (m_ref = -inf)
          m_ref = tmax;
        }
        if (__ballot(raise)) {
#pragma unroll
          for (int mt = 0; mt < kVTiles; ++mt) acc[mt] *= alpha;
          l_run *= alpha;
        }
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        float psum = 0.f;
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = fast_exp2(x[2 * i] - m_use);
          const float p1 = fast_exp2(x[2 * i + 1] - m_use);
          const uint16_t b0 = Elt<FP8>::from_f32(FP8 ? p0 * sig[2 * i] : p0);
          const uint16_t b1 = Elt<FP8>::from_f32(FP8 ? p1 * sig[2 * i + 1] : p1);
          psum += p0 + p1;  // the normaliser keeps the fp32 probabilities
          pk[i] = static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16);
        }
        l_run += psum;
        const i32x4 pki = {static_cast<int>(pk[0]), static_cast<int>(pk[1]),
                           static_cast<int>(pk[2]), static_cast<int>(pk[3])};
        const auto pb = __builtin_bit_cast(typename Elt<FP8>::vec, pki);

        // ---- O^T += C_tile^T . P^T : 32 M tiles of 16 value columns, one K step
#pragma unroll
        for (int mt = 0; mt < kVTiles; ++mt) {
          const int base = 128 * (mt >> 2);
          const s16x4 lo = lds_read_tr(tile + t_off0[mt & 3] + base);
          const s16x4 hi = lds_read_tr(tile + t_off1[mt & 3] + base);
          const short __attribute__((ext_vector_type(8))) cat = {lo[0], lo[1], lo[2], lo[3],
                                                                 hi[0], hi[1], hi[2], hi[3]};
          acc[mt] = Elt<FP8>::mfma(__builtin_bit_cast(typename Elt<FP8>::vec, cat), pb, acc[mt]);
        }
      }
      __syncthreads();  // ring stages and ids are reused by the next window / piece
    }

    // ---- finalise the piece: normalise and store (O, LSE) in slot s + g
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse = l_tot > 0.f ? (m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
    const size_t slot = static_cast<size_t>(s) + g;
    float* orow = a.ws_o + (slot * a.Hq + h) * kV + 4 * q4;
#pragma unroll
    for (int mt = 0; mt < kVTiles; ++mt) *reinterpret_cast<f32x4*>(orow + 16 * mt) = acc[mt] * inv;
    if (q4 == 0) a.ws_lse[slot * a.Hq + h] = lse;
    pos = pe;
  }
}

}  // namespace

int mla_groups() { return kGroups; }

bool mla_supported(const dcp_attn_desc_t* d) {
  return d->kv_kind == DCP_KV_LATENT && d->num_kv_heads == 1 && d->qk_dim == kQK &&
         d->v_dim == kV && d->q_dtype == DCP_BF16 &&
         (d->kv_dtype == DCP_BF16 || d->kv_dtype == DCP_FP8_E4M3) &&
         (d->num_q_heads == 16 || d->num_q_heads == 32 || d->num_q_heads % 64 == 0) &&
         d->num_q_heads <= 256;
}

hipError_t launch_mla(const AttnLaunch& L, hipStream_t stream) {
  const dcp_attn_desc_t* d = L.desc;
  MlaArgs a;
  a.q = static_cast<const uint16_t*>(L.q);
  a.kv = static_cast<const char*>(L.k_cache);
  a.kv_scale = reinterpret_cast<const char*>(L.kv_scale);
  a.map = L.map;
  a.hdr = L.ws.header;
  a.seg_off = L.ws.seg_off;
  a.ws_o = L.ws.o;
  a.ws_lse = L.ws.lse;
  const int elt = d->kv_dtype == DCP_BF16 ? 2 : 1;
  a.block_stride_b = d->kv_block_stride * elt;
  a.token_stride_b = d->kv_token_stride * elt;
  a.S = L.S;
  a.ncb = d->num_cache_blocks;
  a.Hq = d->num_q_heads;
  a.scale_log2 = d->softmax_scale * kLog2e;
  const bool fp8 = d->kv_dtype == DCP_FP8_E4M3;
  const int heads = d->num_q_heads < kHeadsPerGroup ? d->num_q_heads : kHeadsPerGroup;
  const int nw = heads / 16;
  const dim3 grid(kGroups, d->num_q_heads / heads);
#define DCP_MLA_CASE(NW_)                                                                     \
  case NW_:                                                                                   \
    if (fp8)                                                                                  \
      hipLaunchKernelGGL((mla_partial_kernel<NW_, true>), grid, dim3(NW_ * 64), 0, stream, a); \
    else                                                                                      \
      hipLaunchKernelGGL((mla_partial_kernel<NW_, false>), grid, dim3(NW_ * 64), 0, stream, a); \
    break;
  switch (nw) {
    DCP_MLA_CASE(1)
    DCP_MLA_CASE(2)
    DCP_MLA_CASE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef DCP_MLA_CASE
  return hipGetLastError();
}

}  // namespace dcp
