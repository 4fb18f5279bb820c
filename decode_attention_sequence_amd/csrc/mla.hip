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
// Kernel design: one work group per CU processes one stream-K range of cache
// blocks for up to 64 query heads, split into HG groups of 16 heads, with
// 2 * HG waves (two per SIMD at 64 heads):
//  * 32-token latent tiles (36 KB bf16) are copied HBM -> LDS with 16-byte
//    direct-to-LDS loads through a 4-stage ring, three tiles in flight; every
//    wave issues a fixed number of copies per tile, so `s_waitcnt vmcnt(n)`
//    names exactly the tiles still in flight. Rows past the end of the range
//    (or with an unusable block id) are read from a safe in-pool address and
//    zero-filled once landed;
//  * scores: wave (g, t) computes S^T for the 16 tokens of half t of the tile
//    and the 16 heads of group g, S^T = C_tile . Q^T with
//    v_mfma_f32_16x16x32_bf16 (A = latent rows from LDS, B = the heads' query
//    rows held in registers for the whole range);
//  * online softmax in the exp2 domain: the two token halves exchange their
//    per-head maxima through LDS, so every wave tracks the same reference max
//    for every head; the reference only rises (and accumulators are
//    rescaled) when a tile's max exceeds it by more than 8, so rescales are
//    rare and probabilities stay <= 256;
//  * values: probabilities go through LDS once (8 bytes per lane) and wave w
//    computes O^T for its 512 / (2 HG)-column slice of the value dimension for
//    all heads, O^T += C_tile^T . P^T, the transposed A operand read from the
//    same LDS tile by ds_read_b64_tr_b16 -- every latent byte is fetched from
//    HBM once and serves both products, and each transposed byte is read once;
//  * LDS fragment reads are issued ahead of their MFMAs through register rings
//    (inline asm with explicit lgkmcnt waits tied to the destination registers);
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
constexpr int kT = 32;                     // tokens per tile
constexpr int kRowB = kQK * 2;             // 16-bit row bytes (1152)
constexpr int kRowCh = kRowB / 16;         // 16-byte chunks per row (72)
constexpr int kTileB = kT * kRowB;         // 36864
constexpr int kTileCh = kT * kRowCh;       // 2304
constexpr int kDmaInst = kTileCh / 64;     // 36 wave-wide copies per bf16 tile
constexpr int kKSteps = kQK / 32;          // 18
constexpr int kF8RowB = kQK;               // 576 code bytes per row
constexpr int kF8TileB = kT * kF8RowB;     // 18432
constexpr int kF8RowCh = kF8RowB / 16;     // 36
constexpr int kF8DmaInst = kF8TileB / 1024;  // 18
constexpr int kGroups = 256;               // work groups per head group (one per CU)
constexpr int kStages = 4;                 // copy ring depth
constexpr int kIdWin = 512;                // block ids staged in LDS at a time
constexpr int kPadB = 1024;                // landing pad for filler copies
constexpr int kSDist = 4;                  // S^T: K steps of A fragments read ahead
constexpr int kSRing = kSDist + 2;         // ring slot reused two MFMA steps after its use

// Row swizzle: logical chunk c of row r sits at (c & ~7) | ((c & 7) ^ swz(r)).
// With 1152-byte rows the two read patterns are 16 rows x one 16-byte chunk
// (MFMA A fragments, ds_read_b128) and 4 rows x 32 bytes per 16-lane group
// (ds_read_b64_tr_b16). Among the XOR swizzles measured on MI355X this one
// gives both patterns their full LDS rate (about 200 B/clk per CU for the
// 16-byte reads, 125 B/clk for the transposed reads; unswizzled rows reach 61).
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ (r & 1); }
__device__ __forceinline__ int chunk_off(int r, int c) {
  return r * kRowB + 16 * ((c & ~7) | ((c & 7) ^ swz(r)));
}

struct MlaArgs {
  const uint16_t* q;      // [B, Hq, 576] bf16 bits
  const char* kv;         // latent cache base
  const char* kv_scale;   // fp8: fp32, scale of slot j of block id at id * scale_bs + scale_ts * j
  int scale_bs, scale_ts;
  SegMap map;
  const PlanHeader* hdr;
  PlanSig sig;              // the plan's expected signature
  const int32_t* wg_start;  // [G + 1] block range of each work group
  const int32_t* wg_seg;    // [G + 1] segment of each range's first block
  const int32_t* seg_off;
  float* ws_o;
  float* ws_lse;
  long long block_stride_b;  // bytes
  long long token_stride_b;  // bytes
  const char* zero;         // 16 zero bytes (workspace)
  int S;
  int ncb;
  int Hq;   // query rows per sequence (q_len * heads per token)
  float scale_log2;
  Causal cz;
  bool causal;  // multi-token decode or explicit query positions: mask by position
};

template <int V>
struct IC {
  static constexpr int value = V;
};
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IC<I>{});
    static_for<I + 1, N>(f);
  }
}

// LDS fragment reads as inline asm: the compiler does not treat them as reads
// that may alias the in-flight direct-to-LDS copies (it would otherwise wait
// for every copy before each one), and the explicit waits below order them.
template <int OFF>
__device__ __forceinline__ void lds_b128(i32x4& r, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}
__device__ __forceinline__ void lds_store_b8(uint32_t addr, int v) {
  asm volatile("ds_write_b8 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
template <int OFF>
__device__ __forceinline__ void lds_b64(i32x2& r, uint32_t addr) {
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void lds_tr(i32x2& r, uint32_t addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}
// Wait until at most N LDS operations are outstanding; the operand ties the
// awaited registers so their consumers cannot move above the wait.
template <int N, class T0>
__device__ __forceinline__ void wait_lgkm(T0& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
template <int N, class T0, class T1>
__device__ __forceinline__ void wait_lgkm(T0& a, T1& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}

// Work-group barrier that orders LDS accesses only. __syncthreads() also
// completes every earlier memory operation of the wave, which includes the
// direct-to-LDS copies still in flight, so it would drain the prefetch
// pipeline at every barrier. Here each wave waits for its own LDS accesses;
// copy completion is awaited explicitly (wait_vm) before a tile is read.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The value held by the lane 16 (or 32) positions away, through the gfx950
// row-swap permutes (plain VALU, no LDS round trip). With both operands set to
// x, the swap returns x of this lane and x of its partner in some order, so
// only symmetric combinations (max, sum) are formed from the pair.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maxima of operands that are never NaN (finite scores, or -inf for masked
// rows): plain v_max / v_max3, without the canonicalising maxes the compiler
// puts in front of fmaxf.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax8(const float* x) {
  return vmax3(vmax3(x[0], x[1], x[2]), vmax3(x[3], x[4], x[5]), vmax(x[6], x[7]));
}
__device__ __forceinline__ float vmax_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float vmax_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The largest of |a|, |b|, |c| (operand modifiers on v_max3).
__device__ __forceinline__ float vmax3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// A value every lane holds identically, moved to a scalar register.
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Wait until at most N vector-memory operations of this wave are in flight.
// Issued through the builtin, not inline asm: the compiler's own wait
// insertion then knows which loads are complete. (After an asm wait it still
// treats earlier loads as pending and adds a vmcnt(0) before some later
// register reuse -- in the tile loop, which would drain every copy in flight.)
// The empty asm keeps memory accesses from moving across the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8
  // (expcnt and lgkmcnt at their maximum: no wait on them).
  constexpr int kEnc = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
  __builtin_amdgcn_s_waitcnt(kEnc);
  asm volatile("" ::: "memory");
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// e4m3 codes -> fp16, exact: every e4m3 value (4 significant bits, |x| <= 448,
// down to 2^-9) is an fp16 normal or subnormal number.
template <bool HI>
__device__ __forceinline__ uint32_t f8x2_to_f16x2(uint32_t codes) {
  f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes), HI);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f[0], f[1]));
}

// MFMA element type: bf16 for a bf16 cache; fp16 for an fp8 cache, whose codes
// widen to fp16 exactly and whose probability-times-scale products then keep
// 11 significant bits instead of 8.
template <bool FP8>
struct Elt;
template <>
struct Elt<false> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 mfma(i32x4 a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vec, a), b, c, 0, 0, 0);
  }
  // two fp32 -> packed pair, round to nearest even (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
  }
  static __device__ __forceinline__ vec from_bf16(bf16x8 v) { return v; }
};
template <>
struct Elt<true> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 mfma(i32x4 a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(vec, a), b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, f16x2));
  }
  // bf16 -> fp16 (exact inside the fp16 range).
  static __device__ __forceinline__ vec from_bf16(bf16x8 v) {
    vec r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<_Float16>(static_cast<float>(v[i]));
    return r;
  }
  // bf16 * 2^-e -> fp16 (the power of two is exact).
  static __device__ __forceinline__ vec from_bf16_pow2(bf16x8 v, int e) {
    vec r;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r[i] = static_cast<_Float16>(__builtin_amdgcn_ldexpf(static_cast<float>(v[i]), -e));
    return r;
  }
};

// fp8 caches run both products on fp16 MFMAs, whose operands have a narrow
// exponent range. Two powers of two keep every finite query and every token
// scale up to 2^64 inside it, exactly:
//  * query: each head's query is multiplied by 2^-e with e the exponent of
//    its largest magnitude (so |q| < 1, and components down to 2^-14 of the
//    largest keep full precision); the score scale takes 2^e back in fp32;
//  * probability x scale: for any set of tokens whose largest score is x_max
//    and whose largest scale is below 2^E (E its exponent), every
//    p * sigma <= 2^(x_max + E - m) against reference m. The reference rises
//    on the largest such bound over the lanes (or halves) holding a head's
//    tokens rather than on the largest score, which keeps every fp16 weight
//    p * sigma below 2^kRaise whatever sigma is; the fp32 probabilities p (and
//    their sum) take the shift 2^-E, which stays far inside fp32 for scales in
//    [2^-64, 2^64] (E is clamped at -64 so that smaller scales cannot push the
//    sum towards overflow).
__device__ __forceinline__ int max_exponent_head(float amax) {
  return __builtin_amdgcn_frexp_expf(amax);  // amax < 2^e (0 for amax = 0)
}
__device__ __forceinline__ float scale_exponent(float sig_max) {
  const int e = __builtin_amdgcn_frexp_expf(sig_max);
  return static_cast<float>(e < -64 ? -64 : e);
}

// Static configuration: HG groups of 16 heads, 2 * HG waves.
template <int HG, bool FP8>
struct Cfg {
  static constexpr int NW = 2 * HG;
  static constexpr int kMT = 32 / NW;                          // value M tiles per wave
  static constexpr int kInst = FP8 ? kF8DmaInst : kDmaInst;
  static constexpr int kPerWave = (kInst + NW - 1) / NW;      // tile copies per wave (at most)
  // Vector-memory operations per tile of a wave with kPerWave copies and of
  // one with a copy fewer (bf16: the last round of copies covers only the first
  // kInst % NW waves). The fp8 path keeps one count: its waves all issue
  // kPerWave copies (the surplus ones land in the pad) plus the scale copy.
  static constexpr int kOpsHi = kPerWave + (FP8 ? 1 : 0);
  static constexpr int kOpsLo = (FP8 || kInst % NW == 0) ? kOpsHi : kOpsHi - 1;
  static constexpr int kHiWaves = (FP8 || kInst % NW == 0) ? NW : kInst % NW;
  static constexpr int kStageB = FP8 ? kF8TileB : kTileB;
  // LDS is two arrays. The copies write only `ring` (tile stages, fp8 scales,
  // the filler pad); everything the waves store themselves lives in `aux`.
  // As separate objects the compiler can prove that a store to or a load from
  // `aux` never aliases an in-flight copy, so it adds no wait for the copies
  // before such accesses (which would drain the whole prefetch pipeline).
  static constexpr int kScaleOff = kStages * kStageB;          // fp8: kStages x 256 B
  static constexpr int kPadOff = kScaleOff + (FP8 ? kStages * 256 : 0);
  static constexpr int kRingB = kPadOff + kPadB;
  static constexpr int kF16Off = 0;                            // fp8: two fp16 tiles
  static constexpr int kPOff = FP8 ? 2 * kTileB : 0;
  static constexpr int kMxOff = kPOff + HG * 64 * 16;          // [2][16][4] floats
  static constexpr int kLsumOff = kMxOff + 2 * 16 * 4 * 4;     // [2][2][64] floats
  static constexpr int kIdsOff = kLsumOff + 4 * 64 * 4;
  static constexpr int kFlagOff = kIdsOff + kIdWin * 4;        // one byte per wave
  static constexpr int kAuxB = kFlagOff + 16;
  static_assert(kRingB + kAuxB <= 160 * 1024, "LDS budget");
};

// Wait until at most n_after tiles (OPS operations each) issued after the
// awaited one are still in flight. The hardware counter saturates at 63, so
// larger counts are clamped, which only waits for more.
// MAXN: the largest n_after a caller passes (larger values wait as for MAXN).
template <int OPS, int MAXN = 2>
__device__ __forceinline__ void wait_tiles_after_n(int n_after) {
  static_assert(MAXN >= 1 && MAXN <= 3, "one to three later tiles");
  constexpr int k1 = OPS > 63 ? 63 : OPS;
  constexpr int k2 = 2 * OPS > 63 ? 63 : 2 * OPS;
  constexpr int k3 = 3 * OPS > 63 ? 63 : 3 * OPS;
  if (n_after <= 0) wait_vm<0>();
  else if (MAXN == 1 || n_after == 1) wait_vm<k1>();
  else if (MAXN == 2 || n_after == 2) wait_vm<k2>();
  else wait_vm<k3>();
}

// Location of copy slot `slot` of a tile: row and logical 16-byte chunk.
template <bool FP8>
__device__ __forceinline__ void slot_row_chunk(int slot, int& row, int& c) {
  if constexpr (FP8) {
    row = slot / kF8RowCh;
    c = slot - row * kF8RowCh;
  } else {
    row = slot / kRowCh;
    const int pc = slot - row * kRowCh;
    c = (pc & ~7) | ((pc & 7) ^ swz(row));
  }
}

// BS32: every block holds a multiple of 32 tokens, so a tile lies inside one
// block and its copies are a uniform base plus fixed per-lane offsets.
template <int HG, bool FP8, bool BS32>
__global__ __launch_bounds__(2 * HG * 64) void mla_partial_kernel(MlaArgs a) {
  using C = Cfg<HG, FP8>;
  using E = Elt<FP8>;
  constexpr int NW = C::NW;
  constexpr int kMT = C::kMT;
  __shared__ __attribute__((aligned(16))) char ring_raw[C::kRingB];
  __shared__ __attribute__((aligned(16))) char aux_raw[C::kAuxB];
  DCP_LDS char* ring = (DCP_LDS char*)ring_raw;
  DCP_LDS char* aux = (DCP_LDS char*)aux_raw;
  DCP_LDS int* ids = (DCP_LDS int*)(aux + C::kIdsOff);
  DCP_LDS float* mx = (DCP_LDS float*)(aux + C::kMxOff);
  DCP_LDS float* lsum = (DCP_LDS float*)(aux + C::kLsumOff);
  DCP_LDS char* pad = ring + C::kPadOff;
  const uint32_t ring_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
  const uint32_t aux_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(aux));

  const int lane = threadIdx.x & 63;
  const int w = wave_uniform(threadIdx.x >> 6);
  const int hg = w % HG;   // head group of this wave's scores
  const int th = w / HG;   // token half of this wave's scores
  const int q4 = lane >> 4;
  const int l16 = lane & 15;
  const int g = xcd_logical_group(blockIdx.x, kGroups);
  const int head0 = blockIdx.y * 16 * HG;
  if (!plan_matches(a.sig, a.hdr)) return;  // no plan of this launch's shape
  int pos = a.wg_start[g];
  const int end = a.wg_start[g + 1];
  if (pos >= end) return;
  int s = a.wg_seg[g];
  const int bs = a.map.bs;
  const int h_s = head0 + 16 * hg + l16;  // head of this lane's scores
  const uint32_t flags_addr = aux_addr + C::kFlagOff;
  // Wait for the copies of a tile, given how many tiles were issued after it.
  const bool hi_wave = w < C::kHiWaves;
  auto wait_tiles = [&](int n_after) {
    if (hi_wave) wait_tiles_after_n<C::kOpsHi>(n_after);
    else wait_tiles_after_n<C::kOpsLo>(n_after);
  };

  // ---- per-lane constant offsets
  // S^T A fragment: row 16th + l16, chunk 4kk + q4 (even / odd kk).
  const int a_row = 16 * th + l16;
  const uint32_t a_even = a_row * kRowB + 16 * (q4 ^ swz(a_row));
  const uint32_t a_odd = a_row * kRowB + 16 * ((4 + q4) ^ swz(a_row));
  // O^T transposed A fragment: lane (k = l16/4, m = l16%4) points at rows
  // 4q4 + k (tokens of half 0) and 16 + 4q4 + k (half 1), value columns
  // v = vbase + 16mt + 4m .. +3, i.e. chunk vbase/8 + 2mt + m/2.
  const int t_k = l16 >> 2, t_m = l16 & 3;
  const int t_row0 = 4 * q4 + t_k, t_row1 = 16 + 4 * q4 + t_k;
  const int vbase = 16 * kMT * w;
  uint32_t t_off[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 2 * j + (t_m >> 1);
    const int grp = 128 * (vbase / 64);  // the 8-chunk group holding value column vbase
    t_off[j] = grp + t_row0 * kRowB + 16 * (c ^ swz(t_row0)) + 8 * (t_m & 1);
    t_off[4 + j] = grp + t_row1 * kRowB + 16 * (c ^ swz(t_row1)) + 8 * (t_m & 1);
  }
  // Copy offsets of this lane within a tile (BS32 path).
  int32_t cp_off[C::kPerWave];
#pragma unroll
  for (int n = 0; n < C::kPerWave; ++n) {
    const int ii = w + NW * n;
    int row = 0, c = 0;
    if (ii < C::kInst) slot_row_chunk<FP8>(ii * 64 + lane, row, c);
    cp_off[n] = static_cast<int32_t>(row * a.token_stride_b) + 16 * c;
  }

  if (threadIdx.x < 16) aux[C::kFlagOff + threadIdx.x] = 0;  // unused vote bytes stay 0
  while (pos < end) {
    while (a.seg_off[s + 1] <= pos) ++s;
    const int seg_a = a.seg_off[s];
    const int pe = min(end, a.seg_off[s + 1]);
    const Piece p = make_piece(a.map, s, pos - seg_a, pe - seg_a);
    const int32_t* trow = a.map.table + static_cast<size_t>(p.b) * a.map.width;
    const long long qpos0 = a.causal ? first_query_pos(a.cz, a.map, p.b) : 0;

    // Query fragments (B operand of S^T): head h_s, columns 32kk + 8q4 .. +7.
    typename E::vec qf[kKSteps];
    float qsl = a.scale_log2;  // score scale (log2 units) of this lane's head
    {
      const uint16_t* qrow = a.q + (static_cast<size_t>(p.b) * a.Hq + h_s) * kQK + 8 * q4;
      if constexpr (FP8) {
        // fp16 operands: the head's query scaled by a power of two into (-1, 1)
        bf16x8 qv[kKSteps];
        float qm = 0.f;
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
          qv[kk] = *reinterpret_cast<const bf16x8*>(qrow + 32 * kk);
#pragma unroll
          for (int i = 0; i < 8; ++i) qm = fmaxf(qm, fabsf(static_cast<float>(qv[kk][i])));
        }
        const int qe = max_exponent_head(max_xor32(max_xor16(qm)));
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) qf[kk] = E::from_bf16_pow2(qv[kk], qe);
        qsl = __builtin_amdgcn_ldexpf(a.scale_log2, qe);
      } else {
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk)
          qf[kk] = E::from_bf16(*reinterpret_cast<const bf16x8*>(qrow + 32 * kk));
      }
    }
    f32x4 acc[kMT][HG];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < HG; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Reference max (log2 units) of heads 16nt + l16, identical in every wave.
    float m_ref[HG];
#pragma unroll
    for (int nt = 0; nt < HG; ++nt) m_ref[nt] = -INFINITY;
    float l_run = 0.f;  // sum of this lane's probabilities for head h_s
    float l_rnd = 0.f;  // bf16: the same sum over the probabilities as rounded for P^T

    // Windows of at most kIdWin blocks share one LDS copy of their block ids.
    for (int wb = p.i0; wb < p.i1; wb += kIdWin) {
      const int we = min(p.i1, wb + kIdWin);
      const int ntok = (we - wb) * bs - (we == p.i1 ? (p.i1 - p.i0) * bs - p.ntok : 0);
      for (int i = threadIdx.x; i < we - wb; i += NW * 64)
        ids[i] = trow[p.r + a.map.D * (wb + i)];
      wait_vm<0>();
      __syncthreads();
      const int ntiles = (ntok + kT - 1) / kT;

      // Rows of tile j that hold real tokens with usable block ids.
      auto valid_rows = [&](int j) -> unsigned long long {
        const int tau0 = j * kT;
        if constexpr (BS32) {
          const int id = ids[tau0 / bs];
          const int n = min(kT, ntok - tau0);
          return (id >= 0 && id < a.ncb) ? ((1ull << n) - 1) : 0ull;
        } else {
          const int tau = tau0 + (lane & 31);
          bool ok = lane < 32 && tau < ntok;
          if (ok) {
            const int id = ids[tau / bs];
            ok = id >= 0 && id < a.ncb;
          }
          return __ballot(ok);
        }
      };

      // Multi-token decode: rows of tile j visible to this wave's query token
      // (its 16 heads belong to one token), by global position.
      auto causal_rows = [&](int j) -> unsigned long long {
        const int tau0 = j * kT;
        const long long lim = qpos0 + (head0 + 16 * hg) / a.cz.hq;
        if constexpr (BS32) {
          const int col = p.r + a.map.D * (wb + tau0 / bs);
          const long long vis = lim - global_pos(a.cz, col, bs, tau0 % bs) + 1;
          return vis >= 32 ? 0xffffffffull : (vis <= 0 ? 0ull : ((1ull << vis) - 1));
        } else {
          const int tau = tau0 + (lane & 31);
          const int col = p.r + a.map.D * (wb + tau / bs);
          return __ballot(lane < 32 && global_pos(a.cz, col, bs, tau % bs) <= lim);
        }
      };

      // BS32: source of tile j, one block for the whole tile. An unusable id
      // reads block 0 instead (the rows are zeroed after landing).
      auto tile_src = [&](int j) -> const char* {
        const int tau0 = j * kT;
        const int id = wave_uniform(ids[tau0 / bs]);
        const char* base = a.kv;
        if (id >= 0 && id < a.ncb)
          base += static_cast<long long>(id) * a.block_stride_b +
                  static_cast<long long>(tau0 % bs) * a.token_stride_b;
        return base;
      };
      // BS32: copy n of this wave for tile j (16 bytes per lane). A bf16 wave
      // whose last round falls past the tile skips it; fp8 waves send it to the pad.
      auto copy_one = [&](auto nc, const char* base, int j) {
        constexpr int n = decltype(nc)::value;
        const int ii = w + NW * n;
        if (!FP8 && n == C::kPerWave - 1 && ii >= C::kInst) return;
        // (Operands bound to locals: with the expressions inline in the
        // builtin's argument list the host pass drops this kernel's stub.)
        const char* src = base + cp_off[n];
        DCP_LDS char* ldst = ii < C::kInst ? ring + (j % kStages) * C::kStageB + ii * 1024 : pad;
        __builtin_amdgcn_global_load_lds(src, ldst, 16, 0, kCopyPolicy);
      };

      // Copy tile j of this window into ring stage j % kStages. Every wave
      // issues its fixed number of vector-memory operations per tile.
      auto issue = [&](int j) {
        const int tau0 = j * kT;
        DCP_LDS char* dst = ring + (j % kStages) * C::kStageB;
        if constexpr (BS32) {
          const char* base = tile_src(j);
          static_for<0, C::kPerWave>([&](auto nc) { copy_one(nc, base, j); });
        } else {
#pragma unroll
          for (int n = 0; n < C::kPerWave; ++n) {
            const int ii = w + NW * n;
            if (!FP8 && ii >= C::kInst) continue;
            const char* src = a.kv;
            DCP_LDS char* ldst = pad;
            if (ii < C::kInst) {
              int row, c;
              slot_row_chunk<FP8>(ii * 64 + lane, row, c);
              src = a.kv + 16 * c;  // safe filler address (block 0, token 0)
              const int tau = tau0 + row;
              const int id = tau < ntok ? ids[tau / bs] : -1;
              if (id >= 0 && id < a.ncb)
                src += static_cast<long long>(id) * a.block_stride_b +
                       static_cast<long long>(tau % bs) * a.token_stride_b;
              ldst = dst + ii * 1024;
            }
            __builtin_amdgcn_global_load_lds(src, ldst, 16, 0, kCopyPolicy);
          }
        }
        if constexpr (FP8) {
          // Wave 0 copies the tile's 32 token scales; the others pad their count.
          const int tau = tau0 + (lane & 31);
          const int id = tau < ntok ? ids[tau / bs] : -1;
          const char* src = a.kv_scale;
          if (id >= 0 && id < a.ncb)
            src += 4 * (static_cast<long long>(id) * a.scale_bs + static_cast<long long>(a.scale_ts) * (tau % bs));
          __builtin_amdgcn_global_load_lds(
              src, w == 0 ? ring + C::kScaleOff + (j % kStages) * 256 : pad, 4, 0, 0);
        }
      };
      // fp8 tile j -> the fp16 tile the MFMAs read (buffer j & 1).
      auto widen = [&](int j, unsigned long long vm) {
        const uint32_t stg = ring_addr + (j % kStages) * kF8TileB;
        DCP_LDS char* dstb = aux + C::kF16Off + (j & 1) * kTileB;
        for (int u = threadIdx.x; u < kTileCh; u += NW * 64) {
          const int row = u / kRowCh;
          const int c = u - row * kRowCh;
          i32x4 wv = {0, 0, 0, 0};
          if ((vm >> row) & 1ull) {
            i32x2 codes;
            lds_b64<0>(codes, stg + row * kF8RowB + 8 * c);
            wait_lgkm<0>(codes);
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
        wait_tiles(min(kStages - 2, ntiles - 1));
        lds_barrier();
        widen(0, valid_rows(0));
        if (ntiles > 1) vm_next = valid_rows(1);
      }

      for (int k = 0; k < ntiles; ++k) {
        uint32_t tile;
        unsigned long long vm_k;
        // bf16 with whole-tile blocks: the copies of tile k + kStages - 1 are
        // spread over the score MFMAs below instead of issued in one burst, so
        // the waves do not all stall on a full memory queue at the same time.
        constexpr bool kSpread = BS32 && !FP8;
        const bool do_issue = k + kStages - 1 < ntiles;
        const char* nsrc = nullptr;
        if constexpr (!FP8) {
          wait_tiles(min(kStages - 2, ntiles - 1 - k));
          vm_k = valid_rows(k);
          if (vm_k != 0xffffffffull) {
            // Zero the rows that were filled from the safe address, once every
            // wave's copies of this tile have landed.
            lds_barrier();
            DCP_LDS char* st = ring + (k % kStages) * kTileB;
            for (int u = threadIdx.x; u < kTileCh; u += NW * 64)
              if (!((vm_k >> (u / kRowCh)) & 1ull))
                *reinterpret_cast<DCP_LDS i32x4*>(st + 16 * u) = i32x4{0, 0, 0, 0};
          }
          lds_barrier();
          if constexpr (kSpread) {
            if (do_issue) nsrc = tile_src(k + kStages - 1);
          } else {
            if (do_issue) issue(k + kStages - 1);
          }
          tile = ring_addr + (k % kStages) * kTileB;
        } else {
          // Tile k is already widened (previous iteration or prologue).
          vm_k = k == 0 ? valid_rows(0) : vm_next;
          if (k + 1 < ntiles) {
            wait_tiles(min(1, ntiles - 2 - k));
            vm_next = valid_rows(k + 1);
          }
          lds_barrier();
          if (do_issue) issue(k + kStages - 1);
          if (k + 1 < ntiles) widen(k + 1, vm_next);
          tile = aux_addr + C::kF16Off + (k & 1) * kTileB;
        }

        // ---- S^T for the 16 tokens of half th and heads of group hg: 18 K steps,
        // A fragments read kSDist steps ahead, two accumulator chains.
        const uint32_t ae = tile + a_even, ao = tile + a_odd;
        i32x4 ra[kSRing];
        auto s_issue = [&](auto kc) {
          constexpr int kk = decltype(kc)::value;
          constexpr int off = 128 * (kk >> 1);
          if constexpr (kk & 1) lds_b128<off>(ra[kk % kSRing], ao);
          else lds_b128<off>(ra[kk % kSRing], ae);
        };
        static_for<0, kSDist>(s_issue);
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
        static_for<0, kKSteps>([&](auto kc) {
          constexpr int kk = decltype(kc)::value;
          if constexpr (kk + kSDist < kKSteps) s_issue(IC<kk + kSDist>{});
          constexpr int ahead = kk + kSDist < kKSteps ? kSDist : kKSteps - 1 - kk;
          wait_lgkm<ahead>(ra[kk % kSRing]);
          if constexpr (kk & 1) sb = E::mfma(ra[kk % kSRing], qf[kk], sb);
          else sa = E::mfma(ra[kk % kSRing], qf[kk], sa);
          if constexpr (kSpread) {
            // copies n in [n0, n1) go out after this K step
            constexpr int n0 = kk * C::kPerWave / kKSteps;
            constexpr int n1 = (kk + 1) * C::kPerWave / kKSteps;
            if (do_issue)
              static_for<n0, n1>([&](auto nc) { copy_one(nc, nsrc, k + kStages - 1); });
          }
        });
        const f32x4 sv = sa + sb;

        // ---- softmax, part 1: this half's max per head, exchanged through LDS
        // (vm_k, shared by every wave, also drives the cooperative zeroing; the
        // causal rows differ per wave and only mask this wave's scores)
        const unsigned long long vm_s = a.causal ? vm_k & causal_rows(k) : vm_k;
        float x[4], sig[4];
        f32x4 sc4 = {1.f, 1.f, 1.f, 1.f};
        if constexpr (FP8) {
          // The four token scales of this lane's score rows (copied by the engine,
          // so read with an explicit wait rather than a plain load).
          i32x4 raw;
          lds_b128<0>(raw, ring_addr + C::kScaleOff + (k % kStages) * 256 + 4 * (16 * th + 4 * q4));
          wait_lgkm<0>(raw);
          sc4 = __builtin_bit_cast(f32x4, raw);
        }
        float smax = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * th + 4 * q4 + i;
          const bool v = (vm_s >> r) & 1ull;
          sig[i] = sc4[i];
          x[i] = v ? sv[i] * sig[i] * qsl : -INFINITY;
          smax = fmaxf(smax, v ? fabsf(sig[i]) : 0.f);
        }
        float hmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        hmax = max_xor32(max_xor16(hmax));
        // fp8: the half's log2 bound of p * sigma against reference 0 (the
        // reference then rises on it, so every p * sigma stays <= 1)
        if constexpr (FP8) hmax += scale_exponent(max_xor32(max_xor16(smax)));
        // P^T fragment half of this wave: tokens 16th + 4q4 + i of head h_s.
        auto store_p = [&](const float* pv) -> i32x2 {
          const uint32_t lo = E::pack2(FP8 ? pv[0] * sig[0] : pv[0], FP8 ? pv[1] * sig[1] : pv[1]);
          const uint32_t hi = E::pack2(FP8 ? pv[2] * sig[2] : pv[2], FP8 ? pv[3] * sig[3] : pv[3]);
          const i32x2 pk = {static_cast<int>(lo), static_cast<int>(hi)};
          *reinterpret_cast<DCP_LDS i32x2*>(aux + C::kPOff + ((hg * 64 + lane) * 2 + th) * 8) = pk;
          return pk;
        };
        // bf16: the rounded probabilities' sum, for the output normalisation
        auto add_rounded = [&](i32x2 pk, float c) -> float {
          if constexpr (FP8) return c;
          return add_bf16x2(static_cast<uint32_t>(pk[1]), add_bf16x2(static_cast<uint32_t>(pk[0]), c));
        };
        // bf16 cache: probabilities may reach 2^8 before the reference max of a
        // head is raised. fp8 cache: it is raised on any increase of the
        // shifted maximum, so p * scale <= 1.
        constexpr float kRaise = FP8 ? 0.f : 8.f;
        float p[4];
        bool slow = true;
        if constexpr (!FP8) {
          // Fast path: probabilities against the current reference max, and one
          // vote per wave on whether any head of its group needs a raise. Only
          // when some wave votes yes do the waves exchange their maxima.
          float m_own = m_ref[0];
#pragma unroll
          for (int nt = 1; nt < HG; ++nt)
            if (nt == hg) m_own = m_ref[nt];
          const float m_use = m_own == -INFINITY ? 0.f : m_own;
#pragma unroll
          for (int i = 0; i < 4; ++i) p[i] = fast_exp2(x[i] - m_use);
          const i32x2 pk = store_p(p);
          const bool need = __ballot(hmax > m_own + kRaise) != 0ull;
          // (The vote is written and read with explicit-wait asm: as plain LDS
          // accesses the compiler waits for every in-flight copy first.)
          if (lane == 0) lds_store_b8(flags_addr + w, need ? 1 : 0);
          lds_barrier();
          i32x2 votes;
          lds_b64<0>(votes, flags_addr);
          wait_lgkm<0>(votes);
          slow = wave_uniform((votes[0] | votes[1]) != 0);
          if (!slow) {
            l_run += (p[0] + p[1]) + (p[2] + p[3]);
            l_rnd = add_rounded(pk, l_rnd);
          }
        }
        if (slow) {  // some wave votes for a raise (always, for fp8)
          if (q4 == 0) mx[(th * 16 + l16) * 4 + hg] = hmax;
          lds_barrier();

          // Exchange the halves' maxima; every wave then raises the reference
          // max of heads 16nt + l16 where needed, identically in every wave.
          float alpha[HG];
          bool any_raise = false;
          {
            const f32x4 m0 = *reinterpret_cast<const DCP_LDS f32x4*>(mx + l16 * 4);
            const f32x4 m1 = *reinterpret_cast<const DCP_LDS f32x4*>(mx + (16 + l16) * 4);
#pragma unroll
            for (int nt = 0; nt < HG; ++nt) {
              const float tmax = fmaxf(m0[nt], m1[nt]);
              const bool raise = tmax > m_ref[nt] + kRaise;
              alpha[nt] = raise ? fast_exp2(m_ref[nt] - tmax) : 1.f;  // 0 when m_ref = -inf
              m_ref[nt] = raise ? tmax : m_ref[nt];
              any_raise |= raise;
            }
          }
          float m_own = m_ref[0], a_own = alpha[0];
#pragma unroll
          for (int nt = 1; nt < HG; ++nt)
            if (nt == hg) { m_own = m_ref[nt]; a_own = alpha[nt]; }
          const float m_use = m_own == -INFINITY ? 0.f : m_own;
#pragma unroll
          for (int i = 0; i < 4; ++i) p[i] = fast_exp2(x[i] - m_use);
          l_run = l_run * a_own + ((p[0] + p[1]) + (p[2] + p[3]));
          l_rnd = add_rounded(store_p(p), l_rnd * a_own);
          lds_barrier();
          if (__ballot(any_raise)) {
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
              for (int nt = 0; nt < HG; ++nt) acc[mt][nt] *= alpha[nt];
          }
        }

        // ---- O^T += C_tile^T . P^T over this wave's value slice, all head groups
        i32x4 pb[HG];
        const uint32_t pbase = aux_addr + C::kPOff + lane * 16;
        static_for<0, HG>([&](auto nc) {
          constexpr int nt = decltype(nc)::value;
          lds_b128<nt * 1024>(pb[nt], pbase);
        });
        uint32_t tb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) tb[j] = tile + t_off[j];
        constexpr int kPD = kMT < 4 ? kMT : 4;  // M tiles of transposed reads in flight
        i32x2 rlo[kPD + 2], rhi[kPD + 2];
        auto p_issue = [&](auto mc) {
          constexpr int mt = decltype(mc)::value;
          constexpr int off = 128 * (mt >> 2);
          lds_tr<off>(rlo[mt % (kPD + 2)], tb[mt & 3]);
          lds_tr<off>(rhi[mt % (kPD + 2)], tb[4 + (mt & 3)]);
        };
        static_for<0, kPD>(p_issue);
        static_for<0, kMT>([&](auto mc) {
          constexpr int mt = decltype(mc)::value;
          if constexpr (mt + kPD < kMT) p_issue(IC<mt + kPD>{});
          constexpr int ahead = mt + kPD < kMT ? kPD : kMT - 1 - mt;
          wait_lgkm<2 * ahead>(rlo[mt % (kPD + 2)], rhi[mt % (kPD + 2)]);
          const i32x4 av = {rlo[mt % (kPD + 2)][0], rlo[mt % (kPD + 2)][1],
                            rhi[mt % (kPD + 2)][0], rhi[mt % (kPD + 2)][1]};
          static_for<0, HG>([&](auto nc) {
            constexpr int nt = decltype(nc)::value;
            acc[mt][nt] = E::mfma(av, __builtin_bit_cast(typename E::vec, pb[nt]), acc[mt][nt]);
          });
        });
      }
      __syncthreads();  // ring stages and ids are reused by the next window / piece
    }

    // ---- finalise the piece: normalise and store (O, LSE) in slot s + g
    // (bf16: the output is normalised by the rounded probabilities' sum, the
    // LSE takes the fp32 sum)
    const float l_h = sum_xor32(sum_xor16(l_run));
    const float l_o = FP8 ? l_h : sum_xor32(sum_xor16(l_rnd));
    if (q4 == 0) {
      lsum[th * 64 + 16 * hg + l16] = l_h;
      lsum[128 + th * 64 + 16 * hg + l16] = l_o;
    }
    __syncthreads();
    const size_t slot = static_cast<size_t>(s) + g;
#pragma unroll
    for (int nt = 0; nt < HG; ++nt) {
      const float l_tot = lsum[16 * nt + l16] + lsum[64 + 16 * nt + l16];
      const float l_out = lsum[128 + 16 * nt + l16] + lsum[192 + 16 * nt + l16];
      const float inv = l_out > 0.f ? 1.f / l_out : 0.f;
      float* orow = a.ws_o + (slot * a.Hq + head0 + 16 * nt + l16) * kV + vbase + 4 * q4;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) *reinterpret_cast<f32x4*>(orow + 16 * mt) = acc[mt][nt] * inv;
      if (th == 0 && nt == hg && q4 == 0)
        a.ws_lse[slot * a.Hq + h_s] = l_tot > 0.f ? (m_ref[nt] + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
    pos = pe;
  }
}

// ---------------------------------------------------------------------------
// 64 heads per work group, blocks holding a multiple of 32 tokens:
// producer / consumer form with one barrier per tile.
//  * Waves 0-3 ("score waves") own 16 heads each. For tile t they compute S^T
//    over all 32 tokens, run the online softmax of their own heads (so no
//    maxima cross waves) and write P^T and any rescale factors to LDS.
//  * Waves 4-7 ("value waves") own 128 value columns each, for all 64 heads,
//    and accumulate O^T += C^T . P^T for tile t - 1 in the same step.
//  * Waves w and w + 4 share a SIMD, so one wave's softmax, LDS waits and
//    copy issue overlap the other's MFMAs.
//  * The copy ring holds tile t (scores), tile t - 1 (values) and the tiles
//    after t in flight (two of 36 KB for bf16, four of 18 KB for fp8); the
//    copies of the next tile go out during step t, spread over both kinds of
//    waves' MFMA loops.
//  * The tiles of a work group's whole range form one stream: a window of
//    the range (up to kMaxTiles tiles of up to kMaxPieces segments) gets a
//    tile table in LDS, and segment boundaries inside a window are handled
//    per tile (state reset, query reload, result store) without draining the
//    copy pipeline.
//  * fp8 cache: the score waves are pipelined one tile deeper -- during step
//    t they compute S^T of tile t and, interleaved with those MFMAs, the
//    softmax of tile t - 1 (whose scores they kept in registers); the value
//    waves work on tile t - 2. The softmax latency then overlaps the score
//    MFMAs instead of following them. Seven ring stages keep four tiles in
//    flight; every wave issues the same three 16-byte copies per tile (code
//    rows, the token scales, or a filler into a pad), also past the end of a
//    window, so the copy loops have no branches and the copy waits are
//    constant.
//  * fp8 cache: each tile carries its 32 token scales. The codes are widened
//    to fp16 in registers right after each LDS fragment read (exact; see
//    f8x8_to_f16x8) and both products run on v_mfma_f32_16x16x32_f16. A score
//    lane reads one 16-byte chunk of its row per read, which covers two K
//    steps (the query fragments are loaded in the same column order); a value
//    lane reads its eight tokens of one column pair with ds_read_b64_tr_b8,
//    one read per M tile. The token scale multiplies the fp32 score and the
//    probability that weights the token's value (rounded to fp16).
//  * More than 64 query rows per sequence (more heads, or several query
//    tokens in multi-token decode, rows token-major): one work group per
//    (range, 64-row head group), the head groups of a range dispatched next to
//    each other on one XCD so that they read its tiles through the same L2.
//    In multi-token decode a head group holds one query token, which sees the
//    positions up to its own: its tile table clamps each tile's row count at
//    that position.
template <bool FP8>
struct PP {
  static constexpr int kRowBytes = FP8 ? kF8RowB : kRowB;    // cache row bytes in LDS
  static constexpr int kCodeB = FP8 ? kF8TileB : kTileB;     // tile bytes without scales
  static constexpr int kInst = FP8 ? kF8DmaInst : kDmaInst;  // wave-wide 16-byte copies per tile
  static constexpr bool kPipe = FP8;                         // softmax one tile behind the scores
  static constexpr int kScaleOff = kCodeB;                   // fp8: token scales of the tile
  static constexpr int kScaleB = FP8 ? 1024 : 0;             // (one wave-wide copy; 128 B used)
  static constexpr int kStageB = kCodeB + kScaleB;
  static constexpr int kStages = FP8 ? 7 : 4;                // ring stages
  static constexpr int kAhead = kStages - (kPipe ? 3 : 2);   // tiles copied ahead of the scores
  static constexpr int kMT = 8;                              // 16-column M tiles per value wave
  // Waves that issue the tile copies: the four value waves (the score waves'
  // instruction stream is the longer one).
  static constexpr int kCopyWaves = 4;
  static constexpr int kPerWave = (kInst + kCopyWaves - 1) / kCopyWaves;  // copy rounds per tile
  // Copy groups cw < kCodeHi issue kPerWave code copies per tile, the others
  // one fewer (bf16). fp8: group kCodeHi copies the token scales instead and
  // the remaining groups a filler, so every wave issues kPerWave copies.
  static constexpr int kCodeHi = kInst % kCopyWaves ? kInst % kCopyWaves : kCopyWaves;
  static constexpr int kHiWaves = FP8 ? kCopyWaves : kCodeHi;  // groups with kPerWave operations
  static constexpr int kSmAt = 8;                            // fp8: softmax after this score read (the last)
  static constexpr int kSteps = FP8 ? kKSteps / 2 : kKSteps;    // score fragment reads per M tile
  static constexpr int kSDist = 3;                           // score reads in flight (per M tile)
  static constexpr int kSRing = kSDist + 2;
  static constexpr int kPD = FP8 ? 8 : 4;                    // value M tiles of reads in flight
  static constexpr int kPReads = FP8 ? 1 : 2;                // LDS reads per value M tile
  static_assert(2 + 1 + 4 + kPReads * kPD <= 15, "LDS reads in flight exceed the lgkmcnt range");
  static_assert(2 + 2 + 2 * kSDist <= 15, "LDS reads in flight exceed the lgkmcnt range");
  // Copies of the next tile go out one by one over the first kSSpread score
  // reads / kVSpread value M tiles.
  static constexpr int kSSpread = kSteps;
  static constexpr int kVSpread = kMT;
  // A head's reference max rises only when a tile's max exceeds it by more
  // than this (log2 units): probabilities (fp8: probability times token scale,
  // against the shifted reference) stay <= 2^kRaise.
  static constexpr float kRaise = 8.f;
  static constexpr int kMaxPieces = 32;                      // segments per window
  static constexpr int kMaxTiles = 640;                      // tiles per window
  static constexpr int kPadOff = kStages * kStageB;          // fp8: landing pad of the fillers
  static constexpr int kRingB = kPadOff + (FP8 ? 1024 : 0);
  static constexpr int kPBufB = 4 * 64 * 16;                 // P^T of one tile, 4 head groups
  static constexpr int kPOff = 0;                            // [2] tiles
  static constexpr int kAlphaOff = kPOff + 2 * kPBufB;       // [2][16 lanes][4 groups] floats
  static constexpr int kFlagOff = kAlphaOff + 2 * 64 * 4;    // [2][4] bytes
  // Finished segments' head sums: bf16 [2][64]; fp8 [2][2 token halves][64]
  // partial sums, then [2][64] reference maxima.
  static constexpr int kFinOff = kFlagOff + 16;
  static constexpr int kFinMOff = kFinOff + (FP8 ? 2 * 2 * 64 * 4 : 0);
  static constexpr int kFinB = FP8 ? 3 * 2 * 64 * 4 : 2 * 64 * 4;
  static constexpr int kPieceOff = kFinOff + kFinB;          // [kMaxPieces] x 2 int4
  static constexpr int kTileOff = kPieceOff + kMaxPieces * 32;  // [kMaxTiles] int2
  static constexpr int kMiscOff = kTileOff + kMaxTiles * 8;     // tiles, window end
  // fp8: each token half's bounds of its heads, [2 tiles][2 head pairs][2 halves][16][2]
  static constexpr int kXbOff = kMiscOff + 16;
  static constexpr int kAuxB = kXbOff + (FP8 ? 2 * 2 * 2 * 16 * 2 * 4 : 0);
  static_assert(kRingB + kAuxB <= 160 * 1024, "LDS budget");
};
// Tile table entry: x = block id (-1: unusable, the tile's rows read zeros),
// y = tile offset in the block / 32 (bits 0-7), valid rows - 1 (bits 8-15),
// piece (bits 16-23), first tile of its sequence in the work group's range
// (bit 30), last such tile (bit 31). The sequence's partial of this range goes
// to slot b + g.
// Piece entry: {s, b, first local block, -}, {first tile, tiles, tokens, -}.

__device__ __forceinline__ void lds_store_b32(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
template <int OFF>
__device__ __forceinline__ void lds_store_b64(uint32_t addr, i32x2 v) {
  asm volatile("ds_write_b64 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF) : "memory");
}
__device__ __forceinline__ void lds_store_b128(uint32_t addr, i32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
template <int OFF>
__device__ __forceinline__ void lds_b32(int& r, uint32_t addr) {
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}
// Transposed 8-bit read: within each 16-lane group, lanes 2k and 2k + 1 give
// the addresses of bytes 0-7 and 8-15 of row k (k = 0..7), and lane m
// receives byte m of each of the eight rows.
template <int OFF>
__device__ __forceinline__ void lds_tr8(i32x2& r, uint32_t addr) {
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
}

// fp8 rows in LDS (576 bytes, 36 chunks of 16 bytes): logical chunk c of row
// r sits at (c & ~3) | ((c & 3) ^ f8_swz(r)), with f8_swz(r) = (r1 ^ r2) |
// (r2 ^ r4) << 1 over the bits rk of r. The two read patterns are 16 rows x
// one chunk (score fragments, ds_read_b128) and 32 rows x one 8-byte half
// chunk per lane pair (transposed value fragments, rows {4q + k, 16 + 4q + k}
// per 16-lane group q). Of the 2-bit XOR swizzles measured on MI355X this one
// gives both their best rate: ~510 B/ns per CU for the score reads (300 with
// ((r >> 2) & 3), 290 unswizzled) and ~330 for the transposed reads.
__device__ __forceinline__ int f8_swz(int r) {
  return (((r >> 1) ^ (r >> 2)) & 1) | ((((r >> 2) ^ (r >> 4)) & 1) << 1);
}

// Eight e4m3 codes (two dwords, byte order) -> eight fp16 values, exact:
// every e4m3 number (4 significant bits, |x| <= 448, down to 2^-9) is an fp16
// normal or subnormal number.
__device__ __forceinline__ i32x4 f8x8_to_f16x8(int d0, int d1) {
  const auto h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<unsigned>(d0), 1.f, false);
  const auto h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<unsigned>(d0), 1.f, true);
  const auto h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<unsigned>(d1), 1.f, false);
  const auto h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<unsigned>(d1), 1.f, true);
  return i32x4{__builtin_bit_cast(int, h0), __builtin_bit_cast(int, h1), __builtin_bit_cast(int, h2),
               __builtin_bit_cast(int, h3)};
}

// Buffer resource over `bytes` bytes from `base` (raw 32-bit access, the gfx9
// family's descriptor word). Loads at offsets at or past `bytes` return zeros
// without touching memory: a tile's rows past its valid tokens, or every row
// of a tile whose block id is unusable (bytes = 0), land in LDS as zeros with
// no per-lane address select.
constexpr int kBufWord3 = 0x00020000;
constexpr int kOobOff = 0x40000000;  // lane offset past every range (fillers)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, kBufWord3);
}

// Stores one head's value slice of a finished sequence piece and restarts its
// accumulators: the slice's kPieceSlice columns lie on the head's 4 lanes q4
// (lanes 16 apart), kMT tiles of 4 columns on each. The values are normalised
// by inv, then multiplied by the power of two that puts the slice's largest
// magnitude in [2^14, 2^15), and rounded to fp16 (nearest even: at most 2^-11
// of that largest magnitude); the inverse power of two, a normal fp32 number
// for any finite slice (the exponent is clamped), goes to the slice's scale,
// which the merge multiplies back. Half the bytes of fp32 rows, for the
// attention kernel's stores and the merge's loads alike.
template <int kMT>
__device__ __forceinline__ void store_piece_f16(const MlaArgs& a, size_t slot, int head, int vbase,
                                                int q4, f32x4* st, int nt, float inv, bool real) {
  float mx = 0.f;
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    const f32x4 v = st[4 * mt + nt];
    mx = vmax3_abs(mx, v[0], v[1]);
    mx = vmax3_abs(mx, v[2], v[3]);
  }
  mx = vmax_xor32(vmax_xor16(mx));
  // mx * inv = f * 2^e with f in [0.5, 1) (e = 0 for an all-zero slice).
  const int e = min(max(__builtin_amdgcn_frexp_expf(mx * inv), -100), 128);
  const float up = __builtin_amdgcn_ldexpf(1.f, 15 - e);  // in [2^-113, 2^115]
  // (The row's first half: kV fp16 values, then the slices' scales.)
  float* row = a.ws_o + (slot * a.Hq + head) * kV;
  uint16_t* orow = reinterpret_cast<uint16_t*>(row) + vbase + 4 * q4;
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    if (real)
      *reinterpret_cast<i32x2*>(orow + 16 * mt) =
          __builtin_bit_cast(i32x2, __builtin_convertvector(st[4 * mt + nt] * inv * up, f16x4));
    st[4 * mt + nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (real && q4 == 0) row[kV / 2 + vbase / kPieceSlice] = __builtin_amdgcn_ldexpf(1.f, e - 15);
}

// SHARED: several head groups (more than 64 query rows per sequence) stream
// the same tiles. Their work groups run side by side on one XCD and the copies
// keep the default cache policy, so the second group finds the tiles in L2.
template <bool FP8, bool SHARED>
__global__ __launch_bounds__(512) void mla_pp_kernel(MlaArgs a) {
  using E = Elt<FP8>;
  using P = PP<FP8>;
  constexpr int kStages = P::kStages;
  constexpr int kAhead = P::kAhead;
  __shared__ __attribute__((aligned(16))) char ring_raw[P::kRingB];
  __shared__ __attribute__((aligned(16))) char aux_raw[P::kAuxB];
  DCP_LDS char* ring = (DCP_LDS char*)ring_raw;
  DCP_LDS char* aux = (DCP_LDS char*)aux_raw;
  const uint32_t ring_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
  const uint32_t aux_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(aux));

  const int lane = threadIdx.x & 63;
  const int w = wave_uniform(threadIdx.x >> 6);
  const bool scorer = w < 4;
  const int grp = w & 3;  // score waves: head group; value waves: value slice
  const int q4 = lane >> 4;
  const int l16 = lane & 15;
  // Head groups of one range are consecutive on one XCD (hardware dispatches
  // work group i to XCD i % 8): group i covers range g and head group y.
  const int ngrp = gridDim.x / kGroups;
  const int k8 = blockIdx.x >> 3;
  const int g = (blockIdx.x & 7) * (kGroups >> 3) + k8 / ngrp;
  const int head0 = (k8 % ngrp) * 64;
  if (!plan_matches(a.sig, a.hdr)) return;  // no plan of this launch's shape
  const int total = a.hdr->total;
  const int range0 = a.wg_start[g];
  const int end = a.wg_start[g + 1];
  if (range0 >= end) return;
  const int bs = a.map.bs;
  const int D = a.map.D;

  // Copies: value wave 4 + cw issues slots cw + 4n of a tile (the score
  // waves issue none: theirs is the longer instruction stream).
  const int cw = w - 4;  // copy group of a value wave
  const bool copier = !scorer;
  // Every wave issues the same copies for every step, also past the end of a
  // window (fillers that read nothing), so each wait for a tile's copies is a
  // constant count.
  const bool hi_wave = cw < P::kHiWaves;
  int32_t cp_off[P::kPerWave];  // byte offset of this lane's copy n in the tile's rows
#pragma unroll
  for (int n = 0; n < P::kPerWave; ++n) {
    const int ii = cw + P::kCopyWaves * n;
    int row = 0, c = 0;
    if (copier && ii < P::kInst) {
      if constexpr (FP8) {
        const int slot = ii * 64 + lane;
        row = slot / kF8RowCh;
        const int pc = slot - row * kF8RowCh;
        c = (pc & ~3) | ((pc & 3) ^ f8_swz(row));
      } else {
        slot_row_chunk<false>(ii * 64 + lane, row, c);
      }
    }
    cp_off[n] = static_cast<int32_t>(row * a.token_stride_b) + 16 * c;
  }
  if constexpr (FP8) {
    // Last round: code rows (cw < kCodeHi), the token scales (cw == kCodeHi:
    // lanes 0-7 take four tokens each; the others read past the range), or a
    // filler into the pad.
    constexpr int n = P::kPerWave - 1;
    if (cw == P::kCodeHi) cp_off[n] = 16 * lane;
    else if (cw > P::kCodeHi) cp_off[n] = kOobOff;
  }
  auto wait_tiles = [&]() {
    if (!copier) return;
    if (hi_wave) wait_tiles_after_n<P::kPerWave, kAhead - 1>(kAhead - 1);
    else wait_tiles_after_n<P::kPerWave - 1, kAhead - 1>(kAhead - 1);
  };

  // Score waves: A fragments of M tile 0 (row l16) and 1 (row 16 + l16).
  // bf16: chunk 4kk + q4 (even kk) or 4 + 4(kk - 1) + q4 (odd kk), one K step
  // per read. fp8: chunk 4j + q4 of read j, i.e. columns 64j + 16q4 .. +15,
  // K steps 2j (first 8 codes) and 2j + 1 (last 8).
  const int r0 = l16, r1 = 16 + l16;
  uint32_t a0e, a0o, a1e, a1o;
  if constexpr (FP8) {
    a0e = a0o = r0 * kF8RowB + 16 * (q4 ^ f8_swz(r0));
    a1e = a1o = r1 * kF8RowB + 16 * (q4 ^ f8_swz(r1));
  } else {
    a0e = r0 * kRowB + 16 * (q4 ^ swz(r0));
    a0o = r0 * kRowB + 16 * ((4 + q4) ^ swz(r0));
    a1e = r1 * kRowB + 16 * (q4 ^ swz(r1));
    a1o = r1 * kRowB + 16 * ((4 + q4) ^ swz(r1));
  }
  // Value waves: transposed A fragments of value columns vbase + 16mt ..
  // +15 over the tokens 4q4 + k and 16 + 4q4 + k (k = 0..3), the order in
  // which the score waves' MFMA results hold them.
  //  bf16: lane (k = l16 / 4, m = l16 % 4) at rows 4q4 + k and 16 + 4q4 + k,
  //        columns vbase + 16mt + 4m .. +3 (two reads per M tile);
  //  fp8:  lane j = l16 at row T(j / 2) (T(k) = 4q4 + k, then 16 + 4q4 + k - 4),
  //        bytes 8(j % 2) .. +7 of chunk vbase / 16 + mt (one read per M tile).
  const int vbase = 128 * grp;
  constexpr int kTOff = FP8 ? 4 : 8;
  uint32_t t_off[kTOff];
  if constexpr (FP8) {
    const int k = l16 >> 1;
    const int row = k < 4 ? 4 * q4 + k : 16 + 4 * q4 + k - 4;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t_off[j] = row * kF8RowB + 16 * (vbase / 16 + (j ^ f8_swz(row))) + 8 * (l16 & 1);
  } else {
    const int t_k = l16 >> 2, t_m = l16 & 3;
    const int t_row0 = 4 * q4 + t_k, t_row1 = 16 + 4 * q4 + t_k;
    const int cgrp = 128 * (vbase / 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 2 * j + (t_m >> 1);
      t_off[j] = cgrp + t_row0 * kRowB + 16 * (c ^ swz(t_row0)) + 8 * (t_m & 1);
      t_off[4 + j] = cgrp + t_row1 * kRowB + 16 * (c ^ swz(t_row1)) + 8 * (t_m & 1);
    }
  }
  const uint32_t flags_addr = aux_addr + P::kFlagOff;
  const uint32_t tiles_addr = aux_addr + P::kTileOff;
  const uint32_t piece_addr = aux_addr + P::kPieceOff;

  // Tile table entry t of the current window (wave-uniform).
  struct TileInfo {
    int id, y;
    __device__ int nvalid() const { return ((y >> 8) & 0xff) + 1; }
    __device__ int piece() const { return (y >> 16) & 0xff; }
    __device__ bool first() const { return (y >> 30) & 1; }
    __device__ bool last() const { return (y >> 31) & 1; }
    __device__ unsigned rows() const {  // bit r: row r holds a real token of a usable block
      return id >= 0 ? (nvalid() == 32 ? 0xffffffffu : (1u << nvalid()) - 1) : 0u;
    }
  };
  // Tile table entries are read ahead: the read goes out during one step and
  // is consumed after the next step's barrier (whose wait covers it).
  auto entry_read = [&](i32x2& e, int t) { lds_b64<0>(e, tiles_addr + 8 * t); };
  auto entry_take = [&](i32x2& e) -> TileInfo {
    wait_lgkm<0>(e);
    return TileInfo{wave_uniform(e[0]), wave_uniform(e[1])};
  };
  auto tile_info = [&](int t) -> TileInfo {
    i32x2 e;
    lds_b64<0>(e, tiles_addr + 8 * t);
    wait_lgkm<0>(e);
    return TileInfo{wave_uniform(e[0]), wave_uniform(e[1])};
  };
  auto piece_b = [&](int p) -> int {  // sequence of piece p
    int v;
    lds_b32<4>(v, piece_addr + 32 * p);
    wait_lgkm<0>(v);
    return wave_uniform(v);
  };
  // Copy source of a tile: a buffer resource over its valid rows, so rows
  // without a real token of a usable block read as zeros (no tile is ever
  // zeroed in LDS), and for fp8 one over the token scales of whole 4-token
  // chunks (scales of rows past the valid ones are masked by the scores).
  // A filler (past the window's end) reads nothing.
  struct Src {
    __amdgpu_buffer_rsrc_t rows;
    __amdgpu_buffer_rsrc_t last;  // fp8: the last copy round's resource (rows, or the scales)
  };
  const unsigned bstride = static_cast<unsigned>(a.block_stride_b);
  const int tstride = static_cast<int>(a.token_stride_b);
  auto tile_src = [&](const TileInfo& ti, bool real) -> Src {
    const bool ok = real && ti.id >= 0;
    const int nv = ok ? ti.nvalid() : 0;
    const int tok0 = 32 * (ti.y & 0xff);
    const unsigned id = ok ? static_cast<unsigned>(ti.id) : 0u;
    const __amdgpu_buffer_rsrc_t rows = rows_rsrc(
        a.kv + (static_cast<unsigned long long>(id) * bstride + static_cast<unsigned>(tok0 * tstride)),
        nv * tstride);
    if constexpr (FP8) {
      if (cw == P::kCodeHi)
        return Src{rows, rows_rsrc(a.kv_scale + 4 * (static_cast<unsigned long long>(id) * a.scale_bs + tok0),
                                   16 * ((nv + 3) >> 2))};
    }
    return Src{rows, rows};
  };
  auto copy_one = [&](auto nc, const Src& sr, int t) {
    constexpr int n = decltype(nc)::value;
    const int ii = cw + P::kCopyWaves * n;
    DCP_LDS char* stage = ring + (t % kStages) * P::kStageB;
    // (Operands bound to locals: with expressions inline in the builtin's
    // argument list the host pass drops this kernel's stub.)
    const int off = cp_off[n];
    if constexpr (FP8) {
      if constexpr (n == P::kPerWave - 1) {
        const __amdgpu_buffer_rsrc_t rs = sr.last;
        DCP_LDS char* ldst = cw < P::kCodeHi ? stage + ii * 1024
                             : cw == P::kCodeHi ? stage + P::kScaleOff : ring + P::kPadOff;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, ldst, 16, off, 0, 0, SHARED ? 0 : kCopyPolicy);
        return;
      }
    } else {
      if (n == P::kPerWave - 1 && ii >= P::kInst) return;
    }
    const __amdgpu_buffer_rsrc_t rs = sr.rows;
    DCP_LDS char* ldst = stage + ii * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, ldst, 16, off, 0, 0, SHARED ? 0 : kCopyPolicy);
  };

  // The two roles run the same loops and barriers with separate code, so the
  // register allocator sees the query fragments of one and the accumulators
  // of the other as never live at the same time.
  auto run = [&](auto role) {
    constexpr bool kScorer = decltype(role)::value;
    // Score waves: the query fragments (B operand of S^T, K step kk) -- bf16:
    // 18 of head head0 + 16grp + l16; fp8 (fp16 fragments): 18 of each of
    // heads head0 + 32hp + 16nt + l16, nt = 0, 1, at 18nt + kk. Value waves:
    // O^T accumulators, M tile mt and head tile nt at 4mt + nt.
    constexpr int kQTiles = FP8 ? 2 : 1;
    constexpr int kSt = kScorer ? kQTiles * kKSteps : 4 * P::kMT;
    f32x4 st[kSt];
#pragma unroll
    for (int i = 0; i < kSt; ++i) st[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    int qb = -1;
    float qsl[kQTiles];  // score scale (log2 units) of each loaded head
#pragma unroll
    for (int nt = 0; nt < kQTiles; ++nt) qsl[nt] = a.scale_log2;
    const int hp = grp >> 1, th = grp & 1;  // fp8 score waves: head pair, token half
    auto load_q = [&](int b) {
      if constexpr (kScorer) {
      // K step kk covers query columns 32kk + 8q4 .. +7 (bf16), or
      // 64(kk / 2) + 16q4 + 8(kk % 2) .. +7 (fp8, the chunk order above).
#pragma unroll
      for (int nt = 0; nt < kQTiles; ++nt) {
        const int head = FP8 ? head0 + 32 * hp + 16 * nt + l16 : head0 + 16 * grp + l16;
        // (With 16 or 32 query rows the rows past them are zero queries whose
        // results are never stored.)
        const bool real = head < a.Hq;
        const uint16_t* qrow =
            a.q + (static_cast<size_t>(b) * a.Hq + (real ? head : 0)) * kQK + (FP8 ? 16 : 8) * q4;
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
          const int col = FP8 ? 64 * (kk >> 1) + 8 * (kk & 1) : 32 * kk;
          bf16x8 v = {};
          if (real) v = *reinterpret_cast<const bf16x8*>(qrow + col);
          st[nt * kKSteps + kk] = __builtin_bit_cast(f32x4, v);
        }
      }
      // Consume the loads here, in order: the compiler then waits for exactly
      // these loads (and what was issued before them), instead of placing a
      // wait for every outstanding copy in front of each later use.
#pragma unroll
      for (int i = 0; i < kSt; ++i) asm volatile("" : "+v"(st[i]));
      if constexpr (FP8) {
#pragma unroll
        for (int nt = 0; nt < kQTiles; ++nt) {
          // The head's largest magnitude over the four lanes that hold it.
          float qm = 0.f;
#pragma unroll
          for (int kk = 0; kk < kKSteps; ++kk) {
            const bf16x8 v = __builtin_bit_cast(bf16x8, st[nt * kKSteps + kk]);
#pragma unroll
            for (int i = 0; i < 8; ++i) qm = fmaxf(qm, fabsf(static_cast<float>(v[i])));
          }
          const int qe = max_exponent_head(max_xor32(max_xor16(qm)));
#pragma unroll
          for (int kk = 0; kk < kKSteps; ++kk)
            st[nt * kKSteps + kk] = __builtin_bit_cast(
                f32x4, E::from_bf16_pow2(__builtin_bit_cast(bf16x8, st[nt * kKSteps + kk]), qe));
          qsl[nt] = __builtin_amdgcn_ldexpf(a.scale_log2, qe);
        }
      } else {
        // The scale's sign goes into the query (an exact sign flip), so the
        // scores are multiplied by c = |scale| log2(e). A zero scale is taken
        // as 2^-100 (every probability then rounds to exactly 1, as for 0),
        // so that c is positive and -inf scores of masked rows stay -inf.
        if (a.scale_log2 < 0.f) {
#pragma unroll
          for (int kk = 0; kk < kKSteps; ++kk)
            st[kk] = __builtin_bit_cast(f32x4, __builtin_bit_cast(i32x4, st[kk]) ^ static_cast<int>(0x80008000u));
        }
        qsl[0] = fmaxf(fabsf(a.scale_log2), 0x1p-100f);
      }
      qb = b;
      }
    };
    float m_ref = -INFINITY;  // score waves: reference max (log2 units) of head 16grp + l16
    float l_run = 0.f;        // score waves: this lane's probability sum for that head
    float m2[2] = {-INFINITY, -INFINITY};  // fp8: the same for heads 32hp + 16nt + l16
    float l2[2] = {0.f, 0.f};
    float l_rnd = 0.f;        // bf16: the same sum over the probabilities as rounded for P^T
    int nfin = 0;             // segments finished so far (parity selects the fin buffer)

    int wpos = range0;
    int s_cur = a.wg_seg[g];
    while (wpos < end) {
      // ---- window [wpos, wend): piece table (wave 0), then tile table (all)
      if (w == 0) {
        const int sl = s_cur + lane;
        int lo = total, hi = total, qlo = total, qhi = total;
        if (sl < a.S) {
          lo = a.seg_off[sl];
          hi = a.seg_off[sl + 1];
          const int s0 = sl - sl % D;  // the sequence's blocks: [seg_off[s0], seg_off[s0 + D])
          qlo = a.seg_off[s0];
          qhi = a.seg_off[s0 + D];
        }
        int wend = end;
        if (s_cur + P::kMaxPieces <= a.S)
          wend = min(wend, __shfl(hi, P::kMaxPieces - 1));  // start of segment s_cur + 32
        wend = min(wend, wpos + P::kMaxTiles / (bs / kT));
        const int pstart = max(lo, wpos);
        const int pend = min(hi, wend);
        const int nblk = (lane < P::kMaxPieces && sl < a.S) ? max(0, pend - pstart) : 0;
        int ntok = 0, b = 0, i0 = 0;
        if (nblk > 0) {
          b = sl / D;
          const int r = sl - b * D;
          i0 = pstart - lo;
          const int i1 = pend - lo;
          const int tail = bs * (r + D * (i1 - 1) + 1) - seq_tokens(a.map, b);
          ntok = nblk * bs - max(tail, 0);
        }
        const int ntiles = (ntok + kT - 1) / kT;
        int ts = ntiles;  // inclusive prefix sum -> first tile
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int v = __shfl_up(ts, off);
          if (lane >= off) ts += v;
        }
        const int T = __shfl(ts, 63);
        ts -= ntiles;
        // first / last piece of its sequence in this range: the accumulation
        // runs on across the sequence's shards and ends in one partial
        const int flags = (pstart == max(qlo, range0) ? 1 : 0) | (pend == min(qhi, end) ? 2 : 0);
        if (lane < P::kMaxPieces) {
          *reinterpret_cast<DCP_LDS i32x4*>(aux + P::kPieceOff + 32 * lane) = i32x4{sl, b, i0, 0};
          *reinterpret_cast<DCP_LDS i32x4*>(aux + P::kPieceOff + 32 * lane + 16) =
              i32x4{ts, ntiles, ntok, flags};
        }
        if (lane == 0) *reinterpret_cast<DCP_LDS i32x4*>(aux + P::kMiscOff) = i32x4{T, wend, 0, 0};
      }
      __syncthreads();
      const i32x4 misc = *reinterpret_cast<const DCP_LDS i32x4*>(aux + P::kMiscOff);
      const int T = misc[0];
      const int wend = misc[1];
      for (int t = threadIdx.x; t < T; t += 512) {
        // piece p: last piece whose first tile is <= t (a piece without tiles
        // shares its first tile with the next one, which is found instead)
        int p = 0;
        for (int step = P::kMaxPieces / 2; step > 0; step >>= 1) {
          const int ts = *reinterpret_cast<const DCP_LDS int*>(aux + P::kPieceOff + 32 * (p + step) + 16);
          if (ts <= t) p += step;
        }
        const i32x4 pa = *reinterpret_cast<const DCP_LDS i32x4*>(aux + P::kPieceOff + 32 * p);
        const i32x4 pb = *reinterpret_cast<const DCP_LDS i32x4*>(aux + P::kPieceOff + 32 * p + 16);
        const int j = t - pb[0];
        const int tok = j * kT;
        const int b = pa[1];
        const int col = (pa[0] - b * D) + D * (pa[2] + tok / bs);
        int id = a.map.table[static_cast<size_t>(b) * a.map.width + col];
        if (!(id >= 0 && id < a.ncb)) id = -1;
        int nvalid = min(kT, pb[2] - tok);
        if (a.causal) {
          // This work group's 64 rows belong to one query token t_q, which sees
          // the positions up to q_pos + t_q; the tile's rows are consecutive
          // positions of one block, so the visible rows are a prefix.
          const int t_q = head0 / a.cz.hq;
          const long long vis = first_query_pos(a.cz, a.map, b) + t_q -
                                global_pos(a.cz, col, bs, tok % bs) + 1;
          if (vis < nvalid) {
            if (vis <= 0) {
              id = -1;
              nvalid = 1;
            } else {
              nvalid = static_cast<int>(vis);
            }
          }
        }
        const unsigned y = static_cast<unsigned>((tok % bs) / kT) | (static_cast<unsigned>(nvalid - 1) << 8) |
                           (static_cast<unsigned>(p) << 16) |
                           ((j == 0 && (pb[3] & 1)) ? (1u << 30) : 0u) |
                           ((j == pb[1] - 1 && (pb[3] & 2)) ? (1u << 31) : 0u);
        *reinterpret_cast<DCP_LDS i32x2*>(aux + P::kTileOff + 8 * t) = i32x2{id, static_cast<int>(y)};
      }
      wait_vm<0>();
      __syncthreads();
      // prologue: the first kAhead tiles (fillers past the last tile, so that
      // every step is preceded by the same number of copies)
      for (int t = 0; t < kAhead; ++t) {
        const Src sr = tile_src(tile_info(min(t, max(T - 1, 0))), t < T);
        if (copier) static_for<0, P::kPerWave>([&](auto nc) { copy_one(nc, sr, t); });
      }

      // Start of step ks (score waves on tile ks, value waves on tile ks - 1):
      // this wave's copies of tile ks have landed (every step issues one tile,
      // a filler past the window's end, so kAhead - 1 tiles are in flight
      // after it), then the barrier makes every wave's copies visible and
      // guarantees that step ks - 1 is finished, so the stage of tile ks - 2 is
      // free for tile ks + kAhead. Both roles pass the same barriers in the
      // same order.
      auto step_begin = [&](int) {
        wait_tiles();
        lds_barrier();
      };

      if constexpr (P::kPipe) {
       if constexpr (kScorer) {
        // fp8 score waves: wave grp = 2hp + th takes the 32 heads of head pair
        // hp over the 16 tokens of token half th (rows 16th + l16 of the A
        // operand; lane results are tokens 16th + 4q4 + i of heads 32hp + 16nt
        // + l16), so each converted code feeds two MFMAs. A head's two token
        // halves lie in the waves 2hp and 2hp + 1: at the end of step ks each
        // writes its bounds of tile ks to LDS, and in step ks + 1 each reads
        // the other's and runs the softmax of tile ks with the common maximum
        // (both compute the same reference from the same two values).
        i32x2 e_cur = {0, 0};
        if (T > 0) entry_read(e_cur, 0);
        // Tile ks - 1, whose softmax runs in step ks: its table entry, its
        // x = s sigma c (x[4nt + i]: head nt, token 16th + 4q4 + i), its token
        // scales and this half's bound of each head.
        TileInfo tip{-1, 0};
        float xp[8], sgp[4], bop[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) xp[i] = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) sgp[i] = 0.f;
        bop[0] = bop[1] = -INFINITY;
        const uint32_t a_row = th ? a1e : a0e;
        const uint32_t xb_addr = aux_addr + P::kXbOff + (hp * 2 + th) * 128 + l16 * 8;
        const uint32_t xb_other = aux_addr + P::kXbOff + (hp * 2 + (th ^ 1)) * 128 + l16 * 8;
        for (int ks = 0; ks <= T; ++ks) {
          step_begin(ks);
          const bool has_s = ks < T;   // step ks scores tile ks ...
          const bool has_sm = ks > 0;  // ... and runs the softmax of tile ks - 1
          TileInfo ti{-1, 0};
          if (has_s) {
            ti = entry_take(e_cur);
            entry_read(e_cur, min(ks + 1, T - 1));
            if (ti.first()) {
              // A new sequence needs its query. (Loaded here, in the iteration
              // that uses it, the compiler's waits for it are exact.)
              const int b = piece_b(ti.piece());
              if (b != qb) load_q(b);
            }
          }
          if (has_sm && tip.first()) {
            m2[0] = m2[1] = -INFINITY;
            l2[0] = l2[1] = 0.f;
          }
          // (In the window's last step there is no tile ks: the score loop then
          // reads a stale stage and its results are dropped.)
          const uint32_t tile = ring_addr + (ks % kStages) * P::kStageB;
          i32x4 scr;  // scales of this lane's tokens of tile ks
          lds_b128<0>(scr, tile + P::kScaleOff + 64 * th + 16 * q4);
          i32x2 xo;   // the other half's bounds of tile ks - 1
          lds_b64<0>(xo, xb_other + ((ks - 1) & 1) * 512);
          i32x4 ra[P::kSRing];
          auto s_issue = [&](auto kc) {
            constexpr int kk = decltype(kc)::value;
            lds_b128<64 * kk>(ra[kk % P::kSRing], tile + a_row);
          };
          static_for<0, P::kSDist>(s_issue);

          // Online softmax of tile ks - 1 for heads 32hp + 16nt + l16 over this
          // lane's 4 tokens, exp2 domain, against the larger of the two halves'
          // bounds (log2 bounds of p * sigma against reference 0).
          i32x2 pk[2] = {{0, 0}, {0, 0}};
          float alpha[2] = {1.f, 1.f}, m_new[2] = {m2[0], m2[1]}, l_new[2] = {l2[0], l2[1]};
          bool raise = false;
          auto softmax_prev = [&]() {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
              const float bnd = vmax(bop[nt], __int_as_float(xo[nt]));
              const bool up = bnd > m2[nt] + P::kRaise;
              raise |= up;
              alpha[nt] = up ? fast_exp2(m2[nt] - bnd) : 1.f;  // 0 when m = -inf
              m_new[nt] = up ? bnd : m2[nt];
              const float nm = m_new[nt] == -INFINITY ? 0.f : -m_new[nt];
              float pr[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(xp[4 * nt + i] + nm);
              l_new[nt] = l2[nt] * alpha[nt] + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
              // the value waves weight each token's codes by p * scale
              pk[nt] = i32x2{static_cast<int>(E::pack2(pr[0] * sgp[0], pr[1] * sgp[1])),
                             static_cast<int>(E::pack2(pr[2] * sgp[2], pr[3] * sgp[3]))};
            }
          };

          f32x4 s0a = {0.f, 0.f, 0.f, 0.f}, s0b = s0a, s1a = s0a, s1b = s0a;
          static_for<0, P::kSteps>([&](auto kc) {
            constexpr int kk = decltype(kc)::value;
            if constexpr (kk + P::kSDist < P::kSteps) s_issue(IC<kk + P::kSDist>{});
            constexpr int ahead = kk + P::kSDist < P::kSteps ? P::kSDist : P::kSteps - 1 - kk;
            // (LDS reads complete in order: once read kk is in, so are the
            // scales and the other half's bounds issued before it.)
            if constexpr (kk == 0) wait_lgkm<ahead>(ra[0], xo);
            else wait_lgkm<ahead>(ra[kk % P::kSRing]);
            // read kk: K steps 2kk (codes 0-7) and 2kk + 1 (codes 8-15) of row
            // 16th + l16, for both heads of the lane
            const i32x4 ua = ra[kk % P::kSRing];
            const i32x4 a0 = f8x8_to_f16x8(ua[0], ua[1]), a1 = f8x8_to_f16x8(ua[2], ua[3]);
            s0a = E::mfma(a0, __builtin_bit_cast(f16x8, st[2 * kk]), s0a);
            s1a = E::mfma(a0, __builtin_bit_cast(f16x8, st[kKSteps + 2 * kk]), s1a);
            s0b = E::mfma(a1, __builtin_bit_cast(f16x8, st[2 * kk + 1]), s0b);
            s1b = E::mfma(a1, __builtin_bit_cast(f16x8, st[kKSteps + 2 * kk + 1]), s1b);
            if constexpr (kk == P::kSmAt) softmax_prev();
          });
          const f32x4 sv[2] = {s0a + s0b, s1a + s1b};

          // Results of tile ks - 1. (A window's first step has none.)
          const int pp = (ks - 1) & 1;
          if (has_sm) {
            const uint32_t pdst = aux_addr + P::kPOff + pp * P::kPBufB + lane * 16 + 8 * th;
            lds_store_b64<0>(pdst + (2 * hp) * 1024, pk[0]);
            lds_store_b64<0>(pdst + (2 * hp + 1) * 1024, pk[1]);
          }
          const bool any = has_sm && __ballot(raise) != 0ull;
          if (lane == 0) lds_store_b8(flags_addr + pp * 4 + grp, any ? 1 : 0);
          if (any && th == 0 && q4 == 0)
            lds_store_b64<0>(aux_addr + P::kAlphaOff + ((pp * 16 + l16) * 4 + 2 * hp) * 4,
                             i32x2{__float_as_int(alpha[0]), __float_as_int(alpha[1])});
          if (has_sm) {
            m2[0] = m_new[0];
            m2[1] = m_new[1];
            l2[0] = l_new[0];
            l2[1] = l_new[1];
          }
          if (has_sm && tip.last()) {
            // Segment done: this half's head sums and (half 0) the reference
            // maxima, for the value waves' normalisation and LSE.
            const float lh0 = sum_xor32(sum_xor16(l2[0])), lh1 = sum_xor32(sum_xor16(l2[1]));
            if (q4 == 0) {
              const uint32_t fl = aux_addr + P::kFinOff + (((nfin & 1) * 2 + th) * 64 + 32 * hp + l16) * 4;
              lds_store_b32(fl, lh0);
              lds_store_b32(fl + 64, lh1);
              if (th == 0) {
                const uint32_t fm = aux_addr + P::kFinMOff + ((nfin & 1) * 64 + 32 * hp + l16) * 4;
                lds_store_b32(fm, m2[0]);
                lds_store_b32(fm + 64, m2[1]);
              }
            }
            ++nfin;
          }

          // Tile ks: x, and this half's bound of each head (the lanes' largest
          // x plus the exponent of their largest scale, over the four lanes
          // holding the head), written for the other half.
          wait_lgkm<0>(scr);
          float sg[4], xn[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) sg[i] = __int_as_float(scr[i]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) xn[4 * nt + i] = sv[nt][i] * sg[i] * qsl[nt];
          const unsigned vm = ti.rows();
          if (vm != 0xffffffffu) {  // rows past the end (wave-uniform)
            const unsigned rb = vm >> (16 * th + 4 * q4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool v = (rb >> i) & 1u;
              sg[i] = v ? sg[i] : 0.f;
              xn[i] = v ? xn[i] : -INFINITY;
              xn[4 + i] = v ? xn[4 + i] : -INFINITY;
            }
          }
          const float e = scale_exponent(vmax(vmax(sg[0], sg[1]), vmax(sg[2], sg[3])));
          float bn[2];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            bn[nt] = vmax_xor32(vmax_xor16(vmax(vmax(xn[4 * nt], xn[4 * nt + 1]),
                                                vmax(xn[4 * nt + 2], xn[4 * nt + 3])) + e));
          if (has_s && q4 == 0)
            lds_store_b64<0>(xb_addr + (ks & 1) * 512, i32x2{__float_as_int(bn[0]), __float_as_int(bn[1])});
          tip = ti;
#pragma unroll
          for (int i = 0; i < 8; ++i) xp[i] = xn[i];
#pragma unroll
          for (int i = 0; i < 4; ++i) sgp[i] = sg[i];
          bop[0] = bn[0];
          bop[1] = bn[1];
        }
        step_begin(T + 1);  // the value waves' last step
       } else {
        // Steps 0 and 1 have no value tile yet: only this wave's copies. (Kept
        // out of the loop: a loop path that leaves the accumulators untouched
        // makes the register allocator rotate them through fresh registers.)
        for (int ks = 0; ks < 2; ++ks) {
          step_begin(ks);
          const Src nsrc = tile_src(tile_info(min(ks + kAhead, max(T - 1, 0))), ks + kAhead < T);
          static_for<0, P::kPerWave>([&](auto nc) { copy_one(nc, nsrc, ks + kAhead); });
        }
        i32x2 e_kv = {0, 0}, e_iss = {0, 0};
        if (T > 0) {
          entry_read(e_kv, 0);
          entry_read(e_iss, min(2 + kAhead, T - 1));
        }
        for (int ks = 2; ks <= T + 1; ++ks) {
          step_begin(ks);
          const TileInfo tiss = entry_take(e_iss);
          entry_read(e_iss, min(ks + 1 + kAhead, T - 1));
          const Src nsrc = tile_src(tiss, ks + kAhead < T);
          const TileInfo ti = entry_take(e_kv);
          entry_read(e_kv, min(ks - 1, T - 1));
          const int kv = ks - 2;
          // LDS reads of this step, oldest first: the rescale votes of tile kv,
          // its P^T fragments, then its transposed tile fragments; the votes
          // are inspected once they arrive, while the rest is in flight.
          int fl;
          lds_b32<0>(fl, flags_addr + (kv & 1) * 4);
          i32x4 pb[4];
          const uint32_t pbase = aux_addr + P::kPOff + (kv & 1) * P::kPBufB + lane * 16;
          static_for<0, 4>([&](auto nc) {
            constexpr int nt = decltype(nc)::value;
            lds_b128<nt * 1024>(pb[nt], pbase);
          });
          const uint32_t tile = ring_addr + (kv % kStages) * P::kStageB;
          uint32_t tb[kTOff];
#pragma unroll
          for (int j = 0; j < kTOff; ++j) tb[j] = tile + t_off[j];
          i32x2 rv[P::kMT];
          static_for<0, P::kMT>([&](auto mc) {
            constexpr int mt = decltype(mc)::value;
            lds_tr8<64 * (mt >> 2)>(rv[mt], tb[mt & 3]);
          });
          wait_lgkm<4 + P::kMT>(fl);
          const int fb = wave_uniform(fl);
          if (fb != 0) {
            // Rescale factors of heads whose reference max rose in tile kv
            // (vote byte 2hp, the pair's first half, covers head tiles 2hp and
            // 2hp + 1; a head that did not rise has factor 1).
            i32x4 al;
            lds_b128<0>(al, aux_addr + P::kAlphaOff + ((kv & 1) * 16 + l16) * 16);
            wait_lgkm<0>(al);
            const f32x4 alv = __builtin_bit_cast(f32x4, al);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
              if ((fb >> (8 * (nt & ~1))) & 0xff)
#pragma unroll
                for (int mt = 0; mt < P::kMT; ++mt) st[4 * mt + nt] *= alv[nt];
          }
          static_for<0, P::kMT>([&](auto mc) {
            constexpr int mt = decltype(mc)::value;
            wait_lgkm<P::kMT - 1 - mt>(rv[mt]);
            const i32x4 av = f8x8_to_f16x8(rv[mt][0], rv[mt][1]);
            static_for<0, 4>([&](auto nc) {
              constexpr int nt = decltype(nc)::value;
              st[4 * mt + nt] = E::mfma(av, __builtin_bit_cast(typename E::vec, pb[nt]), st[4 * mt + nt]);
            });
            constexpr int n0 = mt * P::kPerWave / P::kVSpread;
            constexpr int n1 = (mt + 1) * P::kPerWave / P::kVSpread;
            static_for<n0, n1>([&](auto nc) { copy_one(nc, nsrc, ks + kAhead); });
          });
          if (ti.last()) {
            // Segment done: normalise by the head sums (the two token halves'
            // partial sums) and store (O, slot b + g); value wave 0 also stores
            // the LSE from the reference maxima. The accumulators restart at 0.
            const size_t slot = static_cast<size_t>(piece_b(ti.piece())) + g;
            // head 16nt + l16: halves at fin[(par * 2 + half) * 64 + head], maximum at finm[par * 64 + head]
            const uint32_t fa = aux_addr + P::kFinOff + ((nfin & 1) * 128 + l16) * 4;
            const uint32_t fm = aux_addr + P::kFinMOff + ((nfin & 1) * 64 + l16) * 4;
            int h0[4], h1[4], mm[4];
            static_for<0, 4>([&](auto nc) {
              constexpr int nt = decltype(nc)::value;
              lds_b32<64 * nt>(h0[nt], fa);
              lds_b32<256 + 64 * nt>(h1[nt], fa);
              lds_b32<64 * nt>(mm[nt], fm);
            });
            wait_lgkm<0>(h0[0], h1[0]);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) asm volatile("" : "+v"(h0[nt]), "+v"(h1[nt]), "+v"(mm[nt]));
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              const float lt = __int_as_float(h0[nt]) + __int_as_float(h1[nt]);
              const float inv = lt > 0.f ? 1.f / lt : 0.f;
              const bool real = head0 + 16 * nt < a.Hq;  // (rows past 16 or 32 query rows)
              store_piece_f16<P::kMT>(a, slot, head0 + 16 * nt + l16, vbase, q4, st, nt, inv, real);
              if (real && grp == 0 && q4 == 0)
                a.ws_lse[slot * a.Hq + head0 + 16 * nt + l16] =
                    lt > 0.f ? (__int_as_float(mm[nt]) + fast_log2(lt)) * kLn2 : -INFINITY;
            }
            ++nfin;
          }
        }
       }
      } else if constexpr (kScorer) {
        // bf16 score waves (fp8 caches take the pipelined branch above). They
        // issue no copies: the value waves copy the tiles.
        static_assert(!FP8, "fp8 score waves are pipelined");
        i32x2 e_cur = {0, 0};
        if (T > 0) entry_read(e_cur, 0);
        for (int ks = 0; ks < T; ++ks) {
          step_begin(ks);
          const TileInfo ti = entry_take(e_cur);
          entry_read(e_cur, min(ks + 1, T - 1));
          if (ti.first()) {
            m_ref = -INFINITY;
            l_run = 0.f;
            l_rnd = 0.f;
            // A new sequence needs its query. (Loaded here, in the iteration
            // that uses it, the compiler's waits for it are exact.)
            const int b = piece_b(ti.piece());
            if (b != qb) load_q(b);
          }
          const uint32_t tile = ring_addr + (ks % kStages) * P::kStageB;
          i32x4 ra[P::kSRing], rb[P::kSRing];
          auto s_issue = [&](auto kc) {
            constexpr int kk = decltype(kc)::value;
            constexpr int off = 128 * (kk >> 1);
            if constexpr (kk & 1) {
              lds_b128<off>(ra[kk % P::kSRing], tile + a0o);
              lds_b128<off>(rb[kk % P::kSRing], tile + a1o);
            } else {
              lds_b128<off>(ra[kk % P::kSRing], tile + a0e);
              lds_b128<off>(rb[kk % P::kSRing], tile + a1e);
            }
          };
          static_for<0, P::kSDist>(s_issue);
          f32x4 s0a = {0.f, 0.f, 0.f, 0.f}, s0b = s0a, s1a = s0a, s1b = s0a;
          static_for<0, P::kSteps>([&](auto kc) {
            constexpr int kk = decltype(kc)::value;
            if constexpr (kk + P::kSDist < P::kSteps) s_issue(IC<kk + P::kSDist>{});
            constexpr int ahead = kk + P::kSDist < P::kSteps ? P::kSDist : P::kSteps - 1 - kk;
            wait_lgkm<2 * ahead>(ra[kk % P::kSRing], rb[kk % P::kSRing]);
            const bf16x8 qv = __builtin_bit_cast(bf16x8, st[kk]);
            if constexpr (kk & 1) {
              s0b = E::mfma(ra[kk % P::kSRing], qv, s0b);
              s1b = E::mfma(rb[kk % P::kSRing], qv, s1b);
            } else {
              s0a = E::mfma(ra[kk % P::kSRing], qv, s0a);
              s1a = E::mfma(rb[kk % P::kSRing], qv, s1a);
            }
          });
          const f32x4 sv0 = s0a + s0b, sv1 = s1a + s1b;

          // Online softmax of head 16grp + l16 over this lane's 8 tokens
          // (4q4 + i and 16 + 4q4 + i), exp2 domain: x_i = c s_i with
          // c = |scale| log2(e) > 0 (the query carries the scale's sign), so
          // the largest score gives the largest x, each probability is
          // exp2(fma(s_i, c, -m)), and a masked row's -inf score gives p = 0.
          float sc[8] = {sv0[0], sv0[1], sv0[2], sv0[3], sv1[0], sv1[1], sv1[2], sv1[3]};
          const unsigned vm = ti.rows();
          if (vm != 0xffffffffu) {  // rows past the end (wave-uniform)
            const unsigned lo = vm >> (4 * q4), hi = vm >> (16 + 4 * q4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              sc[i] = (lo >> i) & 1u ? sc[i] : -INFINITY;
              sc[4 + i] = (hi >> i) & 1u ? sc[4 + i] : -INFINITY;
            }
          }
          const float hmax = vmax_xor32(vmax_xor16(vmax8(sc))) * qsl[0];
          // The reference only rises when the tile's max exceeds it by more
          // than kRaise, so probabilities stay <= 2^kRaise and rescales are rare.
          const bool raise = hmax > m_ref + P::kRaise;
          const float alpha = raise ? fast_exp2(m_ref - hmax) : 1.f;  // 0 when m_ref = -inf
          m_ref = raise ? hmax : m_ref;
          const float nm = m_ref == -INFINITY ? 0.f : -m_ref;
          float pr[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) pr[i] = fast_exp2(fmaf(sc[i], qsl[0], nm));
          l_run = l_run * alpha +
                  (((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7])));
          const i32x4 pk = {static_cast<int>(E::pack2(pr[0], pr[1])),
                            static_cast<int>(E::pack2(pr[2], pr[3])),
                            static_cast<int>(E::pack2(pr[4], pr[5])),
                            static_cast<int>(E::pack2(pr[6], pr[7]))};
          l_rnd = add_bf16x8(pk, l_rnd * alpha);
          lds_store_b128(aux_addr + P::kPOff + (ks & 1) * P::kPBufB + (grp * 64 + lane) * 16, pk);
          const bool any = __ballot(raise) != 0ull;
          if (lane == 0) lds_store_b8(flags_addr + (ks & 1) * 4 + grp, any ? 1 : 0);
          if (any && q4 == 0)
            lds_store_b32(aux_addr + P::kAlphaOff + (((ks & 1) * 16 + l16) * 4 + grp) * 4, alpha);
          if (ti.last()) {
            // Segment done: its head sums for the value waves (of the rounded
            // probabilities), and its LSE.
            const float l_h = sum_xor32(sum_xor16(l_run));
            const float l_o = sum_xor32(sum_xor16(l_rnd));
            if (q4 == 0) {
              lds_store_b32(aux_addr + P::kFinOff + ((nfin & 1) * 64 + 16 * grp + l16) * 4, l_o);
              const size_t slot = static_cast<size_t>(piece_b(ti.piece())) + g;
              if (head0 + 16 * grp < a.Hq)  // (rows past 16 or 32 query rows)
                a.ws_lse[slot * a.Hq + head0 + 16 * grp + l16] =
                    l_h > 0.f ? (m_ref + fast_log2(l_h)) * kLn2 : -INFINITY;
            }
            ++nfin;
          }
        }
        step_begin(T);  // the value waves' last step
      } else {
        // Step 0 has no value tile yet: only this wave's copies of tile kAhead.
        step_begin(0);
        {
          const Src nsrc = tile_src(tile_info(min(kAhead, max(T - 1, 0))), kAhead < T);
          static_for<0, P::kPerWave>([&](auto nc) { copy_one(nc, nsrc, kAhead); });
        }
        i32x2 e_kv = {0, 0}, e_iss = {0, 0};
        if (T > 0) {
          entry_read(e_kv, 0);
          entry_read(e_iss, min(1 + kAhead, T - 1));
        }
        for (int ks = 1; ks <= T; ++ks) {
          step_begin(ks);
          const TileInfo ti = entry_take(e_kv);
          const TileInfo tiss = entry_take(e_iss);
          entry_read(e_kv, min(ks, T - 1));
          entry_read(e_iss, min(ks + 1 + kAhead, T - 1));
          const Src nsrc = tile_src(tiss, ks + kAhead < T);
          const int kv = ks - 1;
          // LDS reads of this step, oldest first: the rescale votes of tile kv,
          // its P^T fragments, then the first transposed tile fragments; the
          // votes are inspected once they arrive, while the rest is in flight.
          int fl;
          lds_b32<0>(fl, flags_addr + (kv & 1) * 4);
          i32x4 pb[4];
          const uint32_t pbase = aux_addr + P::kPOff + (kv & 1) * P::kPBufB + lane * 16;
          static_for<0, 4>([&](auto nc) {
            constexpr int nt = decltype(nc)::value;
            lds_b128<nt * 1024>(pb[nt], pbase);
          });
          const uint32_t tile = ring_addr + (kv % kStages) * P::kStageB;
          uint32_t tb[kTOff];
#pragma unroll
          for (int j = 0; j < kTOff; ++j) tb[j] = tile + t_off[j];
          constexpr int kVRing = P::kPD < P::kMT ? P::kPD + 2 : P::kMT;
          i32x2 rlo[kVRing], rhi[kVRing];
          auto p_issue = [&](auto mc) {
            constexpr int mt = decltype(mc)::value;
            if constexpr (FP8) {
              lds_tr8<64 * (mt >> 2)>(rlo[mt % kVRing], tb[mt & 3]);
            } else {
              constexpr int off = 128 * (mt >> 2);
              lds_tr<off>(rlo[mt % kVRing], tb[mt & 3]);
              lds_tr<off>(rhi[mt % kVRing], tb[4 + (mt & 3)]);
            }
          };
          static_for<0, P::kPD>(p_issue);
          wait_lgkm<4 + P::kPReads * P::kPD>(fl);  // (at most 15 LDS reads are ever outstanding)
          const int fb = wave_uniform(fl);
          if (fb != 0) {
            // Rescale factors of heads whose reference max rose in tile kv.
            i32x4 al;
            lds_b128<0>(al, aux_addr + P::kAlphaOff + ((kv & 1) * 16 + l16) * 16);
            wait_lgkm<0>(al);
            const f32x4 alv = __builtin_bit_cast(f32x4, al);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
              if ((fb >> (8 * nt)) & 0xff)
#pragma unroll
                for (int mt = 0; mt < P::kMT; ++mt) st[4 * mt + nt] *= alv[nt];
          }
          static_for<0, P::kMT>([&](auto mc) {
            constexpr int mt = decltype(mc)::value;
            if constexpr (mt + P::kPD < P::kMT) p_issue(IC<mt + P::kPD>{});
            constexpr int ahead = mt + P::kPD < P::kMT ? P::kPD : P::kMT - 1 - mt;
            i32x4 av;
            if constexpr (FP8) {
              wait_lgkm<ahead>(rlo[mt % kVRing]);
              av = f8x8_to_f16x8(rlo[mt % kVRing][0], rlo[mt % kVRing][1]);
            } else {
              wait_lgkm<2 * ahead>(rlo[mt % kVRing], rhi[mt % kVRing]);
              av = i32x4{rlo[mt % kVRing][0], rlo[mt % kVRing][1], rhi[mt % kVRing][0],
                         rhi[mt % kVRing][1]};
            }
            static_for<0, 4>([&](auto nc) {
              constexpr int nt = decltype(nc)::value;
              st[4 * mt + nt] = E::mfma(av, __builtin_bit_cast(typename E::vec, pb[nt]), st[4 * mt + nt]);
            });
            constexpr int n0 = mt < P::kVSpread ? mt * P::kPerWave / P::kVSpread : P::kPerWave;
            constexpr int n1 = mt < P::kVSpread ? (mt + 1) * P::kPerWave / P::kVSpread : P::kPerWave;
            static_for<n0, n1>([&](auto nc) { copy_one(nc, nsrc, ks + kAhead); });
          });
          if (ti.last()) {
            // Segment done: normalise by the score waves' head sums and store
            // (O, slot s + g); the accumulators restart at zero.
            const size_t slot = static_cast<size_t>(piece_b(ti.piece())) + g;
            // fin[16nt + l16] for nt = 0..3
            const uint32_t fa = aux_addr + P::kFinOff + ((nfin & 1) * 64 + l16) * 4;
            int l0, l1, l2, l3;
            lds_b32<0>(l0, fa);
            lds_b32<64>(l1, fa);
            lds_b32<128>(l2, fa);
            lds_b32<192>(l3, fa);
            wait_lgkm<0>(l0, l1);
            wait_lgkm<0>(l2, l3);
            const float lt[4] = {__int_as_float(l0), __int_as_float(l1), __int_as_float(l2),
                                 __int_as_float(l3)};
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              const float inv = lt[nt] > 0.f ? 1.f / lt[nt] : 0.f;
              const bool real = head0 + 16 * nt < a.Hq;  // (rows past 16 or 32 query rows)
              store_piece_f16<P::kMT>(a, slot, head0 + 16 * nt + l16, vbase, q4, st, nt, inv, real);
            }
            ++nfin;
          }
        }
      }
      __syncthreads();  // ring stages and tables are reused by the next window
      wpos = wend;
      if (wpos < end) s_cur = find_segment(a.seg_off, a.S, wpos);
    }
  };
  if (scorer) run(IC<true>{});
  else run(IC<false>{});
}

}  // namespace

int mla_groups() { return kGroups; }

bool mla_supported(const dcp_attn_desc_t* d) {
  const int rows = desc_rows(d);
  return d->kv_kind == DCP_KV_LATENT && d->num_kv_heads == 1 && d->qk_dim == kQK &&
         d->v_dim == kV && d->q_dtype == DCP_BF16 &&
         (d->kv_dtype == DCP_BF16 || d->kv_dtype == DCP_FP8_E4M3) &&
         (rows == 16 || rows == 32 || rows % 64 == 0) && rows <= 256 &&
         (desc_q_len(d) == 1 || d->num_q_heads % 16 == 0);
}

// The producer/consumer kernel: groups of 64 heads, blocks of a multiple of 32
// tokens (a tile then lies inside one block, and per-lane copy offsets,
// row * token stride, fit in 32 bits) and of at most 8192 tokens (the tile
// table keeps a tile's offset in its block in 8 bits, and a window of
// kMaxTiles tiles must hold at least one whole block). Larger blocks take the
// general kernel. A tile's address is block id * block stride (the stride
// below 4 GiB) plus its offset in the block (the block's rows below 4 GiB).
// Multi-token decode needs each 64-row head group to hold one query token.
// Single-token decode with 16 or 32 query heads runs as one 64-row group
// padded with zero queries whose results are not stored: on MI355X that takes
// the 64-head time (bimodal batch, fp8: 1.6 ms), where the general kernel took
// 3.8 ms at 32 heads and 5.4 ms at 16.
static bool use_pp(const dcp_attn_desc_t* d) {
  const long long elt = d->kv_dtype == DCP_BF16 ? 2 : 1;
  static_assert(PP<false>::kMaxTiles >= 8192 / kT && PP<true>::kMaxTiles >= 8192 / kT,
                "a window holds one block of the largest size");
  const int rows = desc_rows(d);
  return (rows >= 64 || (desc_q_len(d) == 1 && (rows == 16 || rows == 32))) &&
         d->block_size % kT == 0 && d->block_size <= 8192 &&
         d->kv_token_stride * elt * kT < (1ll << 30) &&
         d->kv_block_stride * elt < (1ll << 32) &&
         d->kv_token_stride * elt * d->block_size < (1ll << 32) &&
         (desc_q_len(d) == 1 || d->num_q_heads % 64 == 0);
}

// (The producer/consumer kernel copies four consecutive fp8 token scales per
// lane, so a strided scale view takes the general kernel.)
bool mla_sequence_pieces(const dcp_attn_desc_t* d, int scale_ts) {
  return d->kv_kind == DCP_KV_LATENT && use_pp(d) && (d->kv_dtype != DCP_FP8_E4M3 || scale_ts == 1);
}

template <int HG, bool FP8>
static void launch_mla_hg(const MlaArgs& a, bool bs32, dim3 grid, hipStream_t stream,
                          hipEvent_t e0, hipEvent_t e1) {
  if (bs32)
    hipExtLaunchKernelGGL((mla_partial_kernel<HG, FP8, true>), grid, dim3(2 * HG * 64), 0, stream,
                          e0, e1, 0, a);
  else
    hipExtLaunchKernelGGL((mla_partial_kernel<HG, FP8, false>), grid, dim3(2 * HG * 64), 0, stream,
                          e0, e1, 0, a);
}

hipError_t launch_mla(const AttnLaunch& L, hipStream_t stream) {
  const dcp_attn_desc_t* d = L.desc;
  MlaArgs a;
  a.q = static_cast<const uint16_t*>(L.q);
  a.kv = static_cast<const char*>(L.k_cache);
  a.kv_scale = reinterpret_cast<const char*>(L.kv_scale);
  a.scale_bs = L.scale_bs;
  a.scale_ts = L.scale_ts;
  a.map = L.map;
  a.hdr = L.ws.header;
  a.sig = L.sig;
  a.wg_start = L.ws.wg_start;
  a.wg_seg = L.ws.wg_seg;
  a.seg_off = L.ws.seg_off;
  a.ws_o = L.ws.o;
  a.ws_lse = L.ws.lse;
  a.zero = reinterpret_cast<const char*>(L.ws.header->zero);
  const int elt = d->kv_dtype == DCP_BF16 ? 2 : 1;
  a.block_stride_b = d->kv_block_stride * elt;
  a.token_stride_b = d->kv_token_stride * elt;
  a.S = L.S;
  a.ncb = d->num_cache_blocks;
  a.Hq = desc_rows(d);
  a.scale_log2 = d->softmax_scale * kLog2e;
  a.cz = L.cz;
  a.causal = L.cz.q_len > 1 || L.cz.q_pos != nullptr;
  const bool fp8 = d->kv_dtype == DCP_FP8_E4M3;
  // A tile of 32 tokens lies inside one block when blocks hold a multiple of
  // 32 tokens; per-lane copy offsets (row * token stride) then fit in 32 bits.
  const bool bs32 = d->block_size % kT == 0 && a.token_stride_b * kT < (1ll << 30);
  const int heads = a.Hq < 64 ? a.Hq : 64;
  const dim3 grid(kGroups, a.Hq / heads);
  if (mla_sequence_pieces(d, L.scale_ts)) {
    const int ngrp = a.Hq >= 64 ? a.Hq / 64 : 1;  // 16 or 32 rows: one padded group
    const dim3 pgrid(kGroups * ngrp);
    if (ngrp > 1) {
      if (fp8)
        hipExtLaunchKernelGGL((mla_pp_kernel<true, true>), pgrid, dim3(512), 0, stream, L.ev_begin,
                              L.ev_end, 0, a);
      else
        hipExtLaunchKernelGGL((mla_pp_kernel<false, true>), pgrid, dim3(512), 0, stream,
                              L.ev_begin, L.ev_end, 0, a);
    } else {
      if (fp8)
        hipExtLaunchKernelGGL((mla_pp_kernel<true, false>), pgrid, dim3(512), 0, stream,
                              L.ev_begin, L.ev_end, 0, a);
      else
        hipExtLaunchKernelGGL((mla_pp_kernel<false, false>), pgrid, dim3(512), 0, stream,
                              L.ev_begin, L.ev_end, 0, a);
    }
    return hipGetLastError();
  }
  switch (heads / 16) {
    case 1:
      if (fp8) launch_mla_hg<1, true>(a, bs32, grid, stream, L.ev_begin, L.ev_end);
      else launch_mla_hg<1, false>(a, bs32, grid, stream, L.ev_begin, L.ev_end);
      break;
    case 2:
      if (fp8) launch_mla_hg<2, true>(a, bs32, grid, stream, L.ev_begin, L.ev_end);
      else launch_mla_hg<2, false>(a, bs32, grid, stream, L.ev_begin, L.ev_end);
      break;
    case 4:
      if (fp8) launch_mla_hg<4, true>(a, bs32, grid, stream, L.ev_begin, L.ev_end);
      else launch_mla_hg<4, false>(a, bs32, grid, stream, L.ev_begin, L.ev_end);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dcp
