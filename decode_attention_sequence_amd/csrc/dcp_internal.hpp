// Internal declarations shared by the libdcp translation units (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dcp.h"

namespace dcp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

#define DCP_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Work plan.
//
// The tokens of one decode call are organised in segments: segment s is the
// pair (sequence b = s / D, shard r = s % D) and holds the cache blocks of
// sequence b that shard r owns, in local order i = 0, 1, ...; local block i
// is column r + D * i of row b of the block table. With D = 1 and r = 0 the
// same description covers one shard's local table.
//
// A planning kernel counts the blocks of every segment and writes their
// prefix sums. The attention kernels then split the concatenation of all
// segments into G equal ranges of `chunk` blocks, one per work group, so every
// work group streams the same number of cache blocks whatever the length mix.
// Where a range crosses a segment boundary the work group emits one partial
// (O, LSE) per segment piece; the piece of segment s handled by work group g
// is stored in slot s + g, which is unique because both s and g grow along
// the concatenation. Slots used <= S + G - 1.
// ---------------------------------------------------------------------------
// Signature of a plan: the launch shape it was made for. The planning kernel
// writes it into the workspace header; each kernel that reads a plan compares
// it with its own launch's first and, when they differ, reads nothing of the
// plan (attention: no work; piece merge: NaN outputs), so a workspace planned
// for another shape, or never planned, is never taken for a plan.
struct PlanSig {
  int32_t magic;
  int32_t S, G, B, rows, seq_pieces;
  int32_t D, bs, width, tok_r, tok_D;
  int32_t v_dim;
};
constexpr int32_t kPlanMagic = 0x31504344;  // "DCP1"

struct PlanHeader {
  int32_t total;  // blocks over all segments
  int32_t pad[3];
  int32_t zero[4];  // 16 zero bytes: copy source for tile rows without a token
  PlanSig sig;
};

__device__ __forceinline__ bool plan_matches(const PlanSig& want, const PlanHeader* hdr) {
  const PlanSig h = hdr->sig;
  return h.magic == want.magic && h.S == want.S && h.G == want.G && h.B == want.B &&
         h.rows == want.rows && h.seq_pieces == want.seq_pieces && h.D == want.D &&
         h.bs == want.bs && h.width == want.width && h.tok_r == want.tok_r &&
         h.tok_D == want.tok_D && h.v_dim == want.v_dim;
}
// Workspace layout: PlanHeader, seg_off[S + 1], cost_off[S + 1],
// wg_start[G + 1], seq_slots[B][2], wg_seg[G + 1] and lens[B] (int32), then at
// 256-byte alignment lse slots [num_slots, Hq] fp32, then o slots [num_slots,
// Hq, v_dim] fp32. Sequence pieces (the latent producer/consumer kernel) fill
// only the first half of each row: v_dim fp16 values, each kPieceSlice-column
// slice scaled by a power of two, then the slices' scales (fp32).

struct SegMap {
  const int32_t* table;  // [B, width]
  const int32_t* lens;   // [B], tokens (global, or this shard's local count)
  int32_t width;         // table row width
  int32_t D;             // segments per sequence
  int32_t bs;            // block size
  int32_t batch;
  // Token-level interleave ("vLLM长序列推理优化", section 2.2): one shard's
  // view of a global cache, shard tok_r of tok_D holding the positions
  // t = tok_r + tok_D * i. Its blocks are the global blocks with bs the global
  // block size / tok_D, and lens are global lengths, of which the shard holds
  // ceil((L - tok_r) / tok_D). tok_D = 1: lens are the tokens themselves.
  int32_t tok_r;
  int32_t tok_D;
};

// Tokens of sequence b, clamped to what its table row can address.
__device__ __forceinline__ int seq_tokens(const SegMap& m, int b) {
  int L = m.lens[b];
  const long long cap = static_cast<long long>(m.width) * m.bs * m.tok_D;
  L = L < 0 ? 0 : (L > cap ? static_cast<int>(cap) : L);
  if (m.tok_D > 1) L = L > m.tok_r ? (L - m.tok_r + m.tok_D - 1) / m.tok_D : 0;
  return L;
}

__device__ __forceinline__ int segment_blocks(const SegMap& m, int s) {
  int b = s / m.D, r = s - b * m.D;
  int L = seq_tokens(m, b);
  int nb = (L + m.bs - 1) / m.bs;
  return nb > r ? (nb - r + m.D - 1) / m.D : 0;
}

// Token range of one piece: local blocks [i0, i1) of segment s.
struct Piece {
  int s, b, r;
  int i0, i1;
  int L;     // tokens of the whole sequence (clamped)
  int ntok;  // tokens covered by this piece
};

__device__ __forceinline__ Piece make_piece(const SegMap& m, int s, int i0, int i1) {
  Piece p;
  p.s = s;
  p.b = s / m.D;
  p.r = s - p.b * m.D;
  p.i0 = i0;
  p.i1 = i1;
  p.L = seq_tokens(m, p.b);
  int last_col = p.r + m.D * (i1 - 1);
  int full = (i1 - i0) * m.bs;
  int tail = m.bs * (last_col + 1) - p.L;  // > 0 only for the sequence's last block
  p.ntok = full - (tail > 0 ? tail : 0);
  return p;
}

// Table column of the local block holding piece token tau.
__device__ __forceinline__ int piece_col(const SegMap& m, const Piece& p, int tau) {
  return p.r + m.D * (p.i0 + tau / m.bs);
}

// Segment containing concatenated block index x (seg_off non-decreasing,
// seg_off[0] = 0, x < seg_off[S]).
__device__ __forceinline__ int find_segment(const int32_t* seg_off, int S, int x) {
  int lo = 0, hi = S;  // answer in [0, S)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (seg_off[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Work group whose block range holds concatenated block x: the last g in
// [0, G) with wg_start[g] <= x (ranges are consecutive; empty ones share their
// start with the next range).
__device__ __forceinline__ int wg_of(const int32_t* wg_start, int G, int x) {
  int lo = 0, hi = G;  // answer in [0, G)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (wg_start[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Logical work-group index with consecutive ranges kept on one XCD: hardware
// dispatches work group i to XCD i % 8, so groups that share a sequence (and
// its query rows) read them through the same L2.
__device__ __forceinline__ int xcd_logical_group(int i, int G) {
  int per = G >> 3;
  return (i & 7) * per + (i >> 3);
}

// ---------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------
// Cache policy of the direct-to-LDS copies of cached K/V rows: nontemporal
// ("nt"), since every cached byte is read once per call. Measured on MI355X
// with a pure streaming kernel: 6.6 TB/s with the hint against 6.2 without.
constexpr int kCopyPolicy = 2;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// c + the bf16 values packed in pk (v_dot2c_f32_bf16 against ones).
// A product with bf16 probabilities is normalised by the sum of exactly those
// rounded probabilities: the result is then a convex combination of value rows
// under the rounded weights, and its error scales with how far the value rows
// lie from the result rather than with their magnitude (a head that attends to
// one token returns that token's row).
__device__ __forceinline__ float add_bf16x2(uint32_t pk, float c) {
  const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, c, false);
}
__device__ __forceinline__ float add_bf16x8(i32x4 pk, float c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) c = add_bf16x2(static_cast<uint32_t>(pk[i]), c);
  return c;
}

// ---------------------------------------------------------------------------
// Host-side launchers (defined in the .hip files)
// ---------------------------------------------------------------------------
struct WorkspaceView {
  PlanHeader* header;
  int32_t* seg_off;   // [S + 1] first concatenated block of each segment
  int32_t* cost_off;  // [S + 1] planning scratch: cost prefix sums
  int32_t* wg_start;  // [G + 1] first block of each work group's range
  int32_t* seq_slots; // [B][2] slot range [lo, hi) holding sequence b's pieces
  int32_t* wg_seg;    // [G + 1] segment holding each range's first block
  int32_t* lens;      // [B] the sequence lengths the plan was made with
  float* lse;
  float* o;
  int num_slots;
};

// Columns of a sequence piece's row that share one scale: a value wave's slice.
constexpr int kPieceSlice = 128;

// Partial slots of a launch: one per (work group, segment) piece, S + G - 1;
// with sequence pieces (one partial per work group and sequence), B + G - 1.
size_t workspace_bytes_for(int S, int G, int B, int Hq, int v_dim, bool seq_pieces);
WorkspaceView carve_workspace(void* ws, int S, int G, int B, int Hq, int v_dim, bool seq_pieces);

// The plan also keeps a copy of the lengths it counted (ws.lens): the
// attention and merge kernels of a launch read the lengths from there, so a
// plan and the kernels that run it always agree on them.
hipError_t launch_plan(const SegMap& m, int S, int G, int seg_cost, int Hq, bool seq_pieces,
                       const PlanSig& sig, WorkspaceView ws, hipStream_t stream);
hipError_t launch_merge_pieces(const SegMap& m, const WorkspaceView& ws, const PlanSig& sig, int G,
                               int Hq, int v_dim, void* out, dcp_dtype_t out_dtype,
                               float* lse_out, hipStream_t stream);
hipError_t launch_merge_partials(const float* o, const float* lse, int P, int B, int H, int v_dim,
                                 void* out, dcp_dtype_t out_dtype, float* lse_out,
                                 hipStream_t stream);
hipError_t launch_remap(const int32_t* table, const int32_t* lens, int B, int max_blocks, int bs,
                        int D, bool contiguous, int32_t* local_table, int32_t* local_lens,
                        hipStream_t stream);

hipError_t launch_remap_update(const int32_t* table, const int32_t* old_lens, const int32_t* lens,
                               int B, int max_blocks, int bs, int D, int32_t* local_table,
                               int32_t* local_lens, hipStream_t stream);

hipError_t launch_kv_append(const dcp_attn_desc_t* d, int n_tokens, const int32_t* token_seq,
                            const int32_t* positions, const void* k_new, const void* v_new,
                            dcp_dtype_t new_dtype, int shard, const int32_t* table, void* k_cache,
                            void* v_cache, float* kv_scale, hipStream_t stream);

// Multi-token decode. A sequence carries q_len query tokens (rows t * hq + h
// of q, partials and output); query t of sequence b sits at position
// q_pos[b] + t (q_pos null: seq_tokens - q_len) and sees the positions up to
// its own. Table column col of the segment map holds global block
// pos_r + pos_D * col (fused path: 0 + 1 * col; one shard's local table:
// shard + D * col), which gives every cached token its global position.
struct Causal {
  const int32_t* q_pos;
  int q_len;  // 1: single-token decode, no mask
  int hq;     // query heads per token
  int pos_r, pos_D;
};

__device__ __forceinline__ long long first_query_pos(const Causal& c, const SegMap& m, int b) {
  return c.q_pos ? static_cast<long long>(c.q_pos[b])
                 : static_cast<long long>(seq_tokens(m, b)) - c.q_len;
}
__device__ __forceinline__ long long global_pos(const Causal& c, int col, int bs, int slot) {
  return (static_cast<long long>(c.pos_r) + static_cast<long long>(c.pos_D) * col) * bs + slot;
}

struct AttnLaunch {
  const dcp_attn_desc_t* desc;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* kv_scale;
  SegMap map;
  int S;
  WorkspaceView ws;
  Causal cz;
  // fp8 scale of slot j of block id: kv_scale[id * scale_bs + scale_ts * j]
  // (scale_bs = block size, scale_ts = 1, except for a token-interleave view)
  int scale_bs;
  int scale_ts;
  PlanSig sig;  // the plan this launch reads
  // Optional events that the attention kernel's own dispatch records at its
  // start and end (hipExtLaunchKernel): the kernel's duration without the
  // marker packets a separate hipEventRecord puts between the kernels.
  hipEvent_t ev_begin = nullptr;
  hipEvent_t ev_end = nullptr;
};

// Query tokens per sequence and query rows per sequence of a descriptor (a
// descriptor whose struct_size ends before q_len has one query token).
inline int desc_q_len(const dcp_attn_desc_t* d) {
  const bool has = d->struct_size >= offsetof(dcp_attn_desc_t, q_len) + sizeof(int32_t);
  return has && d->q_len > 1 ? d->q_len : 1;
}
inline int desc_rows(const dcp_attn_desc_t* d) { return desc_q_len(d) * d->num_q_heads; }

// Work groups per launch for each kernel family (a property of the kernel, not
// of the device, so workspace sizes are pure functions of the descriptor).
int mla_groups();
int gqa_groups(const dcp_attn_desc_t* desc);
bool mla_supported(const dcp_attn_desc_t* desc);
// True when the MLA kernel for desc keeps one partial per work group and
// sequence (slot b + g) rather than one per work group and segment (slot s + g).
// scale_ts: token stride of the fp8 scales (1 except in a token-interleave view).
bool mla_sequence_pieces(const dcp_attn_desc_t* desc, int scale_ts = 1);
bool gqa_supported(const dcp_attn_desc_t* desc);
hipError_t launch_mla(const AttnLaunch& a, hipStream_t stream);
hipError_t launch_gqa(const AttnLaunch& a, hipStream_t stream);

}  // namespace dcp
