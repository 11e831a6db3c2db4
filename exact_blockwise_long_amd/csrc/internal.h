// Internal interface between the C-ABI front end (api.hip) and the kernel
// translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/blockattn.h"

namespace ba {

constexpr int kMaxSeg = BLOCKATTN_MAX_VISITS;
constexpr int kMaxParts = BLOCKATTN_MAX_MERGE_PARTS;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One contiguous key range: keys [0, n) of this segment sit at absolute
// positions pos0 + i; k/v point at key 0 of the range of sequence 0, the
// range of sequence b sitting b * ks_b (vs_b) elements further.
struct Seg {
  const void* k;
  const void* v;
  int64_t ks_t, ks_h, vs_t, vs_h;
  int64_t ks_b, vs_b;
  int64_t pos0;
  int32_t n;
  int32_t pad_;
};

// The query side shared by every attention kernel.  Query "flat rows" of KV
// head g of sequence b are f = t * G + j for token t < q_len and group member
// j < G; flat row f reads q head g * G + j of token t of sequence b (b * qs_b
// elements after q), sits at position q_pos0 + t, and owns state row
// (b * q_len + t) * Hq + g * G + j.  A workgroup serves one (sequence, KV head).
struct QSide {
  const void* q;
  int64_t qs_t, qs_h, qs_b;
  int64_t q_pos0;
  int32_t Hq, Hkv, G, q_len;
  int32_t B;      // sequences (>= 1)
  float c;        // logit scale * log2(e): the kernels work in base 2
  int32_t causal;
};

// Walk: each workgroup owns one tile of flat rows of one KV head and visits
// seg[0..n_seg) in order, carrying the state in registers.
struct WalkArgs {
  QSide qs;
  float* m;
  float* l;
  float* o;
  int32_t reset;
  int32_t n_seg;
  Seg seg[kMaxSeg];
  // With fin_out set the walk ends by finalising instead of writing the state:
  // out[r * fin_stride + d] = O / l (bf16 when fin_bf16, else fp32) and, if
  // fin_lse is set, fin_lse[r] = m + ln l; empty rows give 0 and -inf.
  void* fin_out;
  int32_t fin_bf16;
  int64_t fin_stride;
  float* fin_lse;
};

// Split: workgroup (row tile, sequence, KV head) x chunk; chunk c of the segment table
// lies in segment s with chunk_begin[s] <= c < chunk_begin[s+1] and covers
// keys [(c - chunk_begin[s]) * chunk_len, ...) of it.  Each writes the partial
// state of its rows over its chunk into slot c of the workspace:
// ws_m[c * R + r], ws_l[c * R + r], ws_o[(c * R + r) * D + d] with R = q_len * Hq.
struct SplitArgs {
  QSide qs;
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int64_t R;
  int32_t chunk_len;
  int32_t n_seg;
  int32_t wide;      // 1: 8-wave workgroups and 256-row tiles
  int32_t chunk_begin[kMaxSeg + 1];
  Seg seg[kMaxSeg];
};

// Fan-out over the last T tokens of each branch (T = 1: decode): one launch
// of prefix-chunk jobs and branch-suffix jobs.  The query rows are one block
// of n_branches * T tokens (qs.q_len), branch b's tokens being b*T .. b*T+T-1.
// Prefix job (row tile, KV head g, chunk c): flat rows of the tile against
// prefix keys [c * chunk_len, ...), no mask, written to workspace slot c.
// Suffix job for KV head g: with srt == 1, each branch b of a group of bpj
// consecutive branches; otherwise one row tile rt of one branch b -- the
// branch's flat rows [b*T*G, (b+1)*T*G) (tile rt of them) against its own
// suffix (suffix k/v are [n_branches, S, Hkv, D]), causal with new token i at
// suffix position S - T + i, written to slot suffix_slot.  Row tiles are 128
// rows, or 256 with wide.
struct FanoutArgs {
  QSide qs;          // q_len = n_branches, non-causal
  Seg prefix;        // the whole shared prefix
  int32_t row_tiles; // row tiles of one KV head's rows
  int32_t chunk_len;
  int32_t n_chunks;
  const void* sk;
  const void* sv;
  int32_t S;
  int32_t T;         // new tokens per branch
  int32_t suffix_slot;
  int32_t srt;       // row tiles of one branch's rows
  int32_t bpj;       // branches per suffix job (srt == 1)
  int32_t wide;      // 1: 8-wave workgroups and 256-row tiles (row_tiles, srt in those)
  int32_t prefix_keys;  // key tile of the prefix jobs: 128 (wide launches) or 64
  // Paged K/V (prefix_pages != nullptr): prefix.k / prefix.v are the pools,
  // page p of a table starts page_len * Hkv * D elements after the pool base.
  const int32_t* prefix_pages;
  const int32_t* suffix_pages;   // n_branches rows of suffix_pages_per_branch ids
  int32_t page_len;
  int32_t n_pool_pages;
  int32_t suffix_pages_per_branch;
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int64_t R;
};

// Merge of strided workspace partials: group i merges slots
// [part_begin[i], part_begin[i+1]) (plus the current contents of out[i] when
// has_init) into out[i]; or, with fin_out set, finalises straight to bf16.
struct MergeGroupArgs {
  const float* pm;
  const float* pl;
  const float* po;
  int64_t R;
  int32_t n_groups;
  int32_t has_init;
  int32_t part_begin[kMaxSeg + 1];
  float* out_m[kMaxSeg];
  float* out_l[kMaxSeg];
  float* out_o[kMaxSeg];
  uint16_t* fin_out;      // bf16 rows when not null (finalise instead of out_*)
  float* fin_out_f32;     // or fp32 rows when not null
  int64_t fin_stride;     // elements between output rows (0: D)
  float* fin_lse;         // optional with fin_out / fin_out_f32
};

struct MergePtrArgs {
  int32_t n_parts;
  int64_t R;
  const float* m[kMaxParts];
  const float* l[kMaxParts];
  const float* o[kMaxParts];
  float* out_m;
  float* out_l;
  float* out_o;
};

struct FinalizeArgs {
  const float* m;
  const float* l;
  const float* o;
  int64_t R;
  void* out;
  int32_t out_bf16;
  int64_t out_stride;
  float* lse;
};

// Backward of one call's visits: dq (fp32, state-row order [rows, D]) and the
// visited blocks' dk, dv (fp32 [n, Hkv, D] each) accumulate.  dout uses Q's
// strides; lse (natural log) and delta are per state row.  The dK/dV kernel's
// grid covers tile_begin[n_seg] tiles of kDkvKeys keys: tiles [tile_begin[s],
// tile_begin[s+1]) are segment s's.
constexpr int kDkvKeys = 128;   // keys per workgroup of the dK/dV kernel

struct BwdArgs {
  QSide qs;
  const void* dout;
  const float* lse;
  const float* delta;
  float* dq;
  float scale;
  uint32_t q_bytes;      // bytes from one sequence's q (and dout) to the end of its last row
  uint32_t rows_bytes;   // bytes of lse and delta
  uint32_t g_magic;      // floor((2^32 - 1) / G): flat row -> token by one multiply-high and one fix-up
  int32_t n_seg;
  int32_t tile_begin[kMaxSeg + 1];
  Seg seg[kMaxSeg];
  float* dk[kMaxSeg];
  float* dv[kMaxSeg];
};

// delta[r] = sum_d dout[r * dout_stride + d] * out[r * out_stride + d].
struct DeltaArgs {
  int64_t rows;
  const void* out;
  int32_t out_bf16;
  int64_t out_stride;
  const void* dout;
  int64_t dout_stride;
  float* delta;
};

// Rows per workgroup tile of the bf16 attention kernels.
constexpr int kTileRows = 128;
constexpr int kWideTileRows = 256;   // row tile of the 8-wave split and fan-out workgroups

// 8-wave workgroups with 256-row tiles for the split and fan-out launches
// (1 = on, when a KV head's rows fill two or more 128-row tiles).
#ifndef BA_SPLIT_WIDE
#define BA_SPLIT_WIDE 1
#endif
#ifndef BA_FANOUT_WIDE
#define BA_FANOUT_WIDE 1
#endif
// Workgroups the fan-out planner aims for (prefix-chunk jobs plus suffix jobs).
#ifndef BA_FANOUT_TARGET_WG
#define BA_FANOUT_TARGET_WG 512
#endif
constexpr int kFanoutTargetWorkgroups = BA_FANOUT_TARGET_WG;

// Chunk `chunk` of a split launch's segment table as a segment of its own
// (T: the element type of K and V).
template <typename T>
__device__ inline Seg chunk_seg(const Seg* seg, int n_seg, const int32_t* chunk_begin, int chunk_len, int chunk) {
  int s_i = 0;
  while (s_i + 1 < n_seg && chunk_begin[s_i + 1] <= chunk) ++s_i;
  const Seg& base = seg[s_i];
  const int k_off = (chunk - chunk_begin[s_i]) * chunk_len;
  Seg cs = base;
  cs.k = (const T*)base.k + (int64_t)k_off * base.ks_t;
  cs.v = (const T*)base.v + (int64_t)k_off * base.vs_t;
  cs.pos0 = base.pos0 + k_off;
  cs.n = min(chunk_len, base.n - k_off);
  return cs;
}

hipError_t launch_walk_bf16(const WalkArgs& a, int D, hipStream_t s);
hipError_t launch_split_bf16(const SplitArgs& a, int n_chunks, int D, hipStream_t s);
hipError_t launch_fanout_bf16(const FanoutArgs& a, int n_jobs, int D, hipStream_t s);
hipError_t launch_walk_f32(const WalkArgs& a, int D, hipStream_t s);
hipError_t launch_split_f32(const SplitArgs& a, int n_chunks, int D, hipStream_t s);
hipError_t launch_merge_groups(const MergeGroupArgs& a, int D, hipStream_t s);
hipError_t launch_merge_ptrs(const MergePtrArgs& a, int D, hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs& a, int D, hipStream_t s);
hipError_t launch_delta(const DeltaArgs& a, int D, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, int n_key_tiles, int D, hipStream_t s);

}  // namespace ba
