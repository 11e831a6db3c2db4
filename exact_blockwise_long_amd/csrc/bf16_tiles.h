// Shared device plumbing of the bf16 attention kernels on gfx950: operand
// types, LDS tile geometry and swizzles, HBM -> LDS tile loads, cross-lane
// reductions, query-row bookkeeping and the double-buffered key-tile loop.
// Included by the forward (attn_bf16.hip) and backward (attn_bwd.hip)
// translation units; everything here has internal linkage.
#pragma once

#include "internal.h"
#include "tile_addr.h"

namespace ba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr int kThreads = 256;
constexpr int kTileKeys = 64;
constexpr float kTau = 8.0f;   // lazy-rescale headroom, log2 units

// Tile geometry for head_dim D, W waves per workgroup (the W waves share the
// loads of every tile) and TK keys per tile.
template <int D, int W = 4, int TK = kTileKeys>
struct Cfg {
  static constexpr int ROWB = D * 2;                  // bytes per K or V row in LDS
  static constexpr int CPR = D / 8;                   // 16-byte chunks per row
  static constexpr int TILEB = TK * ROWB;             // bytes of one K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;            // one stage: a K tile and a V tile
  static constexpr int RPI = 64 / CPR;                // rows per wave-wide 1 KiB load
  static constexpr int LPW = TK / RPI / W;            // loads per wave per tile (each of K and V)
  static constexpr int DC = D / 32;                   // 32-wide d chunks (QK^T K-dim steps)
  static constexpr int DB = D / 16;                   // 16-wide d blocks of O^T
};

// Reductions over the 4 lanes that share lane % 16 (one query column).
//
// v_permlane16_swap(a, b) returns (a with its odd 16-lane rows replaced by
// b's even rows, b with its even rows replaced by a's odd rows); with a = b = x
// the two results hold x and its lane ^ 16 partner, so combining them is one
// butterfly step, and v_permlane32_swap likewise pairs lane ^ 32 (checked on
// the hardware).  Registers only, no LDS crossbar.  (The two results are
// copied to scalars before the bit casts: a bit cast applied directly to an
// element of the returned vector reads element 0 with this compiler.)
struct PairF {
  float a, b;
};
__device__ inline PairF swap16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  return PairF{__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1)};
}
__device__ inline PairF swap32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  return PairF{__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1)};
}
__device__ inline float xor16_pair_max(float x) { const PairF p = swap16(x); return fmaxf(p.a, p.b); }
__device__ inline float xor32_pair_max(float x) { const PairF p = swap32(x); return fmaxf(p.a, p.b); }
__device__ inline float xor16_pair_sum(float x) { const PairF p = swap16(x); return p.a + p.b; }
__device__ inline float xor32_pair_sum(float x) { const PairF p = swap32(x); return p.a + p.b; }
__device__ inline float wave_max_cols(float x) { return xor32_pair_max(xor16_pair_max(x)); }
__device__ inline float wave_sum_cols(float x) { return xor32_pair_sum(xor16_pair_sum(x)); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to a packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ inline bf16x2 pack_bf16x2(float a, float b) { return __builtin_convertvector(f32x2{a, b}, bf16x2); }

// Cache policy of the K/V tile loads.  kCacheReuse is the default: other
// workgroups read the same tiles (a KV head's keys serve every row tile of its
// query rows) and find them in L2.  kCacheStream marks the loads non-temporal
// (nt): for a launch whose K/V bytes are each read by a single workgroup, as
// in the one-row-tile fan-out decode and shard sweeps, they then do not evict
// lines that are reused.  Measured: the 64K fan-out decode 77 -> 71 us and the
// 1M shard sweep 132 -> 126 us with kCacheStream; the prefill walk, whose
// tiles are re-read, loses 10 % with it.
constexpr int kCacheReuse = 0;
constexpr int kCacheStream = 2;

// One 16-byte-per-lane buffer load straight into LDS (buffer_load_dwordx4 ...
// lds): lane i's bytes land at dst + 16 * i.  The host compilation pass never
// runs device code but rejects this builtin in some template contexts, so the
// call is compiled for the device only.
template <int kAux = kCacheReuse>
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t dst, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(size_t)dst, 16, voff, soff, 0, kAux);
#endif
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Per-workgroup description of the query rows.
struct RowCtx {
  int f0, f1;              // flat row range [f0, f1) of this tile
  int g;                   // KV head
  int b;                   // sequence
  int64_t row0;            // state row of the sequence's first row: b * q_len * Hq
  int64_t qpos_min, qpos_max;
};

// A key range as the kernels see it: K and V of one KV head (the address of
// key 0), the byte stride between keys, the absolute position of key 0 and
// the number of keys.
struct KVSrc {
  const char* kb;
  const char* vb;
  uint32_t kst, vst;       // bytes between consecutive keys
  int64_t pos0;
  int n;
};

template <int D>
__device__ inline KVSrc make_src(const Seg& s, const RowCtx& rc) {
  KVSrc r;
  r.kb = (const char*)s.k + ((int64_t)rc.g * s.ks_h + (int64_t)rc.b * s.ks_b) * 2;
  r.vb = (const char*)s.v + ((int64_t)rc.g * s.vs_h + (int64_t)rc.b * s.vs_b) * 2;
  r.kst = (uint32_t)(s.ks_t * 2);
  r.vst = (uint32_t)(s.vs_t * 2);
  r.pos0 = s.pos0;
  r.n = s.n;
  return r;
}

// Per-lane byte offsets, within a tile, of the 16-byte chunks this lane moves
// (tile_lane_offset).  They depend only on the key strides, so they are
// computed once per segment.
template <int D, int W = 4, int TK = kTileKeys>
struct LaneOffs {
  uint32_t k[Cfg<D, W, TK>::LPW];
  uint32_t v[Cfg<D, W, TK>::LPW];
};

template <int D, int W = 4, int TK = kTileKeys>
__device__ inline LaneOffs<D, W, TK> lane_offsets(const KVSrc& src, int wave, int lane) {
  using C = Cfg<D, W, TK>;
  LaneOffs<D, W, TK> o;
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    o.k[j] = tile_lane_offset<D, W, TK>(src.kst, wave, lane, j);
    o.v[j] = tile_lane_offset<D, W, TK>(src.vst, wave, lane, j);
  }
  return o;
}

// Issue the HBM -> LDS loads of the TK-key tile starting at key k0 of `src`,
// of which the first n_read keys (k0 < n_read <= src.n) may be read.  The
// tile gets buffer resources of its own (tile_addr.h): based at key k0, they
// end at the last byte of key n_read - 1, and the scalar offset is 0, so the
// range check covers every lane's whole offset.  Rows at or past n_read load
// zeros without touching memory; their scores are masked, so their P is
// exactly 0 and 0 * V adds nothing.  `kdst` and `vdst` are the LDS byte
// addresses of the stage's K and V tiles.
template <int D, int kAux = kCacheReuse, int W = 4, int TK = kTileKeys>
__device__ inline void issue_tile(const KVSrc& src, const LaneOffs<D, W, TK>& offs, int k0, int n_read,
                                  uint32_t kdst, uint32_t vdst, int wave) {
  using C = Cfg<D, W, TK>;
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(src.kb + (uint32_t)k0 * src.kst, tile_records<D>(n_read, k0, src.kst));
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(src.vb + (uint32_t)k0 * src.vst, tile_records<D>(n_read, k0, src.vst));
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const uint32_t rbase = (uint32_t)((wave * C::LPW + j) * C::RPI);
    lds_dma16<kAux>(rk, kdst + rbase * C::ROWB, offs.k[j], 0);
    lds_dma16<kAux>(rv, vdst + rbase * C::ROWB, offs.v[j], 0);
  }
}

// The V tile of the stage whose K tile is at `kl` (run_segments' layout).
template <int D, int TK>
__device__ inline const lds_char* v_tile_of(const lds_char* kl) {
  return kl - 2 * Cfg<D, 4, TK>::TILEB;
}

// Number of keys of segment `s` that some row of the tile can see.
__device__ inline int seg_effective(const Seg& s, const QSide& qs, const RowCtx& rc) {
  if (!qs.causal) return s.n;
  int64_t lim = rc.qpos_max - s.pos0 + 1;
  if (lim <= 0) return 0;
  return (int)min((int64_t)s.n, lim);
}

// The per-lane row bookkeeping shared by every kernel.  Cheap to recompute,
// so the kernels rebuild it after the key loop instead of keeping it live.
struct LaneRows {
  int qrel[2];       // query position minus the tile's first query position
  int64_t srow[2];   // state row (b*q_len + t)*Hq + h
  bool valid[2];
  const uint16_t* qptr[2];
};

__device__ inline LaneRows lane_rows(const QSide& qs, const RowCtx& rc, int wave, int lane) {
  LaneRows lr;
  const int t0 = rc.f0 / qs.G;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int f = rc.f0 + wave * 32 + qb * 16 + (lane & 15);
    lr.valid[qb] = f < rc.f1;
    int fc = min(f, rc.f1 - 1);
    int t = fc / qs.G;
    int j = fc - t * qs.G;
    int h = rc.g * qs.G + j;
    lr.qrel[qb] = t - t0;
    lr.srow[qb] = rc.row0 + (int64_t)t * qs.Hq + h;
    lr.qptr[qb] = (const uint16_t*)qs.q + (int64_t)rc.b * qs.qs_b + (int64_t)t * qs.qs_t + (int64_t)h * qs.qs_h;
  }
  return lr;
}

__device__ inline void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The key-tile loop over a list of segments, double-buffered through LDS: the
// next tile loads while the current one is multiplied.  One barrier per tile:
// after it, every wave's loads of the tile about to be used have landed and
// every wave is done with the stage the next load overwrites.  The loop is
// unrolled by two so each stage's LDS offsets are compile-time constants.
// Segment bookkeeping (visible key count, buffer resources, per-lane offsets)
// runs only when a cursor crosses into another segment.
//
// LDS layout: the two stages' V tiles first, then their K tiles (V of stage s
// at s * TILEB, K of stage s at (2 + s) * TILEB), so every transposing read
// of a V tile addresses from a per-lane base with an immediate offset below
// 64 KiB that folds in the stage, the key chunk and the row half.
//
// `tile(stage, need_mask, n_valid, krel)` computes one tile for the calling
// wave: `stage` is the LDS address of the tile's K (its V is at stage -
// 2 * TILEB, see v_tile_of);
// keys at or past n_valid are invalid and, for causal problems, key kk sits
// at position krel + kk relative to the tile's first query.  It runs only in
// waves that own rows.
template <int D, int kAux = kCacheReuse, int W = 4, int TK = kTileKeys, class GetSeg, class TileFn>
__device__ inline void run_segments(const QSide& qs, const RowCtx& rc, int n_seg, GetSeg get_seg, TileFn tile,
                                    lds_char* lds, bool wave_active) {
  using C = Cfg<D, W, TK>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // First segment at or after s with a key some row of the tile can see.
  auto next_nonempty = [&](int s, int& n_eff) {
    for (; s < n_seg; ++s) {
      n_eff = seg_effective(get_seg(s), qs, rc);
      if (n_eff > 0) return s;
    }
    n_eff = 0;
    return n_seg;
  };

  // issue cursor
  int is_n = 0;
  int is = next_nonempty(0, is_n);
  if (is >= n_seg) return;
  int ik = 0;
  KVSrc isrc = make_src<D>(get_seg(is), rc);
  LaneOffs<D, W, TK> ilo = lane_offsets<D, W, TK>(isrc, wave, lane);
  // compute cursor
  int cs = is, ck = 0, cn = is_n;
  int64_t cpos0 = get_seg(cs).pos0;

  const uint32_t lds_addr = (uint32_t)(size_t)lds;
  auto issue_next = [&](int stage) {
    issue_tile<D, kAux, W, TK>(isrc, ilo, ik, is_n, lds_addr + (uint32_t)((2 + stage) * C::TILEB),
                               lds_addr + (uint32_t)(stage * C::TILEB), wave);
    ik += TK;
    if (ik >= is_n) {
      is = next_nonempty(is + 1, is_n);
      ik = 0;
      if (is < n_seg) {
        isrc = make_src<D>(get_seg(is), rc);
        ilo = lane_offsets<D, W, TK>(isrc, wave, lane);
      }
    }
  };

  // One tile: wait for it, let the next one start loading, multiply.
  auto step = [&](int cur, int nxt) {
    wait_all_loads();
    __syncthreads();
    if (is < n_seg) issue_next(nxt);
    if (wave_active) {
      const int n_valid = min(TK, cn - ck);
      const int64_t kpos0 = cpos0 + ck;
      const bool need_mask = (n_valid < TK) || (qs.causal && kpos0 + TK - 1 > rc.qpos_min);
      // Visited keys satisfy kpos0 <= qpos_max, so the offset fits easily in 32 bits
      // whenever a mask is needed; far-past tiles are clamped (never masked).
      const int64_t krel64 = kpos0 - rc.qpos_min;
      const int krel = (int)max((int64_t)-(1 << 30), min((int64_t)(1 << 30), krel64));
      tile(lds + (2 + cur) * C::TILEB, need_mask, n_valid, krel);
    }
    ck += TK;
    if (ck >= cn) {
      cs = next_nonempty(cs + 1, cn);
      ck = 0;
      if (cs < n_seg) cpos0 = get_seg(cs).pos0;
    }
  };

  issue_next(0);
  while (true) {
    step(0, 1);
    if (cs >= n_seg) break;
    step(1, 0);
    if (cs >= n_seg) break;
  }
  // Leave no load in flight into LDS that a later phase might reuse.
  wait_all_loads();
}

__device__ inline RowCtx make_rowctx(const QSide& qs, int f0, int f1, int g, int b) {
  RowCtx rc;
  rc.f0 = f0;
  rc.f1 = f1;
  rc.g = g;
  rc.b = b;
  rc.row0 = (int64_t)b * qs.q_len * qs.Hq;
  rc.qpos_min = qs.q_pos0 + f0 / qs.G;
  rc.qpos_max = qs.q_pos0 + (f1 - 1) / qs.G;
  return rc;
}

}  // namespace
}  // namespace ba
