// bf16 blockwise attention with running online-softmax state, for gfx950.
//
// Computes, for a tile of query rows and a sequence of key ranges, the
// recurrence of "RingAttention and Context Parallelism" (llms.blog), section 2
// (state-transition box): per row, m_new = max(m_old, max_j s_j),
// P = exp(s - m_new), l_new = exp(m_old - m_new) l_old + sum_j P_j,
// O_new = exp(m_old - m_new) O_old + P V, from the initial state of its
// section 3 (m = -inf, l = 0, O = 0), with the causal rule of its section 5.
//
// Mapping onto CDNA4:
//  * A workgroup is 4 waves and owns 128 "flat rows" (query token x member of
//    one GQA group) that all read the same KV head, so one K/V tile in LDS
//    serves every query head of the group ("AHBM Agentic Runtime
//    Architecture" s.1.3: rows batched against shared KV).
//  * K/V tiles of 64 keys go HBM -> LDS with buffer_load_dwordx4 ... lds (no
//    register staging), double-buffered: the next tile's loads are in flight
//    while the current one is multiplied (two LDS stages of 32 KiB fit two
//    workgroups per compute unit; a deeper third stage measured slower).  16-byte chunks of every LDS row are
//    XOR-swizzled by row so both operand reads below are bank-conflict free.
//  * Each wave owns 32 rows.  Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_bf16: K (ds_read_b128 from LDS) is the A operand and
//    Q (kept in registers for the whole kernel) the B operand.  The S^T
//    accumulator holds, per lane, 4 consecutive keys of one query row --
//    exactly the B-operand layout of O^T = V^T P^T, so P never leaves
//    registers.  The V^T A-operand comes straight from the row-major V tile
//    through the LDS transpose read ds_read_b64_tr_b16.
//  * Softmax statistics are per query column: the 4 lanes of a column share a
//    row, the row max needs two cross-lane exchanges, and the row sum is kept
//    as per-lane partial sums until the end.  exp is exp2 on v_exp_f32 with
//    the logit scale folded into one FMA by scale*log2(e).
//  * Lazy rescaling: a row's reference max only moves when a tile's max
//    exceeds it by more than kTau (base 2), so exp2 arguments stay <= kTau and
//    the O rescale is skipped for the whole wave in almost every tile.  The
//    true running max is tracked alongside and the state is renormalised to it
//    when written, so the stored (m, l, O) is exactly the recurrence's.
#include "internal.h"

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

template <int D>
struct Cfg {
  static constexpr int ROWB = D * 2;                  // bytes per K or V row in LDS
  static constexpr int CPR = D / 8;                   // 16-byte chunks per row
  static constexpr int TILEB = kTileKeys * ROWB;      // bytes of one K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;            // K tile then V tile
  static constexpr int RPI = 64 / CPR;                // rows per wave-wide 1 KiB load
  static constexpr int LPW = kTileKeys / RPI / 4;     // loads per wave per tile (each of K and V)
  static constexpr int DC = D / 32;                   // 32-wide d chunks (QK^T K-dim steps)
  static constexpr int DB = D / 16;                   // 16-wide d blocks of O^T
};

// Chunk swizzles (XOR on the 16-byte chunk index within a row).
template <int D>
__device__ inline int swz_k(int row) { return D == 128 ? (row & 15) : (row & 7); }
template <int D>
__device__ inline int swz_v(int row) { return D == 128 ? ((row & 7) << 1) : ((row & 3) << 1); }

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

// One 16-byte-per-lane buffer load straight into LDS (buffer_load_dwordx4 ...
// lds): lane i's bytes land at dst + 16 * i.  The host compilation pass never
// runs device code but rejects this builtin in some template contexts, so the
// call is compiled for the device only.
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t dst, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(size_t)dst, 16, voff, soff, 0, 0);
#endif
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Per-workgroup description of the query rows.
struct RowCtx {
  int f0, f1;              // flat row range [f0, f1) of this tile
  int g;                   // KV head
  int64_t qpos_min, qpos_max;
};

// Per-lane registers of the running state for the wave's 2 column blocks.
template <int D>
struct Acc {
  f32x4 o[Cfg<D>::DB][2];  // O^T[16*db + 4*(lane/16) + i][query col], relative to m2
  float m2[2];             // reference max (base 2): exp2 arguments are <= kTau
  float mt[2];             // true running max (base 2)
  float lp[2];             // per-lane partial of the denominator, relative to m2
};

// A key range as the kernels see it: buffer resources over K and V of one KV
// head, the byte stride between keys, the absolute position of key 0 and the
// number of keys.  Reads past the range return zeros (buffer range check).
struct KVSrc {
  __amdgpu_buffer_rsrc_t k, v;
  uint32_t kst, vst;       // bytes between consecutive keys
  int64_t pos0;
  int n;
};

template <int D>
__device__ inline KVSrc make_src(const Seg& s, int g) {
  KVSrc r;
  const char* kb = (const char*)s.k + (int64_t)g * s.ks_h * 2;
  const char* vb = (const char*)s.v + (int64_t)g * s.vs_h * 2;
  r.kst = (uint32_t)(s.ks_t * 2);
  r.vst = (uint32_t)(s.vs_t * 2);
  r.k = make_rsrc(kb, s.n > 0 ? (uint32_t)((s.n - 1) * (int64_t)r.kst + D * 2) : 0u);
  r.v = make_rsrc(vb, s.n > 0 ? (uint32_t)((s.n - 1) * (int64_t)r.vst + D * 2) : 0u);
  r.pos0 = s.pos0;
  r.n = s.n;
  return r;
}

// Per-lane byte offsets, within a tile, of the 16-byte chunks this lane moves:
// wave-wide load j carries RPI whole rows; lane (row r, chunk position p)
// fetches the global chunk p ^ swizzle(r), which is where the operand reads
// look for it.  They depend only on the key strides, so they are computed once
// per segment.
template <int D>
struct LaneOffs {
  uint32_t k[Cfg<D>::LPW];
  uint32_t v[Cfg<D>::LPW];
};

template <int D>
__device__ inline LaneOffs<D> lane_offsets(const KVSrc& src, int wave, int lane) {
  using C = Cfg<D>;
  LaneOffs<D> o;
  const int rsub = lane / C::CPR;
  const int p = lane % C::CPR;
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const int row = (wave * C::LPW + j) * C::RPI + rsub;
    o.k[j] = (uint32_t)row * src.kst + (uint32_t)((p ^ swz_k<D>(row)) * 16);
    o.v[j] = (uint32_t)row * src.vst + (uint32_t)((p ^ swz_v<D>(row)) * 16);
  }
  return o;
}

// Issue the HBM -> LDS loads of the 64-key tile starting at key k0 of `src`.
// Keys past the end of the range read as zeros (buffer range check); their
// scores are masked, so their P is exactly 0.
// `stage` is the LDS byte address of the stage.
template <int D>
__device__ inline void issue_tile(const KVSrc& src, const LaneOffs<D>& offs, int k0, uint32_t stage, int wave) {
  using C = Cfg<D>;
  const uint32_t soff_k = (uint32_t)k0 * src.kst;
  const uint32_t soff_v = (uint32_t)k0 * src.vst;
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const uint32_t rbase = (uint32_t)((wave * C::LPW + j) * C::RPI);
    lds_dma16(src.k, stage + rbase * C::ROWB, offs.k[j], soff_k);
    lds_dma16(src.v, stage + C::TILEB + rbase * C::ROWB, offs.v[j], soff_v);
  }
}

// One 64-key tile for one wave: S^T = K Q^T, online-softmax update, O^T += V^T P^T.
template <int D>
__device__ inline void tile_compute(const lds_char* stage, int lane, const bf16x8 (&qf)[2][Cfg<D>::DC],
                                    Acc<D>& acc, float c, bool need_mask, bool causal, int n_valid,
                                    int krel, const int (&qrel)[2]) {
  using C = Cfg<D>;
  const lds_char* kl = stage;
  const lds_char* vl = stage + C::TILEB;
  const int lr = lane & 15;
  const int lg = lane >> 4;

  f32x4 s[4][2];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int row = 16 * kb + lr;
      const bf16x8 kf = *(const lds_bf16x8*)(kl + row * C::ROWB + (((4 * dc + lg) ^ swz_k<D>(row)) * 16));
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][dc], s[kb][qb], 0, 0, 0);
    }
  }

  // s[kb][qb][i] = score of key 16*kb + 4*lg + i against query column qb of this lane.
  // Positions are relative to the tile's first query: key kk sits at krel + kk,
  // the lane's query rows at qrel[qb].
  if (need_mask) {
    // Key kk is visible to query column qb iff kk < lim[qb]; with kk = 16*kb + 4*lg + i
    // that is 16*kb + i < lim[qb] - 4*lg, one compare per score against a constant.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int lim = causal ? min(n_valid, qrel[qb] - krel + 1) : n_valid;
      const int t = lim - 4 * lg;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * kb + i >= t) s[kb][qb][i] = -INFINITY;
    }
  }

  bf16x8 pf[2][2];  // [key chunk of 32][qb]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      mx = fmaxf(mx, fmaxf(fmaxf(s[kb][qb][0], s[kb][qb][1]), fmaxf(s[kb][qb][2], s[kb][qb][3])));
    mx = wave_max_cols(mx) * c;            // tile max of this lane's row, base 2
    acc.mt[qb] = fmaxf(acc.mt[qb], mx);
    const float m_old = acc.m2[qb];
    // Move the reference only when the tile max is more than kTau above it
    // (always the case while the row has seen no key: m_old = -inf).
    const bool move = mx > m_old + kTau;
    if (__ballot(move) != 0) {
      const float m_new = move ? mx : m_old;
      const float alpha = __builtin_amdgcn_exp2f(m_old - m_new);  // 0 when m_old = -inf; 1 if unchanged
      acc.m2[qb] = m_new;
      acc.lp[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) acc.o[db][qb] *= alpha;
    }
    const float base = (acc.m2[qb] == -INFINITY) ? 0.f : acc.m2[qb];
    float p[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][i], c, -base));
    // P is rounded to bf16 once; the denominator sums exactly the values PV
    // multiplies (two per v_dot2c_f32_bf16 against (1, 1), fp32 accumulation).
    const bf16x2 ones = bf16x2{(__bf16)1.0f, (__bf16)1.0f};
    float sum = 0.f;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      bf16x2 w[4];
      w[0] = pack_bf16x2(p[2 * ch][0], p[2 * ch][1]);
      w[1] = pack_bf16x2(p[2 * ch][2], p[2 * ch][3]);
      w[2] = pack_bf16x2(p[2 * ch + 1][0], p[2 * ch + 1][1]);
      w[3] = pack_bf16x2(p[2 * ch + 1][2], p[2 * ch + 1][3]);
#pragma unroll
      for (int u = 0; u < 4; ++u) sum = __builtin_amdgcn_fdot2_f32_bf16(w[u], ones, sum, false);
      pf[ch][qb] = __builtin_bit_cast(bf16x8, w);
    }
    acc.lp[qb] += sum;
  }

  // O^T[d][q] += sum_key V^T[d][key] P^T[key][q].  MFMA k-slot 8*lg + i of key chunk ch
  // is key 32*ch + 4*lg + i (i < 4) or 32*ch + 16 + 4*lg + (i - 4) (i >= 4) -- the
  // layout pf was packed in.  A transposing read hands lane j of a 16-lane group
  // element j%4 of the 8-byte pieces addressed by lanes j/4 + 4i (i = 0..3); lane a
  // addresses row key0 + a/4, columns 16*db + 4*(a%4) .. +3, so lane (lg, lr) gets
  // keys key0 + {0..3} at d = 16*db + lr.
#pragma unroll
  for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int row0 = 32 * ch + 4 * lg + (lr >> 2);
      const int row1 = row0 + 16;
      const int cidx = 2 * db + ((lr & 3) >> 1);
      const int half = (lr & 1) * 8;
      const lds_char* a0 = vl + row0 * C::ROWB + ((cidx ^ swz_v<D>(row0)) * 16) + half;
      const lds_char* a1 = vl + row1 * C::ROWB + ((cidx ^ swz_v<D>(row1)) * 16) + half;
      const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a0);
      const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a1);
      const s16x8 xx = s16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      const bf16x8 vf = __builtin_bit_cast(bf16x8, xx);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        acc.o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[ch][qb], acc.o[db][qb], 0, 0, 0);
    }
  }
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
  int64_t srow[2];   // state row t*Hq + h
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
    lr.srow[qb] = (int64_t)t * qs.Hq + h;
    lr.qptr[qb] = (const uint16_t*)qs.q + (int64_t)t * qs.qs_t + (int64_t)h * qs.qs_h;
  }
  return lr;
}

template <int D>
__device__ inline void load_q(const LaneRows& lr, int lane, bf16x8 (&qf)[2][Cfg<D>::DC]) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int dc = 0; dc < Cfg<D>::DC; ++dc)
      qf[qb][dc] = *(const bf16x8*)(lr.qptr[qb] + 32 * dc + 8 * (lane >> 4));
}

template <int D>
__device__ inline void init_acc(Acc<D>& acc) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    acc.m2[qb] = -INFINITY;
    acc.mt[qb] = -INFINITY;
    acc.lp[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < Cfg<D>::DB; ++db) acc.o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

template <int D>
__device__ inline void load_acc(Acc<D>& acc, const LaneRows& lr, int lane, const float* m, const float* l,
                                const float* o) {
  const int lg = lane >> 4;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int64_t r = lr.srow[qb];
    float mm = m[r];
    acc.m2[qb] = (mm == -INFINITY) ? -INFINITY : mm * kLog2e;
    acc.mt[qb] = acc.m2[qb];
    acc.lp[qb] = (lg == 0) ? l[r] : 0.f;
#pragma unroll
    for (int db = 0; db < Cfg<D>::DB; ++db)
      acc.o[db][qb] = *(const f32x4*)(o + r * D + 16 * db + 4 * lg);
  }
}

// Renormalise to the true running max and write the state of valid rows.
template <int D>
__device__ inline void store_acc(Acc<D>& acc, const LaneRows& lr, int lane, float* m, float* l, float* o,
                                 int64_t row_base) {
  const int lg = lane >> 4;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float mt = acc.mt[qb];
    const float ref = acc.m2[qb];
    const float f = (mt == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(ref - mt);
    const float lt = wave_sum_cols(acc.lp[qb]) * f;
    if (!lr.valid[qb]) continue;
    const int64_t r = row_base + lr.srow[qb];
    if (lg == 0) {
      m[r] = (mt == -INFINITY) ? -INFINITY : mt * kLn2;
      l[r] = lt;
    }
#pragma unroll
    for (int db = 0; db < Cfg<D>::DB; ++db) *(f32x4*)(o + r * D + 16 * db + 4 * lg) = acc.o[db][qb] * f;
  }
}

__device__ inline void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The key-tile loop over a list of segments, double-buffered through LDS: the
// next tile loads while the current one is multiplied.  One barrier per tile:
// after it, every wave's loads of the tile about to be used have landed and
// every wave is done with the stage the next load overwrites.  The loop is
// unrolled by two so each stage's LDS offsets are compile-time constants.
// Segment bookkeeping (visible key count, buffer resources, per-lane offsets)
// runs only when a cursor crosses into another segment.
template <int D, class GetSeg>
__device__ inline void run_segments(const QSide& qs, const RowCtx& rc, const LaneRows& lr, int n_seg,
                                    GetSeg get_seg, const bf16x8 (&qf)[2][Cfg<D>::DC], Acc<D>& acc,
                                    lds_char* lds, bool wave_active) {
  using C = Cfg<D>;
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
  KVSrc isrc = make_src<D>(get_seg(is), rc.g);
  LaneOffs<D> ilo = lane_offsets<D>(isrc, wave, lane);
  // compute cursor
  int cs = is, ck = 0, cn = is_n;
  int64_t cpos0 = get_seg(cs).pos0;

  const uint32_t lds_addr = (uint32_t)(size_t)lds;
  auto issue_next = [&](int stage_off) {
    issue_tile<D>(isrc, ilo, ik, lds_addr + (uint32_t)stage_off, wave);
    ik += kTileKeys;
    if (ik >= is_n) {
      is = next_nonempty(is + 1, is_n);
      ik = 0;
      if (is < n_seg) {
        isrc = make_src<D>(get_seg(is), rc.g);
        ilo = lane_offsets<D>(isrc, wave, lane);
      }
    }
  };

  // One tile: wait for it, let the next one start loading, multiply.
  auto step = [&](int cur_off, int nxt_off) {
    wait_all_loads();
    __syncthreads();
    if (is < n_seg) issue_next(nxt_off);
    if (wave_active) {
      const int n_valid = min(kTileKeys, cn - ck);
      const int64_t kpos0 = cpos0 + ck;
      const bool need_mask = (n_valid < kTileKeys) || (qs.causal && kpos0 + kTileKeys - 1 > rc.qpos_min);
      // Visited keys satisfy kpos0 <= qpos_max, so the offset fits easily in 32 bits
      // whenever a mask is needed; far-past tiles are clamped (never masked).
      const int64_t krel64 = kpos0 - rc.qpos_min;
      const int krel = (int)max((int64_t)-(1 << 30), min((int64_t)(1 << 30), krel64));
      tile_compute<D>(lds + cur_off, lane, qf, acc, qs.c, need_mask, qs.causal != 0, n_valid, krel, lr.qrel);
    }
    ck += kTileKeys;
    if (ck >= cn) {
      cs = next_nonempty(cs + 1, cn);
      ck = 0;
      if (cs < n_seg) cpos0 = get_seg(cs).pos0;
    }
  };

  issue_next(0);
  while (true) {
    step(0, C::STAGEB);
    if (cs >= n_seg) break;
    step(C::STAGEB, 0);
    if (cs >= n_seg) break;
  }
  // Leave no load in flight into LDS that a later phase might reuse.
  wait_all_loads();
}

__device__ inline RowCtx make_rowctx(const QSide& qs, int f0, int f1, int g) {
  RowCtx rc;
  rc.f0 = f0;
  rc.f1 = f1;
  rc.g = g;
  rc.qpos_min = qs.q_pos0 + f0 / qs.G;
  rc.qpos_max = qs.q_pos0 + (f1 - 1) / qs.G;
  return rc;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void walk_kernel(WalkArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * Cfg<D>::STAGEB];
  const int Hkv = a.qs.Hkv;
  const int g = blockIdx.x % Hkv;          // consecutive workgroups land on different XCDs;
  const int n_tiles = (a.qs.q_len * a.qs.G + kTileRows - 1) / kTileRows;
  const int tile = n_tiles - 1 - (int)(blockIdx.x / Hkv);  // causal: longest rows first
  const int total = a.qs.q_len * a.qs.G;
  const int f0 = tile * kTileRows;
  const int f1 = min(f0 + kTileRows, total);
  const RowCtx rc = make_rowctx(a.qs, f0, f1, g);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const LaneRows lr = lane_rows(a.qs, rc, wave, lane);
  const bool wave_active = f0 + wave * 32 < f1;

  bf16x8 qf[2][Cfg<D>::DC];
  load_q<D>(lr, lane, qf);
  Acc<D> acc;
  if (a.reset)
    init_acc<D>(acc);
  else
    load_acc<D>(acc, lr, lane, a.m, a.l, a.o);

  run_segments<D>(a.qs, rc, lr, a.n_seg, [&](int i) -> const Seg& { return a.seg[i]; }, qf, acc,
                     (lds_char*)lds, wave_active);
  store_acc<D>(acc, lane_rows(a.qs, rc, wave, lane), lane, a.m, a.l, a.o, 0);
}

// Chunk `chunk` of the segment table as a segment of its own.
__device__ inline Seg chunk_seg(const Seg* seg, int n_seg, const int32_t* chunk_begin, int chunk_len, int chunk) {
  int s_i = 0;
  while (s_i + 1 < n_seg && chunk_begin[s_i + 1] <= chunk) ++s_i;
  const Seg& base = seg[s_i];
  const int k_off = (chunk - chunk_begin[s_i]) * chunk_len;
  Seg cs = base;
  cs.k = (const uint16_t*)base.k + (int64_t)k_off * base.ks_t;
  cs.v = (const uint16_t*)base.v + (int64_t)k_off * base.vs_t;
  cs.pos0 = base.pos0 + k_off;
  cs.n = min(chunk_len, base.n - k_off);
  return cs;
}

// Partial state of one row tile over one key range, written to a workspace slot.
template <int D>
__device__ inline void partial_job(const QSide& qs, int f0, int f1, int g, const Seg& sg, float* ws_m,
                                   float* ws_l, float* ws_o, int64_t row_base, lds_char* lds) {
  const RowCtx rc = make_rowctx(qs, f0, f1, g);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const LaneRows lr = lane_rows(qs, rc, wave, lane);
  const bool wave_active = f0 + wave * 32 < f1;
  bf16x8 qf[2][Cfg<D>::DC];
  load_q<D>(lr, lane, qf);
  Acc<D> acc;
  init_acc<D>(acc);
  run_segments<D>(qs, rc, lr, 1, [&](int) -> const Seg& { return sg; }, qf, acc, lds, wave_active);
  store_acc<D>(acc, lane_rows(qs, rc, wave, lane), lane, ws_m, ws_l, ws_o, row_base);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void split_kernel(SplitArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * Cfg<D>::STAGEB];
  const int Hkv = a.qs.Hkv;
  const int g = blockIdx.x % Hkv;
  const int tile = blockIdx.x / Hkv;
  const int chunk = blockIdx.y;
  const int total = a.qs.q_len * a.qs.G;
  const int f0 = tile * kTileRows;
  const int f1 = min(f0 + kTileRows, total);
  const Seg cs = chunk_seg(a.seg, a.n_seg, a.chunk_begin, a.chunk_len, chunk);
  partial_job<D>(a.qs, f0, f1, g, cs, a.ws_m, a.ws_l, a.ws_o, (int64_t)chunk * a.R, (lds_char*)lds);
}

// Shared-prefix fan-out (decode, or prefill of the private suffixes), one
// launch for both job kinds ("AHBM Agentic Runtime Architecture" s.3.2-3.4,
// s.3.6): jobs [0, n_prefix_jobs) are (row tile,
// KV head, prefix chunk) -- every branch's rows of a KV head against one chunk
// of the shared prefix, written to slot `chunk`; the remaining jobs are
// (branch group or branch row tile, KV head) -- each branch's rows against its
// private suffix under the causal rule, written to slot `suffix_slot`.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void fanout_kernel(FanoutArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * Cfg<D>::STAGEB];
  const int Hkv = a.qs.Hkv;
  const int G = a.qs.G;
  const int total = a.qs.q_len * G;
  const int xs = a.row_tiles * Hkv;
  const int n_prefix_jobs = xs * a.n_chunks;
  const int id = blockIdx.x;
  if (id < n_prefix_jobs) {
    const int x = id % xs;
    const int chunk = id / xs;
    const int g = x % Hkv;
    const int f0 = (x / Hkv) * kTileRows;
    const int f1 = min(f0 + kTileRows, total);
    const int k_off = chunk * a.chunk_len;
    Seg sg = a.prefix;
    sg.k = (const uint16_t*)sg.k + (int64_t)k_off * sg.ks_t;
    sg.v = (const uint16_t*)sg.v + (int64_t)k_off * sg.vs_t;
    sg.pos0 = k_off;
    sg.n = min(a.chunk_len, a.prefix.n - k_off);
    partial_job<D>(a.qs, f0, f1, g, sg, a.ws_m, a.ws_l, a.ws_o, (int64_t)chunk * a.R, (lds_char*)lds);
    return;
  }
  const int j = id - n_prefix_jobs;
  const int g = j % Hkv;
  const int u = j / Hkv;
  const int TG = a.T * G;
  int b0, b1, rt;
  if (a.srt == 1) {
    b0 = u * a.bpj;
    b1 = min(b0 + a.bpj, a.qs.q_len / a.T);
    rt = 0;
  } else {
    b0 = u / a.srt;
    b1 = b0 + 1;
    rt = u % a.srt;
  }
  const int64_t tok = (int64_t)Hkv * D;
  for (int b = b0; b < b1; ++b) {
    if (b > b0) __syncthreads();  // every wave is done with the previous branch's LDS tiles
    Seg sg;
    sg.k = (const uint16_t*)a.sk + (int64_t)b * a.S * tok;
    sg.v = (const uint16_t*)a.sv + (int64_t)b * a.S * tok;
    sg.ks_t = tok;
    sg.vs_t = tok;
    sg.ks_h = D;
    sg.vs_h = D;
    sg.pos0 = 0;
    sg.n = a.S;
    sg.pad_ = 0;
    // Suffix positions: key j at j, branch b's new token i (query token b*T + i)
    // at S - T + i.
    QSide qs = a.qs;
    qs.causal = 1;
    qs.q_pos0 = (int64_t)(a.S - a.T) - (int64_t)b * a.T;
    const int f0 = b * TG + rt * kTileRows;
    const int f1 = min(f0 + kTileRows, (b + 1) * TG);
    partial_job<D>(qs, f0, f1, g, sg, a.ws_m, a.ws_l, a.ws_o, (int64_t)a.suffix_slot * a.R, (lds_char*)lds);
  }
}

}  // namespace

hipError_t launch_walk_bf16(const WalkArgs& a, int D, hipStream_t s) {
  const int tiles = (a.qs.q_len * a.qs.G + kTileRows - 1) / kTileRows;
  dim3 grid(tiles * a.qs.Hkv);
  if (D == 128)
    hipLaunchKernelGGL(walk_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(walk_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split_bf16(const SplitArgs& a, int n_chunks, int D, hipStream_t s) {
  const int tiles = (a.qs.q_len * a.qs.G + kTileRows - 1) / kTileRows;
  dim3 grid(tiles * a.qs.Hkv, n_chunks);
  if (D == 128)
    hipLaunchKernelGGL((split_kernel<128>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((split_kernel<64>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fanout_bf16(const FanoutArgs& a, int n_jobs, int D, hipStream_t s) {
  dim3 grid(n_jobs);
  if (D == 128)
    hipLaunchKernelGGL((fanout_kernel<128>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((fanout_kernel<64>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
