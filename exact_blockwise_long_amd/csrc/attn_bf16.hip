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
//  * A workgroup owns a tile of "flat rows" (query token x member of one GQA
//    group) that all read the same KV head, so one K/V tile in LDS serves
//    every query head of the group ("AHBM Agentic Runtime Architecture"
//    s.1.3: rows batched against shared KV).  The split and fan-out kernels
//    use 4 waves and 128 rows (two workgroups per compute unit); the walk
//    uses 8 waves and 256 rows (one per compute unit), so each K/V byte
//    staged from L2 into LDS serves twice the rows.
//  * K/V tiles of 64 keys (128 in the walk) go HBM -> LDS with
//    buffer_load_dwordx4 ... lds (no register staging), double-buffered: the
//    next tile's loads are in flight while the current one is multiplied (two
//    LDS stages of 32 KiB per workgroup, 64 KiB in the walk).  16-byte chunks of every LDS row are XOR-swizzled by row so
//    both operand reads below are bank-conflict free.
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
#include "bf16_tiles.h"

namespace ba {
namespace {

// Per-lane registers of the running state for the wave's 2 column blocks.
template <int D>
struct Acc {
  f32x4 o[Cfg<D>::DB][2];  // O^T[16*db + 4*(lane/16) + i][query col], relative to m2
  float m2[2];             // reference max (base 2): exp2 arguments are <= kTau
  float mt[2];             // true running max (base 2)
  float lp[2];             // per-lane partial of the denominator, relative to m2
};

// One tile of TK keys (64 or 128) for one wave: S^T = K Q^T, online-softmax
// update, O^T += V^T P^T.
template <int D, int TK = kTileKeys>
__device__ inline void tile_compute(const lds_char* stage, int lane, const bf16x8 (&qf)[2][Cfg<D>::DC],
                                    Acc<D>& acc, float c, bool need_mask, bool causal, int n_valid,
                                    int krel, const int (&qrel)[2]) {
  using C = Cfg<D, 4, TK>;
  constexpr int NKB = TK / 16;
  constexpr int NCH = TK / 32;
  const lds_char* kl = stage;
  const lds_char* vl = v_tile_of<D, TK>(stage);
  const int lr = lane & 15;
  const int lg = lane >> 4;

  f32x4 s[NKB][2];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int row = 16 * kb + lr;
      const bf16x8 kf = *(const lds_bf16x8*)(kl + row * C::ROWB + (((4 * dc + lg) ^ swz<D>(row)) * 16));
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
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * kb + i >= t) s[kb][qb][i] = -INFINITY;
    }
  }

  bf16x8 pf[NCH][2];  // [key chunk of 32][qb]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    // Two chains of three-operand maxima (v_max3_f32): 2 instructions per 4 scores.
    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      m0 = fmaxf(fmaxf(m0, s[kb][qb][0]), s[kb][qb][1]);
      m1 = fmaxf(fmaxf(m1, s[kb][qb][2]), s[kb][qb][3]);
    }
    float mx = wave_max_cols(fmaxf(m0, m1)) * c;   // tile max of this lane's row, base 2
    acc.mt[qb] = fmaxf(acc.mt[qb], mx);
    const float m_old = acc.m2[qb];
    // Move the reference only when the tile max is more than kTau above it
    // (always the case when a row sees its first key: m_old = -inf, mx finite).
    // A row that does not move keeps alpha = 1 exactly -- also a row that has
    // seen no key yet and sees none in this tile either (m_old = mx = -inf,
    // where exp2(m_old - m_old) would be NaN) while another row of the wave
    // moves.
    const bool move = mx > m_old + kTau;
    if (__ballot(move) != 0) {
      const float m_new = move ? mx : m_old;
      const float alpha = move ? __builtin_amdgcn_exp2f(m_old - m_new) : 1.f;  // 0 when m_old = -inf
      acc.m2[qb] = m_new;
      acc.lp[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) acc.o[db][qb] *= alpha;
    }
    const float base = (acc.m2[qb] == -INFINITY) ? 0.f : acc.m2[qb];
    float p[NKB][4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][i], c, -base));
    // P is rounded to bf16 once; the denominator sums exactly the values PV
    // multiplies (two per v_dot2c_f32_bf16 against (1, 1), fp32 accumulation).
    const bf16x2 ones = bf16x2{(__bf16)1.0f, (__bf16)1.0f};
    float sum = 0.f;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
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
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int row0 = 32 * ch + 4 * lg + (lr >> 2);
      const int row1 = row0 + 16;
      const int cidx = 2 * db + ((lr & 3) >> 1);
      const int half = (lr & 1) * 8;
      const lds_char* a0 = vl + row0 * C::ROWB + ((cidx ^ swz<D>(row0)) * 16) + half;
      const lds_char* a1 = vl + row1 * C::ROWB + ((cidx ^ swz<D>(row1)) * 16) + half;
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

// Finalise instead of writing the state ("RingAttention and Context
// Parallelism", sections 2 and 7): A = O / l and LSE = m + ln l of valid rows.
// O and the lane partial sums of l are both relative to the reference max m2
// (base 2), so A = O / sum(lp) and LSE = m2 ln 2 + ln sum(lp); a row that saw
// no key (sum 0) gets A = 0 and LSE = -inf.
template <int D>
__device__ inline void store_final(const Acc<D>& acc, const LaneRows& lr, int lane, void* out, bool out_bf16,
                                   int64_t stride, float* lse) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const int lg = lane >> 4;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lsum = wave_sum_cols(acc.lp[qb]);
    if (!lr.valid[qb]) continue;
    const int64_t r = lr.srow[qb];
    const bool empty = !(lsum > 0.f);
    const float inv = empty ? 0.f : 1.f / lsum;
#pragma unroll
    for (int db = 0; db < Cfg<D>::DB; ++db) {
      const f32x4 v = acc.o[db][qb] * inv;
      const int64_t at = r * stride + 16 * db + 4 * lg;
      if (out_bf16)
        *(bf16x4*)((__bf16*)out + at) = __builtin_convertvector(v, bf16x4);
      else
        *(f32x4*)((float*)out + at) = v;
    }
    if (lse && lg == 0) lse[r] = empty ? -INFINITY : acc.m2[qb] * kLn2 + logf(lsum);
  }
}

// The walk's workgroup: 8 waves of 32 rows.  Against 4 waves of 32 rows at
// two workgroups per compute unit (the same waves per SIMD and registers per
// wave), it moves half the K/V bytes from L2 into LDS per multiply; on the
// power-limited board that made the 32K causal prefill 5 % faster.
constexpr int kWalkWaves = 8;
constexpr int kWalkRows = 32 * kWalkWaves;

// The walk's key tile: 128 keys, two 64 KiB stages (the one workgroup per
// compute unit leaves the LDS for it).  Against 64-key tiles the softmax's
// per-tile work (row max, cross-lane steps, rescale test) and the barrier
// come half as often per key: 1.3 % on the 32K causal prefill, at 251 VGPRs.
constexpr int kWalkKeys = 128;

template <int D>
__global__ __launch_bounds__(64 * kWalkWaves, 1) void walk_kernel(WalkArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * Cfg<D, kWalkWaves, kWalkKeys>::STAGEB];
  // Consecutive workgroups take the KV heads (each XCD keeps one head's K/V in
  // its L2), then the sequences, then the row tiles, longest first.
  const int Hkv = a.qs.Hkv;
  const int g = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int b = rest % a.qs.B;
  const int n_tiles = (a.qs.q_len * a.qs.G + kWalkRows - 1) / kWalkRows;
  const int tile = n_tiles - 1 - rest / a.qs.B;
  const int total = a.qs.q_len * a.qs.G;
  const int f0 = tile * kWalkRows;
  const int f1 = min(f0 + kWalkRows, total);
  const RowCtx rc = make_rowctx(a.qs, f0, f1, g, b);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const LaneRows lr = lane_rows(a.qs, rc, wave, lane);
  const bool wave_active = f0 + wave * 32 < f1;

  bf16x8 qf[2][Cfg<D>::DC];
  load_q<D>(lr, lane, qf);
  Acc<D> acc;
  if (a.reset)
    init_acc<D>(acc);
  else
    load_acc<D>(acc, lr, lane, a.m, a.l, a.o);

  const QSide& qs = a.qs;
  run_segments<D, kCacheReuse, kWalkWaves, kWalkKeys>(
      qs, rc, a.n_seg, [&](int i) -> const Seg& { return a.seg[i]; },
      [&](const lds_char* stage, bool need_mask, int n_valid, int krel) {
        tile_compute<D, kWalkKeys>(stage, lane, qf, acc, qs.c, need_mask, qs.causal != 0, n_valid, krel, lr.qrel);
      },
      (lds_char*)lds, wave_active);
  if (a.fin_out)
    store_final<D>(acc, lane_rows(a.qs, rc, wave, lane), lane, a.fin_out, a.fin_bf16 != 0, a.fin_stride, a.fin_lse);
  else
    store_acc<D>(acc, lane_rows(a.qs, rc, wave, lane), lane, a.m, a.l, a.o, 0);
}

// The query side of a job: its rows' bookkeeping and Q fragments.  The Q
// loads are issued here and waited for only at the first product, so a job
// that must load something else first (a page table) issues both together.
template <int D>
struct JobQ {
  RowCtx rc;
  LaneRows lr;
  bool wave_active;
  bf16x8 qf[2][Cfg<D>::DC];
};

template <int D>
__device__ inline JobQ<D> job_q(const QSide& qs, int f0, int f1, int g, int b) {
  JobQ<D> j;
  j.rc = make_rowctx(qs, f0, f1, g, b);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  j.lr = lane_rows(qs, j.rc, wave, lane);
  j.wave_active = f0 + wave * 32 < f1;
  load_q<D>(j.lr, lane, j.qf);
  return j;
}

// Partial state of a job's rows over the keys of n_seg segments (get_seg(i)
// returns segment i), written to a workspace slot.
template <int D, int kAux, int W, int TK, class GetSeg>
__device__ inline void job_walk(const QSide& qs, const JobQ<D>& j, int n_seg, GetSeg get_seg, float* ws_m,
                                float* ws_l, float* ws_o, int64_t row_base, lds_char* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Acc<D> acc;
  init_acc<D>(acc);
  run_segments<D, kAux, W, TK>(
      qs, j.rc, n_seg, get_seg,
      [&](const lds_char* stage, bool need_mask, int n_valid, int krel) {
        tile_compute<D, TK>(stage, lane, j.qf, acc, qs.c, need_mask, qs.causal != 0, n_valid, krel, j.lr.qrel);
      },
      lds, j.wave_active);
  store_acc<D>(acc, lane_rows(qs, j.rc, wave, lane), lane, ws_m, ws_l, ws_o, row_base);
}

template <int D, int kAux, int W = 4, int TK = kTileKeys, class GetSeg>
__device__ inline void partial_job_segs(const QSide& qs, int f0, int f1, int g, int b, int n_seg, GetSeg get_seg,
                                        float* ws_m, float* ws_l, float* ws_o, int64_t row_base, lds_char* lds) {
  job_walk<D, kAux, W, TK>(qs, job_q<D>(qs, f0, f1, g, b), n_seg, get_seg, ws_m, ws_l, ws_o, row_base, lds);
}

template <int D, int kAux, int W = 4, int TK = kTileKeys>
__device__ inline void partial_job(const QSide& qs, int f0, int f1, int g, int b, const Seg& sg, float* ws_m,
                                   float* ws_l, float* ws_o, int64_t row_base, lds_char* lds) {
  partial_job_segs<D, kAux, W, TK>(qs, f0, f1, g, b, 1, [&](int) -> const Seg& { return sg; }, ws_m, ws_l, ws_o,
                                   row_base, lds);
}

// The page ids of one job's key range [k0, k1) of a paged sequence whose
// page p is pool page ids[p] ("AHBM Agentic Runtime Architecture" s.3.1: a
// branch's page table).  Lane i loads the id of the range's i-th page when
// the job starts, so the key walk reads ids from registers (v_readlane) and
// never waits on memory at a page boundary; a range of more than 64 pages
// reads the rest from memory.
struct PageIds {
  const int32_t* ids;
  int first;     // page of key k0
  int lane_id;   // this lane's page id (lane < 64 pages of the range)
};

__device__ inline int paged_segments(int k0, int k1, int page_len) {
  return k1 > k0 ? (k1 - 1) / page_len - k0 / page_len + 1 : 0;
}

__device__ inline PageIds load_page_ids(const int32_t* ids, int k0, int k1, int page_len) {
  PageIds pi;
  pi.ids = ids;
  pi.first = k0 / page_len;
  const int lane = threadIdx.x & 63;
  pi.lane_id = lane < paged_segments(k0, k1, page_len) ? ids[pi.first + lane] : -1;
  return pi;
}

// Whether any page id of the range [k0, k1) is corrupt: neither a page of
// the pool nor the hole marker -1.  Uniform over the workgroup.
__device__ inline bool pages_corrupt(const PageIds& pi, int k0, int k1, int page_len, int n_pool) {
  const int n = paged_segments(k0, k1, page_len);
  const int lane = threadIdx.x & 63;
  const bool bad = lane < n && (pi.lane_id < -1 || pi.lane_id >= n_pool);
  bool any = __ballot(bad) != 0;
  for (int i = 64; i < n && !any; ++i) {
    const int id = pi.ids[pi.first + i];
    any = id < -1 || id >= n_pool;
  }
  return __builtin_amdgcn_readfirstlane((int)any) != 0;
}

// The partial state that marks rows whose keys could not be read (a corrupt
// page id): m = +inf, l = 1, O = NaN.  The log-sum-exp merge keeps it (every
// other part gets weight exp(m_s - inf) = 0), so the finalised rows come out
// as NaN with LSE +inf instead of a plausible result over a wrong key set.
template <int D, int W>
__device__ inline void store_corrupt(const QSide& qs, int f0, int f1, int g, float* ws_m, float* ws_l, float* ws_o,
                                     int64_t row_base) {
  const RowCtx rc = make_rowctx(qs, f0, f1, g, 0);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const LaneRows lr = lane_rows(qs, rc, wave, lane);
  const int lg = lane >> 4;
  const float nan = __builtin_bit_cast(float, 0x7FC00000u);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!lr.valid[qb] || f0 + wave * 32 >= f1) continue;
    const int64_t r = row_base + lr.srow[qb];
    if (lg == 0) {
      ws_m[r] = INFINITY;
      ws_l[r] = 1.f;
    }
#pragma unroll
    for (int db = 0; db < Cfg<D>::DB; ++db) *(f32x4*)(ws_o + r * D + 16 * db + 4 * lg) = f32x4{nan, nan, nan, nan};
  }
}

// Segment i of the range: the piece of page first + i inside [k0, k1), at
// positions pos_base + key.  A page id of -1 (a hole) gives an empty segment:
// its keys are left out and nothing is read.
template <int D>
__device__ inline Seg paged_seg(const FanoutArgs& a, const PageIds& pi, int k0, int k1, int i, int64_t pos_base) {
  const int PL = a.page_len;
  const int p = pi.first + i;
  const int s0 = max(k0, p * PL);
  const int s1 = min(k1, (p + 1) * PL);
  const int id = i < 64 ? __builtin_amdgcn_readlane(pi.lane_id, i) : pi.ids[p];
  const bool ok = id >= 0 && id < a.n_pool_pages;
  const int64_t tok = (int64_t)a.qs.Hkv * D;
  const int64_t off = ok ? ((int64_t)id * PL + (s0 - p * PL)) * tok : 0;
  Seg sg;
  sg.k = (const uint16_t*)a.prefix.k + off;
  sg.v = (const uint16_t*)a.prefix.v + off;
  sg.ks_t = tok;
  sg.vs_t = tok;
  sg.ks_h = D;
  sg.vs_h = D;
  sg.pos0 = pos_base + s0;
  sg.n = ok ? s1 - s0 : 0;
  sg.ks_b = 0;
  sg.vs_b = 0;
  sg.pad_ = 0;
  return sg;
}

// kWide: 8-wave workgroups of 256-row tiles (more than one 128-row tile per
// KV head), otherwise 4 waves and 128-row tiles.
template <int D, int kAux, bool kWide>
__global__ __launch_bounds__(kWide ? 2 * kThreads : kThreads, kWide ? 1 : 2) void split_kernel(SplitArgs a) {
  constexpr int W = kWide ? 8 : 4;
  constexpr int TR = 32 * W;
  constexpr int TK = kWide ? 128 : kTileKeys;   // one workgroup per compute unit has the LDS for it
  __shared__ __attribute__((aligned(16))) char lds[2 * Cfg<D, W, TK>::STAGEB];
  const int Hkv = a.qs.Hkv;
  const int g = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int b = rest % a.qs.B;
  const int tile = rest / a.qs.B;
  const int chunk = blockIdx.y;
  const int total = a.qs.q_len * a.qs.G;
  const int f0 = tile * TR;
  const int f1 = min(f0 + TR, total);
  const Seg cs = chunk_seg<uint16_t>(a.seg, a.n_seg, a.chunk_begin, a.chunk_len, chunk);
  partial_job<D, kAux, W, TK>(a.qs, f0, f1, g, b, cs, a.ws_m, a.ws_l, a.ws_o, (int64_t)chunk * a.R, (lds_char*)lds);
}

// Shared-prefix fan-out (decode, or prefill of the private suffixes), one
// launch for both job kinds ("AHBM Agentic Runtime Architecture" s.3.2-3.4,
// s.3.6): jobs [0, n_prefix_jobs) are (row tile,
// KV head, prefix chunk) -- every branch's rows of a KV head against one chunk
// of the shared prefix, written to slot `chunk`; the remaining jobs are
// (branch group or branch row tile, KV head) -- each branch's rows against its
// private suffix under the causal rule, written to slot `suffix_slot`.
//
// kWide: 8-wave workgroups of 256-row tiles, one per compute unit, as in the
// walk (for launches with more than one 128-row tile per KV head, which the
// matrix cores bound); otherwise 4 waves and 128-row tiles.
//
// TKP: the prefix jobs' key tile.  Wide launches take the walk's 128-key
// tiles (that workgroup per compute unit has the LDS for them) when the prefix
// is contiguous or its pages are multiples of 128 keys, 64 otherwise: a paged
// walk then visits exactly the contiguous walk's tiles (chunks start at
// multiples of 128 keys) and gives its result bit for bit.  Suffix jobs take
// 64-key tiles.
template <int D, int kAux, bool kWide, int TKP = kTileKeys>
__global__ __launch_bounds__(kWide ? 2 * kThreads : kThreads, kWide ? 1 : 2) void fanout_kernel(FanoutArgs a) {
  constexpr int W = kWide ? 8 : 4;
  constexpr int TR = 32 * W;   // rows of a row tile
  static_assert(TKP == kTileKeys || kWide, "128-key tiles need the LDS of one workgroup per compute unit");
  __shared__ __attribute__((aligned(16))) char lds[2 * Cfg<D, W, TKP>::STAGEB];
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
    const int f0 = (x / Hkv) * TR;
    const int f1 = min(f0 + TR, total);
    const int k_off = chunk * a.chunk_len;
    const int k_end = min(k_off + a.chunk_len, a.prefix.n);
    if (a.prefix_pages) {
      const PageIds pi = load_page_ids(a.prefix_pages, k_off, k_end, a.page_len);
      const JobQ<D> jq = job_q<D>(a.qs, f0, f1, g, 0);   // Q loads in flight with the page ids
      if (pages_corrupt(pi, k_off, k_end, a.page_len, a.n_pool_pages)) {
        store_corrupt<D, W>(a.qs, f0, f1, g, a.ws_m, a.ws_l, a.ws_o, (int64_t)chunk * a.R);
        return;
      }
      job_walk<D, kAux, W, TKP>(a.qs, jq, paged_segments(k_off, k_end, a.page_len),
                                [&](int i) { return paged_seg<D>(a, pi, k_off, k_end, i, 0); }, a.ws_m, a.ws_l,
                                a.ws_o, (int64_t)chunk * a.R, (lds_char*)lds);
      return;
    }
    Seg sg = a.prefix;
    sg.k = (const uint16_t*)sg.k + (int64_t)k_off * sg.ks_t;
    sg.v = (const uint16_t*)sg.v + (int64_t)k_off * sg.vs_t;
    sg.pos0 = k_off;
    sg.n = k_end - k_off;
    partial_job<D, kAux, W, TKP>(a.qs, f0, f1, g, 0, sg, a.ws_m, a.ws_l, a.ws_o, (int64_t)chunk * a.R,
                                 (lds_char*)lds);
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
    // Suffix positions: key j at j, branch b's new token i (query token b*T + i)
    // at S - T + i.
    QSide qs = a.qs;
    qs.causal = 1;
    qs.q_pos0 = (int64_t)(a.S - a.T) - (int64_t)b * a.T;
    const int f0 = b * TG + rt * TR;
    const int f1 = min(f0 + TR, (b + 1) * TG);
    if (a.suffix_pages) {
      const PageIds pi = load_page_ids(a.suffix_pages + (int64_t)b * a.suffix_pages_per_branch, 0, a.S, a.page_len);
      const JobQ<D> jq = job_q<D>(qs, f0, f1, g, 0);   // Q loads in flight with the page ids
      if (pages_corrupt(pi, 0, a.S, a.page_len, a.n_pool_pages)) {
        store_corrupt<D, W>(qs, f0, f1, g, a.ws_m, a.ws_l, a.ws_o, (int64_t)a.suffix_slot * a.R);
        continue;
      }
      job_walk<D, kAux, W, kTileKeys>(qs, jq, paged_segments(0, a.S, a.page_len),
                                      [&](int i) { return paged_seg<D>(a, pi, 0, a.S, i, 0); }, a.ws_m, a.ws_l,
                                      a.ws_o, (int64_t)a.suffix_slot * a.R, (lds_char*)lds);
      continue;
    }
    Seg sg;
    sg.k = (const uint16_t*)a.sk + (int64_t)b * a.S * tok;
    sg.v = (const uint16_t*)a.sv + (int64_t)b * a.S * tok;
    sg.ks_t = tok;
    sg.vs_t = tok;
    sg.ks_h = D;
    sg.vs_h = D;
    sg.pos0 = 0;
    sg.n = a.S;
    sg.ks_b = 0;
    sg.vs_b = 0;
    sg.pad_ = 0;
    partial_job<D, kAux, W>(qs, f0, f1, g, 0, sg, a.ws_m, a.ws_l, a.ws_o, (int64_t)a.suffix_slot * a.R,
                            (lds_char*)lds);
  }
}

}  // namespace

hipError_t launch_walk_bf16(const WalkArgs& a, int D, hipStream_t s) {
  const int tiles = (a.qs.q_len * a.qs.G + kWalkRows - 1) / kWalkRows;
  dim3 grid(tiles * a.qs.Hkv * a.qs.B);
  if (D == 128)
    hipLaunchKernelGGL(walk_kernel<128>, grid, dim3(64 * kWalkWaves), 0, s, a);
  else
    hipLaunchKernelGGL(walk_kernel<64>, grid, dim3(64 * kWalkWaves), 0, s, a);
  return hipGetLastError();
}

template <int D>
void launch_split_d(const SplitArgs& a, dim3 grid, bool stream, hipStream_t s) {
  if (a.wide)
    hipLaunchKernelGGL((split_kernel<D, kCacheReuse, true>), grid, dim3(2 * kThreads), 0, s, a);
  else if (stream)
    hipLaunchKernelGGL((split_kernel<D, kCacheStream, false>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((split_kernel<D, kCacheReuse, false>), grid, dim3(kThreads), 0, s, a);
}

hipError_t launch_split_bf16(const SplitArgs& a, int n_chunks, int D, hipStream_t s) {
  const int tile_rows = a.wide ? kWideTileRows : kTileRows;
  const int per_head = (a.qs.q_len * a.qs.G + tile_rows - 1) / tile_rows;
  dim3 grid(per_head * a.qs.Hkv * a.qs.B, n_chunks);
  // One row tile per KV head, and no K/V shared between sequences: every K/V
  // byte is read by one workgroup.
  bool shared = false;
  for (int i = 0; i < a.n_seg && a.qs.B > 1; ++i) shared = shared || a.seg[i].ks_b == 0 || a.seg[i].vs_b == 0;
  const bool stream = per_head == 1 && !shared;
  if (D == 128)
    launch_split_d<128>(a, grid, stream, s);
  else
    launch_split_d<64>(a, grid, stream, s);
  return hipGetLastError();
}

template <int D, bool kWide>
void launch_fanout_w(const FanoutArgs& a, dim3 grid, hipStream_t s) {
  // All of a KV head's rows in one row tile (the decode): each prefix chunk
  // and each suffix is read by one workgroup.
  const bool stream = a.row_tiles == 1 && a.srt == 1;
  const dim3 block(kWide ? 2 * kThreads : kThreads);
  if (kWide && a.prefix_keys == 128) {
    if (stream)
      hipLaunchKernelGGL((fanout_kernel<D, kCacheStream, kWide, (kWide ? 128 : kTileKeys)>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((fanout_kernel<D, kCacheReuse, kWide, (kWide ? 128 : kTileKeys)>), grid, block, 0, s, a);
  } else if (stream) {
    hipLaunchKernelGGL((fanout_kernel<D, kCacheStream, kWide>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((fanout_kernel<D, kCacheReuse, kWide>), grid, block, 0, s, a);
  }
}

hipError_t launch_fanout_bf16(const FanoutArgs& a, int n_jobs, int D, hipStream_t s) {
  dim3 grid(n_jobs);
  if (D == 128) {
    if (a.wide)
      launch_fanout_w<128, true>(a, grid, s);
    else
      launch_fanout_w<128, false>(a, grid, s);
  } else {
    if (a.wide)
      launch_fanout_w<64, true>(a, grid, s);
    else
      launch_fanout_w<64, false>(a, grid, s);
  }
  return hipGetLastError();
}

}  // namespace ba
