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
//    serves 8 query heads ([AHBM] s.1.3: rows batched against shared KV).
//  * Each wave owns 32 rows.  Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_bf16: K (from LDS) is the A operand and Q (kept in
//    registers for the whole kernel) the B operand.  The S^T accumulator then
//    holds, per lane, 4 consecutive keys of one query row -- exactly the
//    B-operand layout of the second product O^T = V^T P^T, so P never leaves
//    registers.  V is staged into LDS transposed (V^T) for the A operand.
//  * Softmax statistics are per query column: every lane of a 16-lane column
//    group holds one query row, the row max needs two cross-lane exchanges,
//    and the row sum is kept as per-lane partial sums until the end.
//  * exp is computed as exp2 on v_exp_f32 with the logit scale folded into a
//    single multiply by scale*log2(e); the state's m is converted to natural
//    units at load/store.
//  * K/V tiles of 64 keys are double-buffered in LDS: the next tile's global
//    loads are in flight while the current tile is multiplied.
#include "internal.h"

namespace ba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kTileKeys = 64;

template <int D>
struct Cfg {
  static constexpr int KSTR = D + 8;           // bf16 elements per K row in LDS
  static constexpr int VSTR = kTileKeys + 4;   // bf16 elements per V^T row in LDS
  static constexpr int K_ELEMS = kTileKeys * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int DC = D / 32;            // 32-wide d chunks (QK^T K-dim steps)
  static constexpr int DB = D / 16;            // 16-wide d blocks of O^T
  static constexpr int CPK = D / 8;            // 16-byte chunks per K row
  static constexpr int K_PER_THREAD = kTileKeys * CPK / kThreads;
  static constexpr int V_ITEMS = (kTileKeys / 4) * (D / 8);   // (4 keys x 8 d) items
};

__device__ inline float wave_max_cols(float x) {
  // max over the 4 lanes that share lane % 16
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ inline float wave_sum_cols(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ inline unsigned pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a;
  __bf16 y = (__bf16)b;
  return (unsigned)__builtin_bit_cast(unsigned short, x) |
         ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
}

// The 4-key group index of a 64-key tile row of V^T is XOR-swizzled with
// (d / 8) % 16 so that both the transposing stores and the operand loads
// spread over the LDS banks.
__device__ inline int vt_col(int d, int group) { return ((group ^ ((d >> 3) & 15)) << 2); }

// Per-workgroup description of the query rows.
struct RowCtx {
  int f0, f1;              // flat row range [f0, f1) of this tile
  int g;                   // KV head
  int64_t qpos_min, qpos_max;
};

// Per-lane registers of the running state for the wave's 2 column blocks.
template <int D>
struct Acc {
  f32x4 o[Cfg<D>::DB][2];  // O^T[16*db + 4*(lane/16) + i][query col]
  float m2[2];             // running max in base-2 units (scaled logit * log2 e)
  float lp[2];             // per-lane partial of the denominator
};

template <int D>
__device__ inline void load_tile_regs(const Seg& s, int g, int k_off, int n_valid, int tid,
                                      u32x4 (&kr)[Cfg<D>::K_PER_THREAD], u32x4 (&vr)[4]) {
  using C = Cfg<D>;
  const uint16_t* kb = (const uint16_t*)s.k + (int64_t)g * s.ks_h;
  const uint16_t* vb = (const uint16_t*)s.v + (int64_t)g * s.vs_h;
#pragma unroll
  for (int i = 0; i < C::K_PER_THREAD; ++i) {
    int c = tid + i * kThreads;
    int key = c / C::CPK;
    int col = (c % C::CPK) * 8;
    int kk = min(key, n_valid - 1);
    kr[i] = *(const u32x4*)(kb + (int64_t)(k_off + kk) * s.ks_t + col);
  }
  if (tid < C::V_ITEMS) {
    int dq = tid % (D / 8);
    int kq = tid / (D / 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int kk = min(4 * kq + i, n_valid - 1);
      vr[i] = *(const u32x4*)(vb + (int64_t)(k_off + kk) * s.vs_t + dq * 8);
    }
  }
}

template <int D>
__device__ inline void store_tile_lds(uint16_t* st, int tid, const u32x4 (&kr)[Cfg<D>::K_PER_THREAD],
                                      const u32x4 (&vr)[4]) {
  using C = Cfg<D>;
  uint16_t* kl = st;
  uint16_t* vl = st + C::K_ELEMS;
#pragma unroll
  for (int i = 0; i < C::K_PER_THREAD; ++i) {
    int c = tid + i * kThreads;
    int key = c / C::CPK;
    int col = (c % C::CPK) * 8;
    *(u32x4*)(kl + key * C::KSTR + col) = kr[i];
  }
  if (tid < C::V_ITEMS) {
    int dq = tid % (D / 8);
    int kq = tid / (D / 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // dword w of each loaded row holds d = 8*dq + 2w (low half) and 8*dq + 2w + 1 (high half)
      unsigned lo01 = (vr[0][w] & 0xffffu) | (vr[1][w] << 16);
      unsigned lo23 = (vr[2][w] & 0xffffu) | (vr[3][w] << 16);
      unsigned hi01 = (vr[0][w] >> 16) | (vr[1][w] & 0xffff0000u);
      unsigned hi23 = (vr[2][w] >> 16) | (vr[3][w] & 0xffff0000u);
      int d0 = 8 * dq + 2 * w;
      int d1 = d0 + 1;
      *(u32x2*)(vl + d0 * C::VSTR + vt_col(d0, kq)) = u32x2{lo01, lo23};
      *(u32x2*)(vl + d1 * C::VSTR + vt_col(d1, kq)) = u32x2{hi01, hi23};
    }
  }
}

// One 64-key tile for one wave: S^T = K Q^T, online-softmax update, O^T += V^T P^T.
template <int D>
__device__ inline void tile_compute(const uint16_t* st, int lane, const bf16x8 (&qf)[2][Cfg<D>::DC],
                                    Acc<D>& acc, float c, bool need_mask, bool causal, int n_valid,
                                    int64_t kpos0, const int64_t (&qpos)[2]) {
  using C = Cfg<D>;
  const uint16_t* kl = st;
  const uint16_t* vl = st + C::K_ELEMS;
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
      bf16x8 kf = *(const bf16x8*)(kl + (16 * kb + lr) * C::KSTR + 32 * dc + 8 * lg);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][dc], s[kb][qb], 0, 0, 0);
    }
  }

  // s[kb][qb][i] = score of key 16*kb + 4*lg + i against query column qb of this lane.
  if (need_mask) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int kk = 16 * kb + 4 * lg + i;
        int64_t kp = kpos0 + kk;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          if (kk >= n_valid || (causal && kp > qpos[qb])) s[kb][qb][i] = -INFINITY;
      }
  }

  bf16x8 pf[2][2];  // [key chunk of 32][qb]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
    mx = wave_max_cols(mx);
    float m_old = acc.m2[qb];
    float m_new = fmaxf(m_old, mx * c);
    float base = (m_new == -INFINITY) ? 0.f : m_new;
    float alpha = __builtin_amdgcn_exp2f(m_old - base);  // exp2(-inf) = 0 covers m_old = -inf
    acc.m2[qb] = m_new;
    float sum = 0.f;
    float p[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][i], c, -base));
        sum += p[kb][i];
      }
    acc.lp[qb] = acc.lp[qb] * alpha + sum;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc.o[db][qb] *= alpha;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      u32x4 w;
      w[0] = pack_bf16x2(p[2 * ch][0], p[2 * ch][1]);
      w[1] = pack_bf16x2(p[2 * ch][2], p[2 * ch][3]);
      w[2] = pack_bf16x2(p[2 * ch + 1][0], p[2 * ch + 1][1]);
      w[3] = pack_bf16x2(p[2 * ch + 1][2], p[2 * ch + 1][3]);
      pf[ch][qb] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // O^T[d][q] += sum_key V^T[d][key] P^T[key][q].  MFMA k-slot 8*lg + i of key chunk ch
  // is key 32*ch + 4*lg + i (i < 4) or 32*ch + 16 + 4*lg + (i - 4) (i >= 4) -- the
  // layout pf was packed in; the V^T operand is read with the same mapping.
#pragma unroll
  for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      int d = 16 * db + lr;
      const uint16_t* row = vl + d * C::VSTR;
      u32x2 a = *(const u32x2*)(row + vt_col(d, 8 * ch + lg));
      u32x2 b = *(const u32x2*)(row + vt_col(d, 8 * ch + 4 + lg));
      u32x4 w = u32x4{a[0], a[1], b[0], b[1]};
      bf16x8 vf = __builtin_bit_cast(bf16x8, w);
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

// The per-lane row bookkeeping shared by every kernel.
struct LaneRows {
  int64_t qpos[2];
  int64_t srow[2];   // state row t*Hq + h
  bool valid[2];
  const uint16_t* qptr[2];
};

__device__ inline LaneRows lane_rows(const QSide& qs, const RowCtx& rc, int wave, int lane) {
  LaneRows lr;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int f = rc.f0 + wave * 32 + qb * 16 + (lane & 15);
    lr.valid[qb] = f < rc.f1;
    int fc = min(f, rc.f1 - 1);
    int t = fc / qs.G;
    int j = fc - t * qs.G;
    int h = rc.g * qs.G + j;
    lr.qpos[qb] = qs.q_pos0 + t;
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
    acc.lp[qb] = (lg == 0) ? l[r] : 0.f;
#pragma unroll
    for (int db = 0; db < Cfg<D>::DB; ++db)
      acc.o[db][qb] = *(const f32x4*)(o + r * D + 16 * db + 4 * lg);
  }
}

template <int D>
__device__ inline void store_acc(const Acc<D>& acc, const LaneRows& lr, int lane, float* m, float* l, float* o,
                                 int64_t row_base) {
  const int lg = lane >> 4;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = wave_sum_cols(acc.lp[qb]);
    if (!lr.valid[qb]) continue;
    int64_t r = row_base + lr.srow[qb];
    if (lg == 0) {
      float mm = acc.m2[qb];
      m[r] = (mm == -INFINITY) ? -INFINITY : mm * kLn2;
      l[r] = lt;
    }
#pragma unroll
    for (int db = 0; db < Cfg<D>::DB; ++db) *(f32x4*)(o + r * D + 16 * db + 4 * lg) = acc.o[db][qb];
  }
}

// The key-tile loop over a list of segments, double-buffered through LDS.
template <int D, class GetSeg>
__device__ inline void run_segments(const QSide& qs, const RowCtx& rc, const LaneRows& lr, int n_seg,
                                    GetSeg get_seg, const bf16x8 (&qf)[2][Cfg<D>::DC], Acc<D>& acc,
                                    uint16_t* lds, bool wave_active) {
  using C = Cfg<D>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;

  // cursor: segment index, key offset, effective key count of that segment
  int cs = 0, ck = 0, cn = 0;
  auto seek = [&](int& s_i, int& k_o, int& n_e) {
    while (s_i < n_seg) {
      n_e = seg_effective(get_seg(s_i), qs, rc);
      if (k_o < n_e) return;
      ++s_i;
      k_o = 0;
    }
  };
  seek(cs, ck, cn);
  if (cs >= n_seg) return;

  u32x4 kr[C::K_PER_THREAD];
  u32x4 vr[4];
  {
    Seg s = get_seg(cs);
    load_tile_regs<D>(s, rc.g, ck, min(kTileKeys, cn - ck), tid, kr, vr);
    store_tile_lds<D>(lds, tid, kr, vr);
  }
  __syncthreads();
  int buf = 0;
  while (cs < n_seg) {
    int ns = cs, nk = ck + kTileKeys, nn = cn;
    seek(ns, nk, nn);
    const bool has_next = ns < n_seg;
    if (has_next) {
      Seg s = get_seg(ns);
      load_tile_regs<D>(s, rc.g, nk, min(kTileKeys, nn - nk), tid, kr, vr);
    }
    if (wave_active) {
      Seg s = get_seg(cs);
      int n_valid = min(kTileKeys, cn - ck);
      int64_t kpos0 = s.pos0 + ck;
      bool need_mask = (n_valid < kTileKeys) || (qs.causal && kpos0 + kTileKeys - 1 > rc.qpos_min);
      tile_compute<D>(lds + buf * C::STAGE, lane, qf, acc, qs.c, need_mask, qs.causal != 0, n_valid, kpos0,
                      lr.qpos);
    }
    if (has_next) store_tile_lds<D>(lds + (buf ^ 1) * C::STAGE, tid, kr, vr);
    __syncthreads();
    buf ^= 1;
    cs = ns;
    ck = nk;
    cn = nn;
  }
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
__global__ __launch_bounds__(kThreads, 1) void walk_kernel(WalkArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * Cfg<D>::STAGE];
  const int Hkv = a.qs.Hkv;
  const int g = blockIdx.x % Hkv;          // consecutive workgroups land on different XCDs;
  const int tile = blockIdx.x / Hkv;       // with Hkv = 8 each XCD serves one KV head
  const int total = a.qs.q_len * a.qs.G;
  const int f0 = tile * kTileRows;
  const int f1 = min(f0 + kTileRows, total);
  const RowCtx rc = make_rowctx(a.qs, f0, f1, g);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const LaneRows lr = lane_rows(a.qs, rc, wave, lane);
  const bool wave_active = f0 + wave * 32 < f1;

  bf16x8 qf[2][Cfg<D>::DC];
  load_q<D>(lr, lane, qf);
  Acc<D> acc;
  if (a.reset)
    init_acc<D>(acc);
  else
    load_acc<D>(acc, lr, lane, a.m, a.l, a.o);

  run_segments<D>(a.qs, rc, lr, a.n_seg, [&](int i) -> const Seg& { return a.seg[i]; }, qf, acc, lds,
                  wave_active);
  store_acc<D>(acc, lr, lane, a.m, a.l, a.o, 0);
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void split_kernel(SplitArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * Cfg<D>::STAGE];
  const int Hkv = a.qs.Hkv;
  const int g = blockIdx.x % Hkv;
  const int tile = blockIdx.x / Hkv;
  const int chunk = blockIdx.y;
  const int total = a.qs.q_len * a.qs.G;
  const int f0 = tile * kTileRows;
  const int f1 = min(f0 + kTileRows, total);
  const RowCtx rc = make_rowctx(a.qs, f0, f1, g);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const LaneRows lr = lane_rows(a.qs, rc, wave, lane);
  const bool wave_active = f0 + wave * 32 < f1;

  int s_i = 0;
  while (s_i + 1 < a.n_seg && a.chunk_begin[s_i + 1] <= chunk) ++s_i;
  const Seg& base = a.seg[s_i];
  const int k_off = (chunk - a.chunk_begin[s_i]) * a.chunk_len;
  Seg cs = base;
  cs.k = (const uint16_t*)base.k + (int64_t)k_off * base.ks_t;
  cs.v = (const uint16_t*)base.v + (int64_t)k_off * base.vs_t;
  cs.pos0 = base.pos0 + k_off;
  cs.n = min(a.chunk_len, base.n - k_off);

  bf16x8 qf[2][Cfg<D>::DC];
  load_q<D>(lr, lane, qf);
  Acc<D> acc;
  init_acc<D>(acc);
  run_segments<D>(a.qs, rc, lr, 1, [&](int) -> const Seg& { return cs; }, qf, acc, lds, wave_active);
  store_acc<D>(acc, lr, lane, a.ws_m, a.ws_l, a.ws_o, (int64_t)chunk * a.R);
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void suffix_kernel(SuffixArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * Cfg<D>::STAGE];
  const int Hkv = a.qs.Hkv;
  const int g = blockIdx.x % Hkv;
  const int b = blockIdx.x / Hkv;
  const int G = a.qs.G;
  const RowCtx rc = make_rowctx(a.qs, b * G, b * G + G, g);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const LaneRows lr = lane_rows(a.qs, rc, wave, lane);
  const bool wave_active = wave * 32 < G;

  Seg s;
  const int64_t tok = (int64_t)Hkv * D;
  s.k = (const uint16_t*)a.sk + (int64_t)b * a.S * tok;
  s.v = (const uint16_t*)a.sv + (int64_t)b * a.S * tok;
  s.ks_t = tok;
  s.vs_t = tok;
  s.ks_h = D;
  s.vs_h = D;
  s.pos0 = 0;
  s.n = a.S;

  bf16x8 qf[2][Cfg<D>::DC];
  load_q<D>(lr, lane, qf);
  Acc<D> acc;
  init_acc<D>(acc);
  run_segments<D>(a.qs, rc, lr, 1, [&](int) -> const Seg& { return s; }, qf, acc, lds, wave_active);
  store_acc<D>(acc, lr, lane, a.ws_m, a.ws_l, a.ws_o, (int64_t)a.slot * a.R);
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
    hipLaunchKernelGGL(split_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(split_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_suffix_bf16(const SuffixArgs& a, int n_branches, int D, hipStream_t s) {
  dim3 grid(n_branches * a.qs.Hkv);
  if (D == 128)
    hipLaunchKernelGGL(suffix_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(suffix_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
