// Backward pass of the blockwise attention for gfx950 (bf16 inputs, fp32
// gradients).
//
// "RingAttention and Context Parallelism" (llms.blog), section 7: the forward
// keeps Q and the per-row log-sum-exp L = m + ln l; the backward visits the K/V
// blocks again, recomputes each block's scores from Q and L, accumulates dQ for
// the stationary query block and dK, dV for the visiting block.  With
// P = exp(s - L) (the row's final softmax over every visited key):
//   dV += P^T dO,  dP = dO V^T,  dS = P * (dP - D) with D = rowsum(dO * A),
//   dQ += scale dS K,  dK += scale dS^T Q
// (the chain rule of the attention definition of its section 1).
//
// Two kernels, no atomics, so results do not depend on scheduling:
//  * dq_kernel walks key tiles for a tile of 256 query rows, exactly like the
//    forward walk (the same LDS tile pipeline): S^T = K Q^T and dP^T = V dO^T
//    with Q and dO in registers, then dQ^T += K^T dS^T with K^T read from the
//    row-major K tile by ds_read_b64_tr_b16.
//  * dkdv_kernel owns 128 keys of one visited block (32 per pair of waves,
//    their K and V in registers) and walks tiles of 64 query rows staged in
//    LDS: each wave forms S = Q K^T and dP = dO V^T for half the rows, keys
//    along the accumulator columns, so P and dS come out in the B-operand
//    layout of dV^T += dO^T P and dK^T += Q^T dS; the pair swaps them through
//    LDS, and each wave accumulates dK and dV for half the head dim over all
//    the rows, with transposing reads of the dO and Q tiles as A operands.
#include "bf16_tiles.h"

namespace ba {
namespace {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// One 4-byte-per-lane buffer load straight into LDS: lane i's word lands at dst + 4 * i.
__device__ inline void lds_dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t dst, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(size_t)dst, 4, voff, soff, 0, 0);
#endif
}

// The log-sum-exp of a row in base 2, with rows that saw no key (L = -inf)
// mapped to +inf so that exp2(s * c - L2) is 0 for them.
__device__ inline float lse2(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// n / G for 0 <= n < 2^32 with magic = floor((2^32 - 1) / G): the multiply-high
// is n / G rounded down, less at most one (its error is below n / 2^32 < 1),
// and one comparison of the remainder fixes it.
__device__ inline uint32_t div_g(uint32_t n, uint32_t G, uint32_t magic) {
  uint32_t q = __umulhi(n, magic);
  return q + ((n - q * G) >= G ? 1u : 0u);
}

// ---------------------------------------------------------------- D = rowsum(dO * A)

template <int D>
__global__ __launch_bounds__(kThreads) void delta_kernel(DeltaArgs a) {
  constexpr int TPR = D / 8;                 // threads per row, 8 elements each
  constexpr int RPB = kThreads / TPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c8 = threadIdx.x % TPR;
  float s = 0.f;
  if (r < a.rows) {
    const bf16x8 g = *(const bf16x8*)((const uint16_t*)a.dout + r * a.dout_stride + 8 * c8);
    if (a.out_bf16) {
      const bf16x8 o = *(const bf16x8*)((const uint16_t*)a.out + r * a.out_stride + 8 * c8);
#pragma unroll
      for (int i = 0; i < 8; ++i) s = __builtin_fmaf((float)g[i], (float)o[i], s);
    } else {
      const float* o = (const float*)a.out + r * a.out_stride + 8 * c8;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = __builtin_fmaf((float)g[i], o[i], s);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, TPR);
  if (r < a.rows && c8 == 0) a.delta[r] = s;
}

// ---------------------------------------------------------------- dQ

// One 64-key tile for one wave's 32 rows: dQ^T += K^T dS^T, one 32-key chunk
// at a time (its scores, dS and products finish before the next chunk's start,
// which keeps the live scores to one chunk).
template <int D>
__device__ inline void dq_tile(const lds_char* stage, int lane, const bf16x8 (&qf)[2][Cfg<D>::DC],
                               const bf16x8 (&gf)[2][Cfg<D>::DC], f32x4 (&dq)[Cfg<D>::DB][2],
                               const float (&l2)[2], const float (&dl)[2], float c, bool need_mask, bool causal,
                               int n_valid, int krel, const int (&qrel)[2]) {
  using C = Cfg<D>;
  const lds_char* kl = stage;
  const lds_char* vl = v_tile_of<D, kTileKeys>(stage);
  const int lr = lane & 15;
  const int lg = lane >> 4;
#pragma unroll
  for (int ch = 0; ch < 2; ++ch) {
    // s[h][qb][i], dp[h][qb][i]: key 32*ch + 16*h + 4*lg + i against query column qb.
    f32x4 s[2][2], dp[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[h][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[h][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 32 * ch + 16 * h + lr;
        const bf16x8 kf = *(const lds_bf16x8*)(kl + row * C::ROWB + (((4 * dc + lg) ^ swz<D>(row)) * 16));
        const bf16x8 vf = *(const lds_bf16x8*)(vl + row * C::ROWB + (((4 * dc + lg) ^ swz<D>(row)) * 16));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          s[h][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][dc], s[h][qb], 0, 0, 0);
          dp[h][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, gf[qb][dc], dp[h][qb], 0, 0, 0);
        }
      }
    }
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int lim = causal ? min(n_valid, qrel[qb] - krel + 1) : n_valid;
        const int t = lim - 4 * lg;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (32 * ch + 16 * h + i >= t) s[h][qb][i] = -INFINITY;
      }
    }
    // dS^T = P^T * (dP^T - D), rounded to bf16 in the B-operand layout of the
    // product below (k-slot 8*lg + i: key 32*ch + 4*lg + i for i < 4,
    // 32*ch + 16 + 4*lg + i - 4 otherwise).
    bf16x8 df[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float d[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][qb][i], c, -l2[qb]));
          d[h][i] = p * (dp[h][qb][i] - dl[qb]);
        }
      bf16x2 w[4];
      w[0] = pack_bf16x2(d[0][0], d[0][1]);
      w[1] = pack_bf16x2(d[0][2], d[0][3]);
      w[2] = pack_bf16x2(d[1][0], d[1][1]);
      w[3] = pack_bf16x2(d[1][2], d[1][3]);
      df[qb] = __builtin_bit_cast(bf16x8, w);
    }
    // dQ^T[d][q] += sum_key K^T[d][key] dS^T[key][q]: K^T straight from the
    // row-major K tile by transposing reads (the forward's V^T read on K).
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int row0 = 32 * ch + 4 * lg + (lr >> 2);
      const int row1 = row0 + 16;
      const int cidx = 2 * db + ((lr & 3) >> 1);
      const int half = (lr & 1) * 8;
      const lds_char* a0 = kl + row0 * C::ROWB + ((cidx ^ swz<D>(row0)) * 16) + half;
      const lds_char* a1 = kl + row1 * C::ROWB + ((cidx ^ swz<D>(row1)) * 16) + half;
      const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a0);
      const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a1);
      const s16x8 xx = s16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      const bf16x8 kt = __builtin_bit_cast(bf16x8, xx);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        dq[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, df[qb], dq[db][qb], 0, 0, 0);
    }
  }
}

// dQ workgroups: 8 waves of 32 query rows, so each K/V tile staged in LDS
// serves 256 rows (as in the forward walk).
constexpr int kDqWaves = 8;
constexpr int kDqRows = 32 * kDqWaves;

template <int D>
__global__ __launch_bounds__(64 * kDqWaves, 1) void dq_kernel(BwdArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char lds[2 * C::STAGEB];
  const QSide& qs = a.qs;
  const int Hkv = qs.Hkv;
  const int g = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int b = rest % qs.B;
  const int n_tiles = (qs.q_len * qs.G + kDqRows - 1) / kDqRows;
  const int tile = n_tiles - 1 - rest / qs.B;  // causal: longest rows first
  const int total = qs.q_len * qs.G;
  const int f0 = tile * kDqRows;
  const int f1 = min(f0 + kDqRows, total);
  const RowCtx rc = make_rowctx(qs, f0, f1, g, b);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const LaneRows lr = lane_rows(qs, rc, wave, lane);
  const bool wave_active = f0 + wave * 32 < f1;

  bf16x8 qf[2][C::DC], gf[2][C::DC];
  float l2[2], dl[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t off = lr.qptr[qb] - (const uint16_t*)qs.q;
    const uint16_t* gp = (const uint16_t*)a.dout + off;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
      qf[qb][dc] = *(const bf16x8*)(lr.qptr[qb] + 32 * dc + 8 * (lane >> 4));
      gf[qb][dc] = *(const bf16x8*)(gp + 32 * dc + 8 * (lane >> 4));
    }
    l2[qb] = lse2(a.lse[lr.srow[qb]]);
    dl[qb] = a.delta[lr.srow[qb]];
  }
  f32x4 dq[C::DB][2];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) dq[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  run_segments<D, kCacheReuse, kDqWaves>(
      qs, rc, a.n_seg, [&](int i) -> const Seg& { return a.seg[i]; },
      [&](const lds_char* stage, bool need_mask, int n_valid, int krel) {
        dq_tile<D>(stage, lane, qf, gf, dq, l2, dl, qs.c, need_mask, qs.causal != 0, n_valid, krel, lr.qrel);
      },
      (lds_char*)lds, wave_active);

  // dq[r, 16*db + 4*lg + i] += scale * dQ^T.
  const LaneRows lw = lane_rows(qs, rc, wave, lane);
  const int lg = lane >> 4;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!lw.valid[qb] || !wave_active) continue;
    float* dst = a.dq + lw.srow[qb] * D + 4 * lg;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      f32x4 v = *(f32x4*)(dst + 16 * db);
      v += dq[db][qb] * a.scale;
      *(f32x4*)(dst + 16 * db) = v;
    }
  }
}

// ---------------------------------------------------------------- dK, dV

constexpr int kRowTile = 64;    // query rows per LDS stage of the dK/dV kernel
constexpr int kDkvWaves = 8;    // four pairs of waves, each pair on 32 of the workgroup's kDkvKeys keys
static_assert(kDkvKeys == 32 * kDkvWaves / 2, "a dK/dV workgroup covers 32 keys per pair of waves");

template <int D>
struct BwdCfg {
  static constexpr int ROWB = D * 2;
  static constexpr int CPR = D / 8;
  static constexpr int TILEB = kRowTile * ROWB;        // one Q (or dO) tile
  static constexpr int RPI = 64 / CPR;                 // rows per wave-wide 1 KiB load
  static constexpr int LPW = kRowTile / RPI / kDkvWaves;   // loads per wave per tile
  static constexpr int DC = D / 32;
  static constexpr int DB = D / 16;
  static constexpr int DBH = DB / 2;                   // 16-wide d blocks in half of D
  // LDS: the two stages' Q tiles, then their dO tiles, then per stage the
  // rows' log-sum-exp and D (64 floats each), then per wave the P and dS
  // fragments it hands to the other wave of its pair.  Every Q and dO read
  // addresses from a per-lane base with an immediate offset below 64 KiB
  // that folds in the stage.
  static constexpr int QOFF = 0;
  static constexpr int GOFF = 2 * TILEB;
  static constexpr int LOFF = 4 * TILEB;
  static constexpr int LSTAGE = 2 * kRowTile * 4;
  static constexpr int XOFF = LOFF + 2 * LSTAGE;
  static constexpr int XWAVE = 2 * 2 * 64 * 16;       // [key block][P, dS][lane] x 16 bytes
  static constexpr int LDSB = XOFF + kDkvWaves * XWAVE;
  static_assert(LPW >= 1 && LPW * RPI * kDkvWaves == kRowTile, "row tile loads split evenly over the waves");
};

// Per-lane byte offsets of one row tile's loads: Q and dO rows (load j of
// this lane) and, in waves 0 and 1, the log-sum-exp or D of row f0 + lane.
template <int D>
struct RowOffs {
  uint32_t q[BwdCfg<D>::LPW];
  uint32_t l;
};

// The offsets of the loads of query-row tile f0 .. f0 + 63 (flat rows of KV
// head g).  Rows past the last are loaded as the last row; the caller masks
// them.
template <int D>
__device__ inline RowOffs<D> row_offsets(const BwdArgs& a, int f0, int g, int wave, int lane) {
  using C = BwdCfg<D>;
  const QSide& qs = a.qs;
  const uint32_t G = (uint32_t)qs.G;
  const uint32_t last = (uint32_t)(qs.q_len * qs.G - 1);
  const uint32_t st = (uint32_t)qs.qs_t, sh = (uint32_t)qs.qs_h;   // q spans < 4 GiB: 32-bit offsets
  const int rsub = lane / C::CPR;
  const int p = lane % C::CPR;
  RowOffs<D> o;
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const int row = (wave * C::LPW + j) * C::RPI + rsub;
    const uint32_t f = min((uint32_t)(f0 + row), last);
    const uint32_t t = div_g(f, G, a.g_magic);
    const uint32_t h = (uint32_t)g * G + (f - t * G);
    o.q[j] = (t * st + h * sh) * 2u + (uint32_t)((p ^ swz<D>(row)) * 16);
  }
  const uint32_t f = min((uint32_t)(f0 + lane), last);
  const uint32_t t = div_g(f, G, a.g_magic);
  const uint32_t h = (uint32_t)g * G + (f - t * G);
  o.l = (t * (uint32_t)qs.Hq + h) * 4u;
  return o;
}

// Issues the loads of one row tile into the stage whose Q tile is at `qdst`
// (its dO tile at qdst + GOFF, its log-sum-exp and D at `ldst`): Q and dO
// rows, swizzled as the K/V tiles are, then the rows' log-sum-exp and D.
template <int D>
__device__ inline void issue_rows(__amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rg, __amdgpu_buffer_rsrc_t rl,
                                  __amdgpu_buffer_rsrc_t rd, const RowOffs<D>& o, uint32_t qdst, uint32_t ldst,
                                  int wave) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const uint32_t dst = qdst + (uint32_t)((wave * C::LPW + j) * C::RPI) * C::ROWB;
    lds_dma16(rq, dst, o.q[j], 0);
    lds_dma16(rg, dst + C::GOFF, o.q[j], 0);
  }
  if (wave < 2) lds_dma4(wave == 0 ? rl : rd, ldst + (uint32_t)(wave * kRowTile * 4), o.l, 0);
}

// Every wave's LDS writes done and visible to the workgroup, without waiting
// for the next row tile's loads still in flight into the other stage.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One tile of 64 query rows for one wave of a pair.  The pair shares 32 keys,
// two 16-key blocks kb whose K and V the wave keeps in registers.  Wave half h
// forms S = Q K^T and dP = dO V^T for rows 32h .. 32h + 31 (keys along the
// accumulator columns, so P and dS come out in the B-operand layout of the
// products over rows), hands P and dS to the other wave through LDS at `xl`
// (the other wave's at `xo`), and then accumulates dV^T += dO^T P and
// dK^T += Q^T dS over all 64 rows for its half of D, whose A operands are
// transposing reads of the dO and Q tiles.  Stage: Q tile at `ql`, dO tile at
// `gl`, the rows' log-sum-exp and D at `ls`.
template <int D>
__device__ inline void dkdv_tile(const lds_char* ql, const lds_char* gl, const lds_char* ls, lds_char* xl,
                                 const lds_char* xo, int lane, int h, const bf16x8 (&kf)[2][BwdCfg<D>::DC],
                                 const bf16x8 (&vf)[2][BwdCfg<D>::DC], f32x4 (&dk)[BwdCfg<D>::DBH][2],
                                 f32x4 (&dv)[BwdCfg<D>::DBH][2], float c, bool need_mask, int f0,
                                 const int (&f_begin)[2], const int (&f_end)[2]) {
  using C = BwdCfg<D>;
  const float* l2s = (const float*)ls;
  const float* dls = l2s + kRowTile;
  const int lr = lane & 15;
  const int lg = lane >> 4;

  // s[rb][kb][i], dp[rb][kb][i]: row 32h + 16*rb + 4*lg + i of the tile against key 16*kb + lr.
  f32x4 s[2][2], dp[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // Each 32-wide d chunk: its four Q and dO fragment reads first, then the
  // eight products, each fragment serving both key blocks.
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
    bf16x8 qa[2], ga[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = 32 * h + 16 * rb + lr;
      const int off = row * C::ROWB + (((4 * dc + lg) ^ swz<D>(row)) * 16);
      qa[rb] = *(const lds_bf16x8*)(ql + off);
      ga[rb] = *(const lds_bf16x8*)(gl + off);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rb], kf[kb][dc], s[rb][kb], 0, 0, 0);
        dp[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[rb], vf[kb][dc], dp[rb][kb], 0, 0, 0);
      }
  }
  // A row that saw no key has L = -inf and gives exp2(+inf) here; every pair
  // of such a row is masked below (an unmasked tile holds only rows that see
  // all its keys), so no per-element test is needed.
  float p[2][2][4], d[2][2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const f32x4 lse = *(const __attribute__((address_space(3))) f32x4*)(l2s + 32 * h + 16 * rb + 4 * lg);
    const f32x4 dl = *(const __attribute__((address_space(3))) f32x4*)(dls + 32 * h + 16 * rb + 4 * lg);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[rb][kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][kb][i], c, -kLog2e * lse[i]));
        d[rb][kb][i] = p[rb][kb][i] * (dp[rb][kb][i] - dl[i]);
      }
  }
  if (need_mask) {
    // Key 16*kb + lr of this lane is visible to flat rows in [f_begin[kb],
    // f_end[kb]): from the first row of the first token at or after its
    // position (causal) up to the last valid row; f_end is 0 for a key past
    // the block's end.
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = f0 + 32 * h + 16 * rb + 4 * lg + i;
          const bool vis = (f >= f_begin[kb]) & (f < f_end[kb]);
          p[rb][kb][i] = vis ? p[rb][kb][i] : 0.f;
          d[rb][kb][i] = vis ? d[rb][kb][i] : 0.f;
        }
  }
  // P and dS of row chunk h (rows 32h .. 32h + 31) in the B-operand layout of
  // the products over rows: k-slot 8*lg + i is row 32h + 4*lg + i (i < 4) or
  // 32h + 16 + 4*lg + i - 4.
  bf16x8 pf[2][2], df[2][2];   // [own chunk, other wave's chunk][kb]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    bf16x2 w[4], x[4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      w[2 * rb] = pack_bf16x2(p[rb][kb][0], p[rb][kb][1]);
      w[2 * rb + 1] = pack_bf16x2(p[rb][kb][2], p[rb][kb][3]);
      x[2 * rb] = pack_bf16x2(d[rb][kb][0], d[rb][kb][1]);
      x[2 * rb + 1] = pack_bf16x2(d[rb][kb][2], d[rb][kb][3]);
    }
    pf[0][kb] = __builtin_bit_cast(bf16x8, w);
    df[0][kb] = __builtin_bit_cast(bf16x8, x);
    *(lds_bf16x8*)(xl + ((2 * kb) * 64 + lane) * 16) = pf[0][kb];
    *(lds_bf16x8*)(xl + ((2 * kb + 1) * 64 + lane) * 16) = df[0][kb];
  }
  // The other wave wrote the same lanes' fragments of its row chunk 1 - h.
  lds_barrier();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    pf[1][kb] = *(const lds_bf16x8*)(xo + ((2 * kb) * 64 + lane) * 16);
    df[1][kb] = *(const lds_bf16x8*)(xo + ((2 * kb + 1) * 64 + lane) * 16);
  }
  // dV^T[d][key] += sum_row dO^T[d][row] P[row][key];  dK^T += Q^T dS, over
  // both row chunks, for d blocks DBH*h .. DBH*h + DBH - 1.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ch = j == 0 ? h : 1 - h;
#pragma unroll
    for (int dbl = 0; dbl < C::DBH; ++dbl) {
      const int db = C::DBH * h + dbl;
      const int row0 = 32 * ch + 4 * lg + (lr >> 2);
      const int row1 = row0 + 16;
      const int cidx = 2 * db + ((lr & 3) >> 1);
      const int half = (lr & 1) * 8;
      const int o0 = row0 * C::ROWB + ((cidx ^ swz<D>(row0)) * 16) + half;
      const int o1 = row1 * C::ROWB + ((cidx ^ swz<D>(row1)) * 16) + half;
      const s16x4 g0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(gl + o0));
      const s16x4 g1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(gl + o1));
      const s16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(ql + o0));
      const s16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(ql + o1));
      const bf16x8 gt = __builtin_bit_cast(bf16x8, s16x8{g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]});
      const bf16x8 qt = __builtin_bit_cast(bf16x8, s16x8{q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]});
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dv[dbl][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gt, pf[j][kb], dv[dbl][kb], 0, 0, 0);
        dk[dbl][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt, df[j][kb], dk[dbl][kb], 0, 0, 0);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(64 * kDkvWaves, 1) void dkdv_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) char lds[C::LDSB];
  const QSide& qs = a.qs;
  const int Hkv = qs.Hkv;
  const int g = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int b = rest % qs.B;                    // sequence
  const int tile = rest / qs.B;
  int si = 0;
  while (si + 1 < a.n_seg && a.tile_begin[si + 1] <= tile) ++si;
  const Seg& sg = a.seg[si];
  const int k0 = (tile - a.tile_begin[si]) * kDkvKeys;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = wave & 1;                       // half of the pair: its rows in S, its half of D in dK, dV
  const int n_keys = sg.n;
  const int total = qs.q_len * qs.G;
  // Flat row from which a key at position pos is visible (causal): the first
  // row of token pos - q_pos0, clamped to [0, total].
  auto first_row = [&](int64_t pos) -> int {
    if (!qs.causal) return 0;
    const int64_t r = (pos - qs.q_pos0) * qs.G;
    return (int)(r < 0 ? 0 : (r > total ? total : r));
  };
  // This lane's keys (columns of S): 16*kb + lane%16 of the pair's 32.
  int key_idx[2], f_begin[2], f_end[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    key_idx[kb] = k0 + 32 * (wave >> 1) + 16 * kb + (lane & 15);
    f_begin[kb] = first_row(sg.pos0 + key_idx[kb]);
    f_end[kb] = key_idx[kb] < n_keys ? total : 0;
  }

  // The pair's keys as B operands: key 32*(wave/2) + 16*kb + lane%16, d = 32*dc + 8*(lane/16) .. +7.
  bf16x8 kf[2][C::DC], vf[2][C::DC];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kk = min(key_idx[kb], n_keys - 1);
    const uint16_t* kp = (const uint16_t*)sg.k + (int64_t)b * sg.ks_b + (int64_t)kk * sg.ks_t + (int64_t)g * sg.ks_h +
                         8 * (lane >> 4);
    const uint16_t* vp = (const uint16_t*)sg.v + (int64_t)b * sg.vs_b + (int64_t)kk * sg.vs_t + (int64_t)g * sg.vs_h +
                         8 * (lane >> 4);
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
      kf[kb][dc] = *(const bf16x8*)(kp + 32 * dc);
      vf[kb][dc] = *(const bf16x8*)(vp + 32 * dc);
    }
  }
  f32x4 dk[C::DBH][2], dv[C::DBH][2];
#pragma unroll
  for (int dbl = 0; dbl < C::DBH; ++dbl)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      dk[dbl][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[dbl][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // Query-row tiles that can see a key of this tile: with the causal rule,
  // rows from the first token at or after the tile's first key position.  Rows
  // below full_from miss at least one of the tile's keys.
  const int r_begin = first_row(sg.pos0 + k0);
  const int full_from = first_row(sg.pos0 + min(k0 + kDkvKeys, n_keys) - 1);
  const int t_end = (total + kRowTile - 1) / kRowTile;
  const int t_begin = r_begin >= total ? t_end : r_begin / kRowTile;

  if (t_begin < t_end) {
    // The sequence's own Q, dO, LSE and delta rows: q_bytes and rows_bytes are
    // one sequence's extents.
    const int64_t q_off = (int64_t)b * qs.qs_b;
    const int64_t row0 = (int64_t)b * qs.q_len * qs.Hq;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t*)qs.q + q_off, a.q_bytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc((const uint16_t*)a.dout + q_off, a.q_bytes);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lse + row0, a.rows_bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.delta + row0, a.rows_bytes);
    const uint32_t lds_addr = (uint32_t)(size_t)(lds_char*)lds;
    lds_char* xl = (lds_char*)lds + C::XOFF + wave * C::XWAVE;
    const lds_char* xo = (const lds_char*)lds + C::XOFF + (wave ^ 1) * C::XWAVE;
    // When the group size divides the row tile, the rows of tile t are those
    // of tile 0 moved by 64 t / G tokens: each lane's offsets are computed once
    // and stepped.  A tile that reaches past the last row (clamped loads), or
    // any tile when G does not divide 64, computes them in full.
    const bool stepped = kRowTile % qs.G == 0;
    RowOffs<D> base = {};
    if (stepped) base = row_offsets<D>(a, 0, g, wave, lane);
    const uint32_t tok_step = stepped ? (uint32_t)(kRowTile / qs.G) : 0u;
    const uint32_t q_step = tok_step * (uint32_t)qs.qs_t * 2u;
    const uint32_t l_step = tok_step * (uint32_t)qs.Hq * 4u;
    auto issue = [&](int t, int stage) {
      RowOffs<D> o;
      if (stepped && (t + 1) * kRowTile <= total) {
        o = base;
#pragma unroll
        for (int j = 0; j < C::LPW; ++j) o.q[j] += (uint32_t)t * q_step;
        o.l += (uint32_t)t * l_step;
      } else {
        o = row_offsets<D>(a, t * kRowTile, g, wave, lane);
      }
      issue_rows<D>(rq, rg, rl, rd, o, lds_addr + (uint32_t)(C::QOFF + stage * C::TILEB),
                    lds_addr + (uint32_t)(C::LOFF + stage * C::LSTAGE), wave);
    };
    // One row tile in stage `cur` (a constant in each unrolled copy below, so
    // the stage's LDS offsets are immediates): wait for it, let the next one
    // start loading into the other stage, multiply.  The barrier also ends
    // every wave's reads of the other stage and of the P/dS hand-over area
    // from the previous tile.
    auto step = [&](int t, int cur) {
      wait_all_loads();
      __syncthreads();
      if (t > t_begin) issue(t - 1, cur ^ 1);
      const int f0 = t * kRowTile;
      const bool need_mask = (k0 + kDkvKeys > n_keys) || (f0 + kRowTile > total) || (f0 < full_from);
      const lds_char* l = (const lds_char*)lds;
      dkdv_tile<D>(l + C::QOFF + cur * C::TILEB, l + C::GOFF + cur * C::TILEB, l + C::LOFF + cur * C::LSTAGE, xl,
                   xo, lane, h, kf, vf, dk, dv, qs.c, need_mask, f0, f_begin, f_end);
    };
    // Row tiles are walked from the last one down: every workgroup of a KV
    // head then starts at the same row tile and the resident ones stream Q
    // and dO in step, so each tile is fetched once into L2 and read from there
    // by the others (the causal rule only moves where a workgroup stops).
    issue(t_end - 1, 0);
    for (int t = t_end - 1;;) {
      step(t, 0);
      if (--t < t_begin) break;
      step(t, 1);
      if (--t < t_begin) break;
    }
    wait_all_loads();
  }

  // dk[b, key, g, 16*db + 4*(lane/16) + i] += scale * dK^T; dv likewise, unscaled.
  if (t_begin < t_end) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (key_idx[kb] >= n_keys) continue;
      const int64_t base = (((int64_t)b * n_keys + key_idx[kb]) * Hkv + g) * D + 4 * (lane >> 4);
      float* dkp = a.dk[si] + base;
      float* dvp = a.dv[si] + base;
#pragma unroll
      for (int dbl = 0; dbl < C::DBH; ++dbl) {
        const int db = C::DBH * h + dbl;
        f32x4 x = *(f32x4*)(dkp + 16 * db);
        x += dk[dbl][kb] * a.scale;
        *(f32x4*)(dkp + 16 * db) = x;
        f32x4 y = *(f32x4*)(dvp + 16 * db);
        y += dv[dbl][kb];
        *(f32x4*)(dvp + 16 * db) = y;
      }
    }
  }
}

}  // namespace

hipError_t launch_delta(const DeltaArgs& a, int D, hipStream_t s) {
  const int rpb = kThreads / (D / 8);
  dim3 grid((unsigned)((a.rows + rpb - 1) / rpb));
  if (D == 128)
    hipLaunchKernelGGL(delta_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(delta_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int n_key_tiles, int D, hipStream_t s) {
  const int tiles = (a.qs.q_len * a.qs.G + kDqRows - 1) / kDqRows;
  dim3 grid_q(tiles * a.qs.Hkv * a.qs.B);
  dim3 grid_k(n_key_tiles * a.qs.Hkv * a.qs.B);
  if (D == 128) {
    hipLaunchKernelGGL(dq_kernel<128>, grid_q, dim3(64 * kDqWaves), 0, s, a);
    if (n_key_tiles > 0) hipLaunchKernelGGL(dkdv_kernel<128>, grid_k, dim3(64 * kDkvWaves), 0, s, a);
  } else {
    hipLaunchKernelGGL(dq_kernel<64>, grid_q, dim3(64 * kDqWaves), 0, s, a);
    if (n_key_tiles > 0) hipLaunchKernelGGL(dkdv_kernel<64>, grid_k, dim3(64 * kDkvWaves), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ba
