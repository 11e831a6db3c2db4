// fp32 blockwise attention with running online-softmax state (the fp32 path).
//
// Same recurrence as the bf16 kernels -- "RingAttention and Context
// Parallelism" (llms.blog), section 2 state-transition box, from the section 3
// initial state, causal rule of section 5 -- with every product, sum and
// exponential in fp32 on the vector ALUs.  One lane owns one query row and
// keeps q, O, m, l in registers; 32-key K/V tiles are staged in LDS and read
// by broadcast.  Meant for exactness checks at small sizes, not for speed.  A
// call whose row tiles do not fill the GPU splits its keys into chunks walked
// in parallel (split_f32_kernel) whose partial states merge afterwards, as
// on the bf16 path.
#include "internal.h"

namespace ba {
namespace {

constexpr int kRows = 64;   // one wave, one row per lane
constexpr int kKeys = 32;   // keys per LDS tile

// The recurrence for one workgroup's tile of 64 flat rows of KV head g of
// sequence b over get_seg(0..n_seg): from the initial state when `reset`, else
// from the state rows of (m_in, l_in, o_in); the result goes to state row
// row_base + r of (m_out, l_out, o_out).  Every lane of the workgroup runs the
// key loops (their barriers), also lanes past the tile's last row.
template <int D, class GetSeg>
__device__ inline void f32_tile(const QSide& qs, int b, int g, int tile, int n_seg, GetSeg get_seg, bool reset,
                                const float* m_in, const float* l_in, const float* o_in, float* m_out, float* l_out,
                                float* o_out, int64_t row_base) {
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];
  const int total = qs.q_len * qs.G;
  const int f0 = tile * kRows;
  const int f1 = min(f0 + kRows, total);
  const int lane = threadIdx.x;
  const int f = f0 + lane;
  const bool valid = f < f1;
  const int fc = min(f, f1 - 1);
  const int t = fc / qs.G;
  const int h = g * qs.G + (fc - t * qs.G);
  const int64_t qpos = qs.q_pos0 + t;
  const int64_t qpos_max = qs.q_pos0 + (f1 - 1) / qs.G;
  const int64_t srow = ((int64_t)b * qs.q_len + t) * qs.Hq + h;

  float q[D], o[D];
  const float* qp = (const float*)qs.q + (int64_t)b * qs.qs_b + (int64_t)t * qs.qs_t + (int64_t)h * qs.qs_h;
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = qp[d];
  float m2, l;
  if (reset) {
    m2 = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = 0.f;
  } else {
    float mm = m_in[srow];
    m2 = (mm == -INFINITY) ? -INFINITY : mm * kLog2e;
    l = l_in[srow];
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = o_in[srow * D + d];
  }

  for (int si = 0; si < n_seg; ++si) {
    const Seg& s = get_seg(si);
    int n = s.n;
    if (qs.causal) {
      int64_t lim = qpos_max - s.pos0 + 1;
      n = (int)max((int64_t)0, min((int64_t)n, lim));
    }
    const float* kb = (const float*)s.k + (int64_t)b * s.ks_b + (int64_t)g * s.ks_h;
    const float* vb = (const float*)s.v + (int64_t)b * s.vs_b + (int64_t)g * s.vs_h;
    for (int k0 = 0; k0 < n; k0 += kKeys) {
      const int nv = min(kKeys, n - k0);
      __syncthreads();
      for (int e = lane; e < kKeys * D; e += kRows) {
        int j = e / D, d = e % D;
        int jj = min(j, nv - 1);
        ks[j][d] = kb[(int64_t)(k0 + jj) * s.ks_t + d];
        vs[j][d] = vb[(int64_t)(k0 + jj) * s.vs_t + d];
      }
      __syncthreads();
      float sc[kKeys];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kKeys; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc = __builtin_fmaf(q[d], ks[j][d], acc);
        bool vis = j < nv && (!qs.causal || s.pos0 + k0 + j <= qpos);
        sc[j] = vis ? acc * qs.c : -INFINITY;
        mx = fmaxf(mx, sc[j]);
      }
      const float m_new = fmaxf(m2, mx);
      const float base = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m2 - base);
      m2 = m_new;
      float sum = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
      for (int j = 0; j < kKeys; ++j) {
        float p = __builtin_amdgcn_exp2f(sc[j] - base);
        sum += p;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, vs[j][d], o[d]);
      }
      l = l * alpha + sum;
    }
  }
  if (!valid) return;
  const int64_t r = row_base + srow;
  m_out[r] = (m2 == -INFINITY) ? -INFINITY : m2 * kLn2;
  l_out[r] = l;
#pragma unroll
  for (int d = 0; d < D; ++d) o_out[r * D + d] = o[d];
}

// Workgroups take the KV heads, then the sequences, then the row tiles.
template <int D>
__global__ __launch_bounds__(kRows) void walk_f32_kernel(WalkArgs a) {
  const int g = blockIdx.x % a.qs.Hkv;
  const int rest = blockIdx.x / a.qs.Hkv;
  f32_tile<D>(a.qs, rest % a.qs.B, g, rest / a.qs.B, a.n_seg, [&](int i) -> const Seg& { return a.seg[i]; },
              a.reset != 0, a.m, a.l, a.o, a.m, a.l, a.o, 0);
}

// The split form: workgroup (row tile, sequence, KV head) x chunk walks one
// key chunk from the initial state and writes its partial state to workspace
// slot `chunk` (see SplitArgs); the partial states merge afterwards.
template <int D>
__global__ __launch_bounds__(kRows) void split_f32_kernel(SplitArgs a) {
  const int g = blockIdx.x % a.qs.Hkv;
  const int rest = blockIdx.x / a.qs.Hkv;
  const int chunk = blockIdx.y;
  const Seg cs = chunk_seg<float>(a.seg, a.n_seg, a.chunk_begin, a.chunk_len, chunk);
  f32_tile<D>(a.qs, rest % a.qs.B, g, rest / a.qs.B, 1, [&](int) -> const Seg& { return cs; }, true, nullptr,
              nullptr, nullptr, a.ws_m, a.ws_l, a.ws_o, (int64_t)chunk * a.R);
}

}  // namespace

hipError_t launch_walk_f32(const WalkArgs& a, int D, hipStream_t s) {
  const int tiles = (a.qs.q_len * a.qs.G + kRows - 1) / kRows;
  dim3 grid(tiles * a.qs.Hkv * a.qs.B);
  if (D == 128)
    hipLaunchKernelGGL(walk_f32_kernel<128>, grid, dim3(kRows), 0, s, a);
  else
    hipLaunchKernelGGL(walk_f32_kernel<64>, grid, dim3(kRows), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split_f32(const SplitArgs& a, int n_chunks, int D, hipStream_t s) {
  const int tiles = (a.qs.q_len * a.qs.G + kRows - 1) / kRows;
  dim3 grid(tiles * a.qs.Hkv * a.qs.B, n_chunks);
  if (D == 128)
    hipLaunchKernelGGL(split_f32_kernel<128>, grid, dim3(kRows), 0, s, a);
  else
    hipLaunchKernelGGL(split_f32_kernel<64>, grid, dim3(kRows), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
