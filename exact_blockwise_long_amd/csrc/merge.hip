// Log-sum-exp merge of partial online-softmax states, and finalisation.
//
// Merge ("AHBM Agentic Runtime Architecture", s.3.4-3.5; "Supporting Agentic
// Workloads", Stationary-KV policy): states of the same row computed over
// disjoint key sets combine as m* = max_s m_s, w_s = exp(m_s - m*),
// l* = sum_s w_s l_s, O* = sum_s w_s O_s -- the rescale step of the online
// softmax ("RingAttention and Context Parallelism", section 2) applied to a
// whole partial state.  Rows never mix.  Finalisation is A = O / l (section 2)
// and LSE = m + ln l (section 7).
//
// These kernels stream rows: D/4 lanes own one row, each lane 4 consecutive
// floats (16-byte loads and stores), so a wave covers 2 (D = 128) or 4
// (D = 64) rows with fully coalesced traffic.  Bandwidth bound.
#include "internal.h"

namespace ba {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

__device__ inline float exp_nat(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ inline unsigned pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a;
  __bf16 y = (__bf16)b;
  return (unsigned)__builtin_bit_cast(unsigned short, x) |
         ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
}

__device__ inline void write_final(const f32x4& acc, float m, float l, int64_t r, int q4, uint16_t* out_bf16,
                                   float* out_f32, int64_t stride, float* lse) {
  const bool empty = !(l > 0.f);
  f32x4 a;
  if (empty) {
    a = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    a = f32x4{acc[0] / l, acc[1] / l, acc[2] / l, acc[3] / l};
  }
  if (out_bf16) {
    u32x2 w = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
    *(u32x2*)(out_bf16 + r * stride + 4 * q4) = w;
  } else {
    *(f32x4*)(out_f32 + r * stride + 4 * q4) = a;
  }
  if (lse && q4 == 0) lse[r] = empty ? -INFINITY : m + logf(l);
}

template <int D>
__global__ __launch_bounds__(kThreads) void merge_groups_kernel(MergeGroupArgs a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = kThreads / TPR;
  const int gi = blockIdx.y;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int q4 = threadIdx.x % TPR;
  if (r >= a.R) return;
  const int p0 = a.part_begin[gi];
  const int p1 = a.part_begin[gi + 1];
  const int64_t R = a.R;

  float init_m = -INFINITY, init_l = 0.f;
  f32x4 init_o = f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.has_init) {
    init_m = a.out_m[gi][r];
    if (init_m != -INFINITY) {
      init_l = a.out_l[gi][r];
      init_o = *(const f32x4*)(a.out_o[gi] + r * D + 4 * q4);
    }
  }
  float mstar = init_m;
  for (int p = p0; p < p1; ++p) mstar = fmaxf(mstar, a.pm[p * R + r]);
  const float base = (mstar == -INFINITY) ? 0.f : mstar;
  float l = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (init_m != -INFINITY) {
    float w = exp_nat(init_m - base);
    l = w * init_l;
    acc = w * init_o;
  }
  for (int p = p0; p < p1; ++p) {
    float mp = a.pm[p * R + r];
    if (mp == -INFINITY) continue;
    float w = exp_nat(mp - base);
    l += w * a.pl[p * R + r];
    f32x4 op = *(const f32x4*)(a.po + (p * R + r) * D + 4 * q4);
    acc += w * op;
  }
  if (a.fin_out) {
    write_final(acc, mstar, l, r, q4, a.fin_out, nullptr, D, a.fin_lse);
    return;
  }
  *(f32x4*)(a.out_o[gi] + r * D + 4 * q4) = acc;
  if (q4 == 0) {
    a.out_m[gi][r] = mstar;
    a.out_l[gi][r] = l;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void merge_ptrs_kernel(MergePtrArgs a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = kThreads / TPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int q4 = threadIdx.x % TPR;
  if (r >= a.R) return;
  float mstar = -INFINITY;
  for (int p = 0; p < a.n_parts; ++p) mstar = fmaxf(mstar, a.m[p][r]);
  const float base = (mstar == -INFINITY) ? 0.f : mstar;
  float l = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < a.n_parts; ++p) {
    float mp = a.m[p][r];
    if (mp == -INFINITY) continue;
    float w = exp_nat(mp - base);
    l += w * a.l[p][r];
    acc += w * *(const f32x4*)(a.o[p] + r * D + 4 * q4);
  }
  *(f32x4*)(a.out_o + r * D + 4 * q4) = acc;
  if (q4 == 0) {
    a.out_m[r] = mstar;
    a.out_l[r] = l;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void finalize_kernel(FinalizeArgs a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = kThreads / TPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int q4 = threadIdx.x % TPR;
  if (r >= a.R) return;
  const float l = a.l[r];
  const float m = a.m[r];
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (l > 0.f) acc = *(const f32x4*)(a.o + r * D + 4 * q4);
  write_final(acc, m, l, r, q4, a.out_bf16 ? (uint16_t*)a.out : nullptr, a.out_bf16 ? nullptr : (float*)a.out,
              a.out_stride, a.lse);
}

template <int D>
inline int blocks_for(int64_t R) {
  constexpr int RPB = kThreads / (D / 4);
  return (int)((R + RPB - 1) / RPB);
}

}  // namespace

hipError_t launch_merge_groups(const MergeGroupArgs& a, int D, hipStream_t s) {
  if (D == 128)
    hipLaunchKernelGGL(merge_groups_kernel<128>, dim3(blocks_for<128>(a.R), a.n_groups), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(merge_groups_kernel<64>, dim3(blocks_for<64>(a.R), a.n_groups), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge_ptrs(const MergePtrArgs& a, int D, hipStream_t s) {
  if (D == 128)
    hipLaunchKernelGGL(merge_ptrs_kernel<128>, dim3(blocks_for<128>(a.R)), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(merge_ptrs_kernel<64>, dim3(blocks_for<64>(a.R)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, int D, hipStream_t s) {
  if (D == 128)
    hipLaunchKernelGGL(finalize_kernel<128>, dim3(blocks_for<128>(a.R)), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(finalize_kernel<64>, dim3(blocks_for<64>(a.R)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
