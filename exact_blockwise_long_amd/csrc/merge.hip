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
// Layout of the work: a "slice" of D/4 lanes covers one row's D floats (16
// bytes per lane, coalesced).  A workgroup of 256 lanes holds 256/(D/4)
// slices; they are spread over rows and over the parts of each row, so a row
// with many parts is merged by several slices in parallel (each folds its
// parts with a running max, loads unrolled so several are in flight), and
// the slices of a row are combined through LDS with the same rule.  With few
// parts per row the slices cover more rows instead.  Bandwidth bound.
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

// Running merge accumulator of one slice lane: (m, l, 4 floats of O).
struct Run {
  float m, l;
  f32x4 o;
};

__device__ inline void run_init(Run& r) {
  r.m = -INFINITY;
  r.l = 0.f;
  r.o = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Fold one part into the running state.  A part with m = -inf contributes
// nothing (its l and O are not used, so garbage there cannot leak in).  A
// part with m = +inf marks a row whose keys could not be read (the fan-out's
// corrupt page ids): the row takes that part as it is (l = 1, O = NaN) and
// ignores every other part, so it finalises to NaN with LSE +inf.
__device__ inline void run_add(Run& r, float m, float l, const f32x4& o) {
  if (m == -INFINITY || r.m == INFINITY) return;
  if (m == INFINITY) {
    r.m = m;
    r.l = l;
    r.o = o;
    return;
  }
  if (m > r.m) {
    const float a = exp_nat(r.m - m);  // 0 when r.m = -inf
    r.l = r.l * a + l;
    r.o = r.o * a + o;
    r.m = m;
  } else {
    const float w = exp_nat(m - r.m);
    r.l += w * l;
    r.o += w * o;
  }
}

__device__ inline void write_final(const Run& r, int64_t row, int q4, uint16_t* out_bf16, float* out_f32,
                                   int64_t stride, float* lse) {
  const bool empty = !(r.l > 0.f);
  f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
  if (!empty) a = f32x4{r.o[0] / r.l, r.o[1] / r.l, r.o[2] / r.l, r.o[3] / r.l};
  if (out_bf16) {
    *(u32x2*)(out_bf16 + row * stride + 4 * q4) = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
  } else {
    *(f32x4*)(out_f32 + row * stride + 4 * q4) = a;
  }
  if (lse && q4 == 0) lse[row] = empty ? -INFINITY : r.m + logf(r.l);
}

// Slices per row for a given part count: a power of two, at most the slices
// of a workgroup, about one per 4 parts.
template <int D>
__host__ __device__ inline int splits_for(int n_parts) {
  constexpr int NS = kThreads / (D / 4);
  int s = 1;
  while (s < NS && s * 4 < n_parts) s *= 2;
  return s;
}

// Parts accessor for strided workspace partials.
struct StridedParts {
  const float* m;
  const float* l;
  const float* o;
  int64_t R;
  int D;
  __device__ inline float pm(int p, int64_t r) const { return m[p * R + r]; }
  __device__ inline float pl(int p, int64_t r) const { return l[p * R + r]; }
  __device__ inline f32x4 po(int p, int64_t r, int q4) const {
    return *(const f32x4*)(o + (p * R + r) * D + 4 * q4);
  }
};

// Parts accessor for a pointer table.
struct PtrParts {
  const MergePtrArgs* a;
  int D;
  __device__ inline float pm(int p, int64_t r) const { return a->m[p][r]; }
  __device__ inline float pl(int p, int64_t r) const { return a->l[p][r]; }
  __device__ inline f32x4 po(int p, int64_t r, int q4) const {
    return *(const f32x4*)(a->o[p] + r * D + 4 * q4);
  }
};

// Fold parts [p0, p1) with stride `step` of row r; loads batched 4 at a time.
template <class Parts>
__device__ inline void fold(Run& run, const Parts& P, int64_t r, int q4, int p0, int p1, int step) {
  int p = p0;
  for (; p + 3 * step < p1; p += 4 * step) {
    float m[4], l[4];
    f32x4 o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      m[u] = P.pm(p + u * step, r);
      l[u] = P.pl(p + u * step, r);
      o[u] = P.po(p + u * step, r, q4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) run_add(run, m[u], l[u], o[u]);
  }
  for (; p < p1; p += step) run_add(run, P.pm(p, r), P.pl(p, r), P.po(p, r, q4));
}

// Combine the `splits` slices of each row through LDS; slice 0 of a row ends
// with the merged state.  Returns true for the lanes that hold it.
template <int D>
__device__ inline bool combine(Run& run, int splits, int slice, int q4, float* sm) {
  constexpr int TPR = D / 4;
  constexpr int NS = kThreads / TPR;
  float* s_m = sm;
  float* s_l = sm + NS;
  f32x4* s_o = (f32x4*)(sm + 2 * NS);
  if (splits == 1) return true;
  if (q4 == 0) {
    s_m[slice] = run.m;
    s_l[slice] = run.l;
  }
  s_o[slice * TPR + q4] = run.o;
  __syncthreads();
  const int sub = slice % splits;
  if (sub != 0) return false;
  for (int k = 1; k < splits; ++k) run_add(run, s_m[slice + k], s_l[slice + k], s_o[(slice + k) * TPR + q4]);
  return true;
}

template <int D>
__global__ __launch_bounds__(kThreads) void merge_groups_kernel(MergeGroupArgs a) {
  constexpr int TPR = D / 4;
  constexpr int NS = kThreads / TPR;
  __shared__ __attribute__((aligned(16))) float sm[2 * NS + NS * D];
  const int gi = blockIdx.y;
  const int p0 = a.part_begin[gi];
  const int p1 = a.part_begin[gi + 1];
  const int splits = splits_for<D>(p1 - p0 + (a.has_init ? 1 : 0));
  const int rows_per_wg = NS / splits;
  const int slice = threadIdx.x / TPR;
  const int q4 = threadIdx.x % TPR;
  const int sub = slice % splits;
  const int64_t r_raw = (int64_t)blockIdx.x * rows_per_wg + slice / splits;
  const bool valid = r_raw < a.R;
  const int64_t r = valid ? r_raw : a.R - 1;
  StridedParts P{a.pm, a.pl, a.po, a.R, D};

  Run run;
  run_init(run);
  if (a.has_init && sub == 0) {
    const float mi = a.out_m[gi][r];
    if (mi != -INFINITY) run_add(run, mi, a.out_l[gi][r], *(const f32x4*)(a.out_o[gi] + r * D + 4 * q4));
  }
  fold(run, P, r, q4, p0 + sub, p1, splits);
  if (!combine<D>(run, splits, slice, q4, sm) || !valid) return;
  if (a.fin_out || a.fin_out_f32) {
    write_final(run, r, q4, a.fin_out, a.fin_out_f32, a.fin_stride ? a.fin_stride : D, a.fin_lse);
    return;
  }
  *(f32x4*)(a.out_o[gi] + r * D + 4 * q4) = run.o;
  if (q4 == 0) {
    a.out_m[gi][r] = run.m;
    a.out_l[gi][r] = run.l;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void merge_ptrs_kernel(MergePtrArgs a) {
  constexpr int TPR = D / 4;
  constexpr int NS = kThreads / TPR;
  __shared__ __attribute__((aligned(16))) float sm[2 * NS + NS * D];
  const int splits = splits_for<D>(a.n_parts);
  const int rows_per_wg = NS / splits;
  const int slice = threadIdx.x / TPR;
  const int q4 = threadIdx.x % TPR;
  const int sub = slice % splits;
  const int64_t r_raw = (int64_t)blockIdx.x * rows_per_wg + slice / splits;
  const bool valid = r_raw < a.R;
  const int64_t r = valid ? r_raw : a.R - 1;
  PtrParts P{&a, D};

  Run run;
  run_init(run);
  fold(run, P, r, q4, sub, a.n_parts, splits);
  // With several slices per row every read of every part happens before the
  // barrier inside combine(), so writing `out` afterwards is safe even when it
  // is one of the parts; with one slice per row the same lanes read then write.
  if (!combine<D>(run, splits, slice, q4, sm) || !valid) return;
  *(f32x4*)(a.out_o + r * D + 4 * q4) = run.o;
  if (q4 == 0) {
    a.out_m[r] = run.m;
    a.out_l[r] = run.l;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void finalize_kernel(FinalizeArgs a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = kThreads / TPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int q4 = threadIdx.x % TPR;
  if (r >= a.R) return;
  Run run;
  run.m = a.m[r];
  run.l = a.l[r];
  run.o = f32x4{0.f, 0.f, 0.f, 0.f};
  if (run.l > 0.f) run.o = *(const f32x4*)(a.o + r * D + 4 * q4);
  write_final(run, r, q4, a.out_bf16 ? (uint16_t*)a.out : nullptr, a.out_bf16 ? nullptr : (float*)a.out,
              a.out_stride, a.lse);
}

template <int D>
inline int merge_blocks(int64_t R, int n_parts) {
  constexpr int NS = kThreads / (D / 4);
  const int rows_per_wg = NS / splits_for<D>(n_parts);
  return (int)((R + rows_per_wg - 1) / rows_per_wg);
}

template <int D>
inline int finalize_blocks(int64_t R) {
  constexpr int RPB = kThreads / (D / 4);
  return (int)((R + RPB - 1) / RPB);
}

int max_group_parts(const MergeGroupArgs& a) {
  int mx = 0;
  for (int i = 0; i < a.n_groups; ++i) {
    int n = a.part_begin[i + 1] - a.part_begin[i] + (a.has_init ? 1 : 0);
    mx = n > mx ? n : mx;
  }
  return mx;
}

}  // namespace

// Groups share one grid only when they have the same part count (the kernel
// derives its row/slice layout from the count); otherwise one launch per group.
hipError_t launch_merge_groups(const MergeGroupArgs& a, int D, hipStream_t s) {
  bool uniform = true;
  for (int i = 1; i < a.n_groups; ++i)
    if (a.part_begin[i + 1] - a.part_begin[i] != a.part_begin[1] - a.part_begin[0]) uniform = false;
  if (!uniform) {
    for (int i = 0; i < a.n_groups; ++i) {
      MergeGroupArgs one = a;
      one.n_groups = 1;
      one.part_begin[0] = a.part_begin[i];
      one.part_begin[1] = a.part_begin[i + 1];
      one.out_m[0] = a.out_m[i];
      one.out_l[0] = a.out_l[i];
      one.out_o[0] = a.out_o[i];
      hipError_t e = launch_merge_groups(one, D, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int n = max_group_parts(a);
  if (D == 128)
    hipLaunchKernelGGL(merge_groups_kernel<128>, dim3(merge_blocks<128>(a.R, n), a.n_groups), dim3(kThreads), 0,
                       s, a);
  else
    hipLaunchKernelGGL(merge_groups_kernel<64>, dim3(merge_blocks<64>(a.R, n), a.n_groups), dim3(kThreads), 0,
                       s, a);
  return hipGetLastError();
}

hipError_t launch_merge_ptrs(const MergePtrArgs& a, int D, hipStream_t s) {
  if (D == 128)
    hipLaunchKernelGGL(merge_ptrs_kernel<128>, dim3(merge_blocks<128>(a.R, a.n_parts)), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(merge_ptrs_kernel<64>, dim3(merge_blocks<64>(a.R, a.n_parts)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, int D, hipStream_t s) {
  if (D == 128)
    hipLaunchKernelGGL(finalize_kernel<128>, dim3(finalize_blocks<128>(a.R)), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(finalize_kernel<64>, dim3(finalize_blocks<64>(a.R)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ba
