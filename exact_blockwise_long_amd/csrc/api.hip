// C-ABI front end of libblockattn.so: argument checks, work splitting and
// kernel dispatch.  Every check runs before anything is enqueued; the library
// allocates nothing and never synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "internal.h"

namespace {

thread_local char g_err[512] = "";

ba_status fail(ba_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ba_status ok() {
  g_err[0] = '\0';
  return BA_OK;
}

ba_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workgroups a split launch aims for: two per compute unit of a 256-CU part,
// one round (fastest for the bandwidth-bound shard sweep: 109 us against
// 126 us at 1024 and 132 us at 256).
constexpr int kTargetWorkgroups = 512;
// Below this many (row tile x KV head) workgroups the keys are split.
constexpr int kWalkMinWorkgroups = 512;
constexpr int kMaxChunks = 8192;

float resolve_scale(float s, int D) { return s > 0.f ? s : 1.0f / sqrtf((float)D); }

// Sequences of a problem (batch 0 or 1: one) and its state rows.
int batch_of(const ba_problem* p) { return p->batch > 1 ? p->batch : 1; }
int64_t state_rows(const ba_problem* p) { return (int64_t)batch_of(p) * p->q_len * p->n_q_heads; }

ba_status check_problem(const ba_problem* p, const void* q) {
  if (!p) return fail(BA_ERR_NULL, "problem is NULL");
  if (p->dtype != BA_F32 && p->dtype != BA_BF16) return fail(BA_ERR_UNSUPPORTED, "dtype %d", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(BA_ERR_SHAPE, "head_dim %d (64 or 128 supported)", p->head_dim);
  if (p->n_q_heads <= 0 || p->n_kv_heads <= 0 || p->n_q_heads % p->n_kv_heads != 0)
    return fail(BA_ERR_SHAPE, "n_q_heads %d must be a positive multiple of n_kv_heads %d", p->n_q_heads,
                p->n_kv_heads);
  if (p->q_len < 0) return fail(BA_ERR_SHAPE, "q_len %d < 0", p->q_len);
  if (p->batch < 0) return fail(BA_ERR_SHAPE, "batch %d < 0", p->batch);
  if (state_rows(p) > (int64_t)1 << 30) return fail(BA_ERR_SHAPE, "too many query rows");
  if (p->q_len > 0) {
    if (!q) return fail(BA_ERR_NULL, "q is NULL");
    if (p->q_stride_token <= 0 || p->q_stride_head <= 0) return fail(BA_ERR_SHAPE, "q strides must be positive");
    if (p->batch > 1 && p->q_stride_batch <= 0) return fail(BA_ERR_SHAPE, "q_stride_batch must be positive");
    if (p->dtype == BA_BF16) {
      if (((uintptr_t)q % 16) != 0) return fail(BA_ERR_SHAPE, "q not 16-byte aligned");
      if (p->q_stride_token % 8 != 0 || p->q_stride_head % 8 != 0 || (p->batch > 1 && p->q_stride_batch % 8 != 0))
        return fail(BA_ERR_SHAPE, "bf16 q strides must be multiples of 8 elements");
    }
  }
  if (p->split_mode < 0 || p->split_mode > 2) return fail(BA_ERR_SHAPE, "split_mode %d", p->split_mode);
  return BA_OK;
}

// Bytes one KV head of `len` keys spans at `stride_token` bf16 elements per key.
int64_t head_extent_bf16(int64_t len, int64_t stride_token, int head_dim) {
  return len <= 0 ? 0 : ((len - 1) * stride_token + head_dim) * 2;
}

ba_status check_block(const ba_kv_block& b, int i, const ba_problem* p) {
  const int dtype = p->dtype, head_dim = p->head_dim;
  const bool batched = p->batch > 1;
  if (b.len < 0) return fail(BA_ERR_SHAPE, "block %d: len %d < 0", i, b.len);
  if (b.len == 0) return BA_OK;
  if (!b.k || !b.v) return fail(BA_ERR_NULL, "block %d: k or v is NULL", i);
  if (b.k_stride_token <= 0 || b.k_stride_head <= 0 || b.v_stride_token <= 0 || b.v_stride_head <= 0)
    return fail(BA_ERR_SHAPE, "block %d: strides must be positive", i);
  if (batched && (b.k_stride_batch < 0 || b.v_stride_batch < 0))
    return fail(BA_ERR_SHAPE, "block %d: batch strides must be >= 0", i);
  if (dtype == BA_BF16) {
    if (((uintptr_t)b.k % 16) != 0 || ((uintptr_t)b.v % 16) != 0)
      return fail(BA_ERR_SHAPE, "block %d: k/v not 16-byte aligned", i);
    if (b.k_stride_token % 8 || b.k_stride_head % 8 || b.v_stride_token % 8 || b.v_stride_head % 8 ||
        (batched && (b.k_stride_batch % 8 || b.v_stride_batch % 8)))
      return fail(BA_ERR_SHAPE, "block %d: bf16 strides must be multiples of 8 elements", i);
    // The tile loads' range check ends a block after its last key only when
    // one key's row does not run into the next key's.
    if (b.k_stride_token < head_dim || b.v_stride_token < head_dim)
      return fail(BA_ERR_SHAPE, "block %d: bf16 token strides must be >= head_dim", i);
    // The bf16 kernels read one KV head of a block through a buffer resource
    // with 32-bit byte offsets.
    if (head_extent_bf16(b.len, b.k_stride_token, head_dim) > (int64_t)UINT32_MAX ||
        head_extent_bf16(b.len, b.v_stride_token, head_dim) > (int64_t)UINT32_MAX)
      return fail(BA_ERR_SHAPE, "block %d: one KV head spans 4 GiB or more (bf16 kernels use 32-bit offsets)", i);
  }
  return BA_OK;
}

ba_status check_state(const ba_state& s, const char* what) {
  if (!s.m || !s.l || !s.o) return fail(BA_ERR_NULL, "%s: m, l or o is NULL", what);
  if (((uintptr_t)s.o % 16) != 0) return fail(BA_ERR_SHAPE, "%s: o not 16-byte aligned", what);
  return BA_OK;
}

// Resolved visit list.
struct Visits {
  std::vector<int> idx;
};

ba_status resolve_order(int n_blocks, const int32_t* order, int n_visit, Visits& v) {
  if (n_visit < 0) return fail(BA_ERR_ORDER, "n_visit %d < 0", n_visit);
  if (n_visit > BLOCKATTN_MAX_VISITS)
    return fail(BA_ERR_ORDER, "n_visit %d > %d per call", n_visit, BLOCKATTN_MAX_VISITS);
  if (n_visit > n_blocks) return fail(BA_ERR_ORDER, "n_visit %d > n_blocks %d", n_visit, n_blocks);
  std::vector<char> seen(n_blocks > 0 ? n_blocks : 1, 0);
  v.idx.clear();
  for (int t = 0; t < n_visit; ++t) {
    int j = order ? order[t] : t;
    if (j < 0 || j >= n_blocks) return fail(BA_ERR_ORDER, "order[%d] = %d out of range [0, %d)", t, j, n_blocks);
    if (seen[j]) return fail(BA_ERR_ORDER, "order[%d] = %d repeats a block", t, j);
    seen[j] = 1;
    v.idx.push_back(j);
  }
  return BA_OK;
}

ba::QSide make_qside(const ba_problem* p, const void* q) {
  ba::QSide qs;
  qs.q = q;
  qs.qs_t = p->q_stride_token;
  qs.qs_h = p->q_stride_head;
  qs.B = batch_of(p);
  qs.qs_b = qs.B > 1 ? p->q_stride_batch : 0;
  qs.q_pos0 = p->q_pos0;
  qs.Hq = p->n_q_heads;
  qs.Hkv = p->n_kv_heads;
  qs.G = p->n_q_heads / p->n_kv_heads;
  qs.q_len = p->q_len;
  qs.c = resolve_scale(p->scale, p->head_dim) * ba::kLog2e;
  qs.causal = p->causal ? 1 : 0;
  return qs;
}

// `batch`: the problem's sequences; the block's batch strides count only for
// more than one.
ba::Seg make_seg(const ba_kv_block& b, int batch) {
  ba::Seg s;
  s.k = b.k;
  s.v = b.v;
  s.ks_t = b.k_stride_token;
  s.ks_h = b.k_stride_head;
  s.vs_t = b.v_stride_token;
  s.vs_h = b.v_stride_head;
  s.ks_b = batch > 1 ? b.k_stride_batch : 0;
  s.vs_b = batch > 1 ? b.v_stride_batch : 0;
  s.pos0 = b.pos0;
  s.n = b.len;
  s.pad_ = 0;
  return s;
}

// Keys of a block some query of the whole block can see.
int64_t usable_keys(const ba_problem* p, const ba_kv_block& b) {
  if (!p->causal || p->q_len == 0) return b.len;
  int64_t qmax = p->q_pos0 + p->q_len - 1;
  int64_t lim = qmax - b.pos0 + 1;
  if (lim <= 0) return 0;
  return lim < b.len ? lim : b.len;
}

int row_tiles(const ba_problem* p) {
  int64_t flat = (int64_t)p->q_len * (p->n_q_heads / p->n_kv_heads);
  return (int)((flat + ba::kTileRows - 1) / ba::kTileRows) * p->n_kv_heads * batch_of(p);
}

// Row tiling of a split launch.  More than one 128-row tile per KV head makes
// it matrix-core bound: it then runs 8-wave workgroups of 256-row tiles, one
// per compute unit, aiming for half as many workgroups (as the walk and the
// fan-out do).  One tile per KV head stays on 4-wave workgroups.
struct SplitGeom {
  bool wide = false;
  int tiles = 0;       // row tiles x KV heads x sequences
  int target = 0;      // workgroups the planner aims for
  int key_align = 64;  // chunk lengths are multiples of this
  int min_chunk = 256;
};

// Rows per workgroup of the fp32 walk and its split form (one wave).
constexpr int kF32TileRows = 64;

int f32_row_tiles(const ba_problem* p) {
  int64_t flat = (int64_t)p->q_len * (p->n_q_heads / p->n_kv_heads);
  return (int)((flat + kF32TileRows - 1) / kF32TileRows) * p->n_kv_heads * batch_of(p);
}

SplitGeom split_geom(const ba_problem* p) {
  SplitGeom sg;
  if (p->dtype == BA_F32) {
    // One-wave workgroups over 32-key LDS tiles: aim for four per compute unit.
    sg.tiles = f32_row_tiles(p);
    sg.target = 2 * kTargetWorkgroups;
    sg.key_align = 32;
    sg.min_chunk = 32;
    return sg;
  }
  const int64_t flat = (int64_t)p->q_len * (p->n_q_heads / p->n_kv_heads);
  const int64_t narrow = (flat + ba::kTileRows - 1) / ba::kTileRows;
  sg.wide = BA_SPLIT_WIDE && narrow >= 2;
  const int64_t per_head = sg.wide ? (flat + ba::kWideTileRows - 1) / ba::kWideTileRows : narrow;
  sg.tiles = (int)per_head * p->n_kv_heads * batch_of(p);
  sg.target = sg.wide ? kTargetWorkgroups / 2 : kTargetWorkgroups;
  return sg;
}

// Split plan: chunk length and per-visit chunk offsets.
struct SplitPlan {
  bool wide = false;
  int chunk_len = 0;
  int n_chunks = 0;
  std::vector<int> begin;  // size n_seg + 1
};

SplitPlan plan_split(const std::vector<int64_t>& keys, const SplitGeom& geom) {
  SplitPlan sp;
  sp.wide = geom.wide;
  const int tiles = geom.tiles;
  int64_t total = 0;
  for (int64_t k : keys) total += k;
  int64_t want = (geom.target + tiles - 1) / (tiles > 0 ? tiles : 1);
  if (want < 1) want = 1;
  int64_t cl = (total + want - 1) / want;
  cl = (cl + geom.key_align - 1) / geom.key_align * geom.key_align;
  if (cl < geom.min_chunk) cl = geom.min_chunk;
  for (;;) {
    int64_t n = 0;
    for (int64_t k : keys) n += (k + cl - 1) / cl;
    if (n <= kMaxChunks) break;
    cl *= 2;
  }
  sp.chunk_len = (int)cl;
  sp.begin.push_back(0);
  for (int64_t k : keys) {
    sp.n_chunks += (int)((k + cl - 1) / cl);
    sp.begin.push_back(sp.n_chunks);
  }
  return sp;
}

size_t partial_bytes(int64_t slots, int64_t R, int D) {
  size_t ml = align_up((size_t)slots * R * sizeof(float));
  return 2 * ml + align_up((size_t)slots * R * D * sizeof(float));
}

void partial_ptrs(void* ws, int64_t slots, int64_t R, float** m, float** l, float** o) {
  size_t ml = align_up((size_t)slots * R * sizeof(float));
  char* b = (char*)ws;
  *m = (float*)b;
  *l = (float*)(b + ml);
  *o = (float*)(b + 2 * ml);
}

bool fwd_uses_split(const ba_problem* p) {
  if (p->split_mode == 1) return false;
  if (p->split_mode == 2) return true;
  return (p->dtype == BA_F32 ? f32_row_tiles(p) : row_tiles(p)) < kWalkMinWorkgroups;
}

hipError_t launch_split(const ba_problem* p, const ba::SplitArgs& a, int n_chunks, hipStream_t stream) {
  return p->dtype == BA_F32 ? ba::launch_split_f32(a, n_chunks, p->head_dim, stream)
                            : ba::launch_split_bf16(a, n_chunks, p->head_dim, stream);
}

// Full validation of a forward call; fills the visit list and split plan.
ba_status prepare_fwd(const ba_problem* p, const void* q, const ba_kv_block* blocks, int n_blocks,
                      const int32_t* order, int n_visit, Visits& v, SplitPlan& sp, bool& split) {
  ba_status st = check_problem(p, q);
  if (st) return st;
  if (n_blocks < 0) return fail(BA_ERR_SHAPE, "n_blocks %d < 0", n_blocks);
  if (n_visit > 0 && !blocks) return fail(BA_ERR_NULL, "blocks is NULL");
  st = resolve_order(n_blocks, order, n_visit, v);
  if (st) return st;
  for (int j : v.idx) {
    st = check_block(blocks[j], j, p);
    if (st) return st;
  }
  split = fwd_uses_split(p);
  if (split) {
    std::vector<int64_t> keys;
    for (int j : v.idx) keys.push_back(usable_keys(p, blocks[j]));
    sp = plan_split(keys, split_geom(p));
  }
  return BA_OK;
}

// Where a forward call that finalises writes: A rows of out_row_stride
// elements (bf16 or fp32) and, optionally, the rows' log-sum-exp.
struct FinOut {
  void* out = nullptr;
  int32_t dtype = BA_BF16;
  int64_t stride = 0;
  float* lse = nullptr;
};

// The same checks as blockattn_finalize applies to its output.
ba_status check_fin(const FinOut& f, int head_dim) {
  if (!f.out) return fail(BA_ERR_NULL, "out is NULL");
  if (f.dtype != BA_F32 && f.dtype != BA_BF16) return fail(BA_ERR_UNSUPPORTED, "out_dtype %d", f.dtype);
  if (f.stride < head_dim) return fail(BA_ERR_SHAPE, "out_row_stride %lld < head_dim", (long long)f.stride);
  if (f.stride % 4 != 0) return fail(BA_ERR_SHAPE, "out_row_stride must be a multiple of 4");
  if (((uintptr_t)f.out % (f.dtype == BA_BF16 ? 8 : 16)) != 0) return fail(BA_ERR_SHAPE, "out misaligned");
  return BA_OK;
}

ba_status finalize_run(ba_state s, int64_t rows, int head_dim, const FinOut& f, hipStream_t stream) {
  ba::FinalizeArgs a;
  a.m = s.m;
  a.l = s.l;
  a.o = s.o;
  a.R = rows;
  a.out = f.out;
  a.out_bf16 = f.dtype == BA_BF16;
  a.out_stride = f.stride;
  a.lse = f.lse;
  return hip_status(ba::launch_finalize(a, head_dim, stream), "finalize launch");
}

// The visits of one forward call: update the state, or (fin set) end with the
// finalised output instead.  Everything is validated before the first launch.
ba_status fwd_run(const ba_problem* p, const void* q, const ba_kv_block* blocks, int32_t n_blocks,
                  const int32_t* order, int32_t n_visit, ba_state state, int32_t reset_state, const FinOut* fin,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Visits v;
  SplitPlan sp;
  bool split = false;
  ba_status st = prepare_fwd(p, q, blocks, n_blocks, order, n_visit, v, sp, split);
  if (st) return st;
  if (p->q_len == 0) return ok();
  st = check_state(state, "state");
  if (st) return st;
  if (fin) {
    st = check_fin(*fin, p->head_dim);
    if (st) return st;
  }
  const int D = p->head_dim;
  const int64_t R = state_rows(p);
  const size_t need = split ? partial_bytes(sp.n_chunks, R, D) : 0;
  if (split && sp.n_chunks > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(BA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (((uintptr_t)workspace % 16) != 0) return fail(BA_ERR_WORKSPACE, "workspace not 16-byte aligned");
  }

  if (!split) {
    ba::WalkArgs a;
    memset(&a, 0, sizeof(a));
    a.qs = make_qside(p, q);
    a.m = state.m;
    a.l = state.l;
    a.o = state.o;
    a.reset = reset_state ? 1 : 0;
    a.n_seg = 0;
    for (int j : v.idx) {
      // blocks no query of the block can see (causal future, or empty) are skipped
      if (usable_keys(p, blocks[j]) == 0) continue;
      a.seg[a.n_seg++] = make_seg(blocks[j], batch_of(p));
    }
    if (fin && p->dtype != BA_BF16) {
      // The fp32 walk keeps the state; finalisation follows as its own launch.
      if (a.reset || a.n_seg > 0) {
        hipError_t e = ba::launch_walk_f32(a, D, stream);
        if (e != hipSuccess) return hip_status(e, "fwd_block walk launch");
      }
      return finalize_run(state, R, D, *fin, stream);
    }
    if (fin) {
      a.fin_out = fin->out;
      a.fin_bf16 = fin->dtype == BA_BF16 ? 1 : 0;
      a.fin_stride = fin->stride;
      a.fin_lse = fin->lse;
    } else if (!a.reset && a.n_seg == 0) {
      return ok();
    }
    hipError_t e = (p->dtype == BA_BF16) ? ba::launch_walk_bf16(a, D, stream) : ba::launch_walk_f32(a, D, stream);
    return hip_status(e, "fwd_block walk launch");
  }

  float *wm = nullptr, *wl = nullptr, *wo = nullptr;
  if (sp.n_chunks > 0) {
    partial_ptrs(workspace, sp.n_chunks, R, &wm, &wl, &wo);
    ba::SplitArgs a;
    memset(&a, 0, sizeof(a));
    a.qs = make_qside(p, q);
    a.ws_m = wm;
    a.ws_l = wl;
    a.ws_o = wo;
    a.R = R;
    a.chunk_len = sp.chunk_len;
    a.wide = sp.wide ? 1 : 0;
    a.n_seg = (int)v.idx.size();
    for (int i = 0; i < a.n_seg; ++i) {
      a.seg[i] = make_seg(blocks[v.idx[i]], batch_of(p));
      a.chunk_begin[i] = sp.begin[i];
    }
    a.chunk_begin[a.n_seg] = sp.begin[a.n_seg];
    hipError_t e = launch_split(p, a, sp.n_chunks, stream);
    if (e != hipSuccess) return hip_status(e, "fwd_block split launch");
  }
  if (!fin && !reset_state && sp.n_chunks == 0) return ok();
  ba::MergeGroupArgs mg;
  memset(&mg, 0, sizeof(mg));
  mg.pm = wm;
  mg.pl = wl;
  mg.po = wo;
  mg.R = R;
  mg.n_groups = 1;
  mg.has_init = reset_state ? 0 : 1;
  mg.part_begin[0] = 0;
  mg.part_begin[1] = sp.n_chunks;
  mg.out_m[0] = state.m;
  mg.out_l[0] = state.l;
  mg.out_o[0] = state.o;
  if (fin) {
    if (fin->dtype == BA_BF16)
      mg.fin_out = (uint16_t*)fin->out;
    else
      mg.fin_out_f32 = (float*)fin->out;
    mg.fin_stride = fin->stride;
    mg.fin_lse = fin->lse;
  }
  return hip_status(ba::launch_merge_groups(mg, D, stream), "fwd_block merge launch");
}

}  // namespace

extern "C" {

const char* blockattn_status_str(int32_t s) {
  switch (s) {
    case BA_OK: return "ok";
    case BA_ERR_NULL: return "a required pointer is NULL";
    case BA_ERR_SHAPE: return "inconsistent or out-of-range sizes or strides";
    case BA_ERR_UNSUPPORTED: return "unsupported request";
    case BA_ERR_ORDER: return "invalid visit order";
    case BA_ERR_WORKSPACE: return "workspace missing or too small";
    case BA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* blockattn_last_error(void) { return g_err; }

int32_t blockattn_abi_version(void) { return BLOCKATTN_ABI_VERSION; }

size_t blockattn_fwd_workspace_bytes(const ba_problem* p, const ba_kv_block* blocks, int32_t n_blocks,
                                     const int32_t* order, int32_t n_visit) {
  Visits v;
  SplitPlan sp;
  bool split = false;
  if (prepare_fwd(p, p ? (const void*)256 : nullptr, blocks, n_blocks, order, n_visit, v, sp, split) != BA_OK)
    return 0;
  if (!split || p->q_len == 0) return 0;
  return partial_bytes(sp.n_chunks, state_rows(p), p->head_dim);
}

ba_status blockattn_fwd_block(const ba_problem* p, const void* q, const ba_kv_block* blocks, int32_t n_blocks,
                              const int32_t* order, int32_t n_visit, ba_state state, int32_t reset_state,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fwd_run(p, q, blocks, n_blocks, order, n_visit, state, reset_state, nullptr, workspace, workspace_bytes,
                 stream);
}

ba_status blockattn_fwd_block_finalize(const ba_problem* p, const void* q, const ba_kv_block* blocks,
                                       int32_t n_blocks, const int32_t* order, int32_t n_visit, ba_state state,
                                       int32_t reset_state, void* out, int32_t out_dtype, int64_t out_row_stride,
                                       float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  FinOut fin;
  fin.out = out;
  fin.dtype = out_dtype;
  fin.stride = out_row_stride;
  fin.lse = lse;
  return fwd_run(p, q, blocks, n_blocks, order, n_visit, state, reset_state, &fin, workspace, workspace_bytes,
                 stream);
}

ba_status blockattn_bwd_delta(int64_t rows, int32_t head_dim, const void* out, int32_t out_dtype,
                              int64_t out_row_stride, const void* dout, int64_t dout_row_stride, float* delta,
                              hipStream_t stream) {
  if (head_dim != 64 && head_dim != 128) return fail(BA_ERR_SHAPE, "head_dim %d", head_dim);
  if (rows < 0) return fail(BA_ERR_SHAPE, "rows %lld < 0", (long long)rows);
  if (out_dtype != BA_BF16 && out_dtype != BA_F32) return fail(BA_ERR_UNSUPPORTED, "out dtype %d", out_dtype);
  if (rows == 0) return ok();
  if (!out || !dout || !delta) return fail(BA_ERR_NULL, "out, dout or delta is NULL");
  if (out_row_stride < head_dim || dout_row_stride < head_dim)
    return fail(BA_ERR_SHAPE, "row strides must be >= head_dim");
  if (out_row_stride % 8 != 0 || dout_row_stride % 8 != 0)
    return fail(BA_ERR_SHAPE, "row strides must be multiples of 8 elements");
  if (((uintptr_t)out % 16) != 0 || ((uintptr_t)dout % 16) != 0) return fail(BA_ERR_SHAPE, "out/dout not 16-byte aligned");
  ba::DeltaArgs a;
  memset(&a, 0, sizeof(a));
  a.rows = rows;
  a.out = out;
  a.out_bf16 = out_dtype == BA_BF16 ? 1 : 0;
  a.out_stride = out_row_stride;
  a.dout = dout;
  a.dout_stride = dout_row_stride;
  a.delta = delta;
  return hip_status(ba::launch_delta(a, head_dim, stream), "bwd_delta launch");
}

ba_status blockattn_bwd_block(const ba_problem* p, const void* q, const void* dout, const float* lse,
                              const float* delta, const ba_kv_block* blocks, int32_t n_blocks, const int32_t* order,
                              int32_t n_visit, float* dq, float* const* dk, float* const* dv, hipStream_t stream) {
  ba_status st = check_problem(p, q);
  if (st) return st;
  if (p->dtype != BA_BF16) return fail(BA_ERR_UNSUPPORTED, "the backward pass is bf16 only");
  if (n_blocks < 0) return fail(BA_ERR_SHAPE, "n_blocks %d < 0", n_blocks);
  if (n_visit > 0 && !blocks) return fail(BA_ERR_NULL, "blocks is NULL");
  Visits v;
  st = resolve_order(n_blocks, order, n_visit, v);
  if (st) return st;
  for (int j : v.idx) {
    st = check_block(blocks[j], j, p);
    if (st) return st;
  }
  if (p->q_len == 0 || v.idx.empty()) return ok();
  if (!dout || !lse || !delta || !dq) return fail(BA_ERR_NULL, "dout, lse, delta or dq is NULL");
  if (((uintptr_t)dout % 16) != 0 || ((uintptr_t)dq % 16) != 0) return fail(BA_ERR_SHAPE, "dout/dq not 16-byte aligned");
  if (!dk || !dv) return fail(BA_ERR_NULL, "dk or dv pointer array is NULL");
  const int D = p->head_dim;
  const int64_t q_extent =
      ((int64_t)(p->q_len - 1) * p->q_stride_token + (int64_t)(p->n_q_heads - 1) * p->q_stride_head + D) * 2;
  const int64_t seq_rows = (int64_t)p->q_len * p->n_q_heads;   // one sequence's lse and delta rows
  if (q_extent > (int64_t)UINT32_MAX || seq_rows * 4 > (int64_t)UINT32_MAX)
    return fail(BA_ERR_SHAPE, "the backward pass addresses a sequence's q, dout, lse and delta with 32-bit offsets");
  ba::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.qs = make_qside(p, q);
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.scale = a.qs.c / ba::kLog2e;
  a.q_bytes = (uint32_t)q_extent;
  a.rows_bytes = (uint32_t)(seq_rows * 4);
  a.g_magic = 0xFFFFFFFFu / (uint32_t)a.qs.G;
  a.n_seg = 0;
  int tiles = 0;
  // Blocks in key-position order: under the causal rule the earliest keys
  // are seen by the most rows, so the dK/dV grid hands out its longest
  // workgroups first.  The gradients are sums over blocks; the order only
  // changes rounding.
  std::vector<int> by_pos(v.idx.begin(), v.idx.end());
  std::stable_sort(by_pos.begin(), by_pos.end(), [&](int x, int y) { return blocks[x].pos0 < blocks[y].pos0; });
  for (int j : by_pos) {
    if (usable_keys(p, blocks[j]) == 0) continue;   // causal future or empty: no gradient terms
    if (!dk[j] || !dv[j]) return fail(BA_ERR_NULL, "dk or dv of visited block %d is NULL", j);
    if (((uintptr_t)dk[j] % 16) != 0 || ((uintptr_t)dv[j] % 16) != 0)
      return fail(BA_ERR_SHAPE, "dk/dv of block %d not 16-byte aligned", j);
    a.seg[a.n_seg] = make_seg(blocks[j], batch_of(p));
    a.dk[a.n_seg] = dk[j];
    a.dv[a.n_seg] = dv[j];
    a.tile_begin[a.n_seg] = tiles;
    tiles += (int)((blocks[j].len + ba::kDkvKeys - 1) / ba::kDkvKeys);
    ++a.n_seg;
  }
  a.tile_begin[a.n_seg] = tiles;
  if (a.n_seg == 0) return ok();
  return hip_status(ba::launch_bwd_bf16(a, tiles, D, stream), "bwd_block launch");
}

size_t blockattn_shard_workspace_bytes(const ba_problem* p, const ba_kv_block* blocks, int32_t n_blocks) {
  if (check_problem(p, (const void*)256) != BA_OK || !blocks || n_blocks <= 0 || n_blocks > BLOCKATTN_MAX_VISITS)
    return 0;
  if (p->q_len == 0) return 0;
  std::vector<int64_t> keys;
  for (int i = 0; i < n_blocks; ++i) {
    if (check_block(blocks[i], i, p) != BA_OK) return 0;
    keys.push_back(usable_keys(p, blocks[i]));
  }
  SplitPlan sp = plan_split(keys, split_geom(p));
  return partial_bytes(sp.n_chunks, state_rows(p), p->head_dim);
}

ba_status blockattn_shard_states(const ba_problem* p, const void* q, const ba_kv_block* blocks, int32_t n_blocks,
                                 const ba_state* states_out, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  ba_status st = check_problem(p, q);
  if (st) return st;
  if (n_blocks <= 0 || n_blocks > BLOCKATTN_MAX_VISITS)
    return fail(BA_ERR_ORDER, "n_blocks %d outside [1, %d]", n_blocks, BLOCKATTN_MAX_VISITS);
  if (!blocks || !states_out) return fail(BA_ERR_NULL, "blocks or states_out is NULL");
  std::vector<int64_t> keys;
  for (int i = 0; i < n_blocks; ++i) {
    st = check_block(blocks[i], i, p);
    if (st) return st;
    st = check_state(states_out[i], "states_out");
    if (st) return st;
    keys.push_back(usable_keys(p, blocks[i]));
  }
  if (p->q_len == 0) return ok();
  const int D = p->head_dim;
  const int64_t R = state_rows(p);
  SplitPlan sp = plan_split(keys, split_geom(p));
  const size_t need = partial_bytes(sp.n_chunks, R, D);
  float *wm = nullptr, *wl = nullptr, *wo = nullptr;
  if (sp.n_chunks > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(BA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (((uintptr_t)workspace % 16) != 0) return fail(BA_ERR_WORKSPACE, "workspace not 16-byte aligned");
    partial_ptrs(workspace, sp.n_chunks, R, &wm, &wl, &wo);
    ba::SplitArgs a;
    memset(&a, 0, sizeof(a));
    a.qs = make_qside(p, q);
    a.ws_m = wm;
    a.ws_l = wl;
    a.ws_o = wo;
    a.R = R;
    a.chunk_len = sp.chunk_len;
    a.wide = sp.wide ? 1 : 0;
    a.n_seg = n_blocks;
    for (int i = 0; i < n_blocks; ++i) {
      a.seg[i] = make_seg(blocks[i], batch_of(p));
      a.chunk_begin[i] = sp.begin[i];
    }
    a.chunk_begin[n_blocks] = sp.begin[n_blocks];
    hipError_t e = launch_split(p, a, sp.n_chunks, stream);
    if (e != hipSuccess) return hip_status(e, "shard_states split launch");
  }
  ba::MergeGroupArgs mg;
  memset(&mg, 0, sizeof(mg));
  mg.pm = wm;
  mg.pl = wl;
  mg.po = wo;
  mg.R = R;
  mg.n_groups = n_blocks;
  mg.has_init = 0;
  for (int i = 0; i <= n_blocks; ++i) mg.part_begin[i] = sp.begin[i];
  for (int i = 0; i < n_blocks; ++i) {
    mg.out_m[i] = states_out[i].m;
    mg.out_l[i] = states_out[i].l;
    mg.out_o[i] = states_out[i].o;
  }
  return hip_status(ba::launch_merge_groups(mg, D, stream), "shard_states merge launch");
}

ba_status blockattn_merge_states(int32_t n_parts, const ba_state* parts, int64_t rows, int32_t head_dim,
                                 ba_state out, hipStream_t stream) {
  if (n_parts < 1 || n_parts > BLOCKATTN_MAX_MERGE_PARTS)
    return fail(BA_ERR_SHAPE, "n_parts %d outside [1, %d]", n_parts, BLOCKATTN_MAX_MERGE_PARTS);
  if (!parts) return fail(BA_ERR_NULL, "parts is NULL");
  if (head_dim != 64 && head_dim != 128) return fail(BA_ERR_SHAPE, "head_dim %d", head_dim);
  if (rows < 0) return fail(BA_ERR_SHAPE, "rows %lld < 0", (long long)rows);
  ba_status st = check_state(out, "out");
  if (st) return st;
  ba::MergePtrArgs a;
  memset(&a, 0, sizeof(a));
  a.n_parts = n_parts;
  a.R = rows;
  for (int i = 0; i < n_parts; ++i) {
    st = check_state(parts[i], "parts");
    if (st) return st;
    if (((uintptr_t)parts[i].o % 16) != 0) return fail(BA_ERR_SHAPE, "parts[%d].o not 16-byte aligned", i);
    a.m[i] = parts[i].m;
    a.l[i] = parts[i].l;
    a.o[i] = parts[i].o;
  }
  if (((uintptr_t)out.o % 16) != 0) return fail(BA_ERR_SHAPE, "out.o not 16-byte aligned");
  if (rows == 0) return ok();
  a.out_m = out.m;
  a.out_l = out.l;
  a.out_o = out.o;
  return hip_status(ba::launch_merge_ptrs(a, head_dim, stream), "merge_states launch");
}

ba_status blockattn_finalize(ba_state s, int64_t rows, int32_t head_dim, void* out, int32_t out_dtype,
                             int64_t out_row_stride, float* lse, hipStream_t stream) {
  ba_status st = check_state(s, "state");
  if (st) return st;
  if (!out) return fail(BA_ERR_NULL, "out is NULL");
  if (head_dim != 64 && head_dim != 128) return fail(BA_ERR_SHAPE, "head_dim %d", head_dim);
  if (rows < 0) return fail(BA_ERR_SHAPE, "rows < 0");
  if (out_dtype != BA_F32 && out_dtype != BA_BF16) return fail(BA_ERR_UNSUPPORTED, "out_dtype %d", out_dtype);
  if (out_row_stride < head_dim) return fail(BA_ERR_SHAPE, "out_row_stride %lld < head_dim", (long long)out_row_stride);
  if (out_row_stride % 4 != 0) return fail(BA_ERR_SHAPE, "out_row_stride must be a multiple of 4");
  if (((uintptr_t)s.o % 16) != 0) return fail(BA_ERR_SHAPE, "state o not 16-byte aligned");
  if (((uintptr_t)out % (out_dtype == BA_BF16 ? 8 : 16)) != 0) return fail(BA_ERR_SHAPE, "out misaligned");
  if (rows == 0) return ok();
  ba::FinalizeArgs a;
  a.m = s.m;
  a.l = s.l;
  a.o = s.o;
  a.R = rows;
  a.out = out;
  a.out_bf16 = out_dtype == BA_BF16;
  a.out_stride = out_row_stride;
  a.lse = lse;
  return hip_status(ba::launch_finalize(a, head_dim, stream), "finalize launch");
}

}  // extern "C"

namespace {

// Fan-out shapes shared by decode (one new token per branch) and prefill
// (the last T tokens of every branch's private suffix).
struct FanoutShape {
  int nb = 0, T = 1, Hq = 0, Hkv = 0, D = 0, P = 0, S = 0;
  float scale = 0.f;
};

ba_status check_fanout_shape(const FanoutShape& f) {
  if (f.D != 64 && f.D != 128) return fail(BA_ERR_SHAPE, "head_dim %d", f.D);
  if (f.Hq <= 0 || f.Hkv <= 0 || f.Hq % f.Hkv != 0)
    return fail(BA_ERR_SHAPE, "bad head counts %d / %d", f.Hq, f.Hkv);
  if (f.nb < 0 || f.P < 0 || f.S < 0) return fail(BA_ERR_SHAPE, "negative size");
  if (f.nb > 0 && f.P + f.S == 0) return fail(BA_ERR_SHAPE, "no keys to attend to");
  if ((int64_t)f.nb * f.T * f.Hq > ((int64_t)1 << 31) / 2) return fail(BA_ERR_SHAPE, "too many query rows");
  return BA_OK;
}

ba_status check_fanout(const ba_fanout* f) {
  if (!f) return fail(BA_ERR_NULL, "fanout descriptor is NULL");
  FanoutShape s;
  s.nb = f->n_branches;
  s.Hq = f->n_q_heads;
  s.Hkv = f->n_kv_heads;
  s.D = f->head_dim;
  s.P = f->prefix_len;
  s.S = f->suffix_len;
  return check_fanout_shape(s);
}

struct FanoutPlan {
  bool wide = false;   // 8-wave workgroups, 256-row tiles
  int row_tiles = 0;   // row tiles of one KV head's rows (n_branches * T * G)
  int chunk_len = 0;
  int n_chunks = 0;    // prefix chunks
  int srt = 1;         // row tiles of one branch's rows (T * G)
  int bpj = 1;         // branches per suffix job (when a branch's rows fit one tile)
  int suffix_jobs = 0;
  int slots = 0;       // workspace partial slots
  int suffix_slot = -1;
  int n_jobs = 0;
};

// The launch is sized to about kFanoutTargetWorkgroups jobs that each walk
// about the same number of (row tile, key) pairs, so no compute unit idles
// while others still work: a job's time is its K/V bytes over its share of
// HBM for a decode and its tile-key pairs over its share of the matrix cores
// for a prefill, both proportional to the keys a row tile walks.  Suffix jobs
// far shorter than that are not counted against the target.  A suffix job
// walks bpj branches' private suffixes of one KV head one after another (or
// one row tile of one branch when a branch has more than one); a prefix job
// walks one chunk of the shared prefix for one row tile of a KV head.
FanoutPlan plan_fanout_tiles(const FanoutShape& f, int tile_rows, int target, int key_align) {
  FanoutPlan fp;
  const int G = f.Hq / f.Hkv;
  const int64_t rows = (int64_t)f.nb * f.T * G;
  fp.row_tiles = (int)((rows + tile_rows - 1) / tile_rows);
  fp.srt = (int)(((int64_t)f.T * G + tile_rows - 1) / tile_rows);
  const int xs = fp.row_tiles * f.Hkv;
  const int64_t keys_total =
      (int64_t)f.Hkv * ((int64_t)f.P * fp.row_tiles + (int64_t)f.nb * fp.srt * f.S);
  const int64_t per_job = keys_total / target > 1 ? keys_total / target : 1;
  if (f.S > 0) {
    if (fp.srt == 1) {
      int64_t bpj = (per_job + f.S / 2) / f.S;
      if (bpj > f.nb) bpj = f.nb;
      if (bpj < 1) bpj = 1;
      fp.bpj = (int)bpj;
      fp.suffix_jobs = f.Hkv * (int)((f.nb + fp.bpj - 1) / fp.bpj);
    } else {
      fp.suffix_jobs = f.Hkv * f.nb * fp.srt;
    }
  }
  if (f.P > 0) {
    // Suffix jobs much shorter than the average job (many new tokens per
    // branch against a short private suffix) run in the gaps the prefix jobs
    // leave; only comparable ones take prefix jobs' places in the launch.
    const int64_t suffix_job_keys = fp.srt == 1 ? (int64_t)fp.bpj * f.S : (int64_t)f.S;
    const bool suffix_small = f.S > 0 && 2 * suffix_job_keys < per_job;
    int64_t want = (target - (suffix_small ? 0 : fp.suffix_jobs)) / xs;
    if (want < 1) want = 1;
    int64_t cl = (f.P + want - 1) / want;
    cl = (cl + key_align - 1) / key_align * key_align;
    if (cl < 256) cl = 256;
    fp.chunk_len = (int)cl;
    fp.n_chunks = (int)((f.P + cl - 1) / cl);
  }
  fp.slots = fp.n_chunks;
  if (f.S > 0) fp.suffix_slot = fp.slots++;
  fp.n_jobs = xs * fp.n_chunks + fp.suffix_jobs;
  return fp;
}

// More than one 128-row tile per KV head (a prefill, or a decode of many
// branches per group) makes the launch matrix-core bound: it then runs 8-wave
// workgroups of 256-row tiles, one per compute unit, sized to half as many
// jobs, so each K/V tile staged in LDS serves twice the rows (as in the walk),
// and its prefix chunks start at multiples of 128 keys for the walk's 128-key
// tiles (fanout_kernel).
FanoutPlan plan_fanout(const FanoutShape& f) {
  FanoutPlan fp = plan_fanout_tiles(f, ba::kTileRows, ba::kFanoutTargetWorkgroups, 64);
  if (BA_FANOUT_WIDE && fp.row_tiles >= 2) {
    fp = plan_fanout_tiles(f, ba::kWideTileRows, ba::kFanoutTargetWorkgroups / 2, 128);
    fp.wide = true;
  }
  return fp;
}

size_t fanout_bytes(const FanoutShape& f) {
  const FanoutPlan fp = plan_fanout(f);
  return partial_bytes(fp.slots, (int64_t)f.nb * f.T * f.Hq, f.D);
}

// With `pages`, prefix_k / prefix_v are the page pools and suffix_k /
// suffix_v are unused.
ba_status fanout_run(const FanoutShape& f, const void* q, const void* prefix_k, const void* prefix_v,
                     const void* suffix_k, const void* suffix_v, void* out, float* lse, void* workspace,
                     size_t workspace_bytes, hipStream_t stream, const ba_kv_pages* pages = nullptr) {
  if (f.nb == 0) return ok();
  if (!q || !out) return fail(BA_ERR_NULL, "q or out is NULL");
  if (pages) {
    if (!prefix_k || !prefix_v) return fail(BA_ERR_NULL, "k_pool or v_pool is NULL");
    if (((uintptr_t)prefix_k % 16) != 0 || ((uintptr_t)prefix_v % 16) != 0)
      return fail(BA_ERR_SHAPE, "k_pool/v_pool not 16-byte aligned");
    if (pages->page_len <= 0 || pages->page_len % 64 != 0)
      return fail(BA_ERR_SHAPE, "page_len %d is not a positive multiple of 64", pages->page_len);
    if (pages->n_pool_pages < 1) return fail(BA_ERR_SHAPE, "n_pool_pages %d < 1", pages->n_pool_pages);
    if (f.P > 0 && !pages->prefix_pages) return fail(BA_ERR_NULL, "prefix_pages is NULL");
    if (f.S > 0 && !pages->suffix_pages) return fail(BA_ERR_NULL, "suffix_pages is NULL");
    // Each segment is a piece of one page, read through a 32-bit buffer range.
    if (head_extent_bf16(pages->page_len, (int64_t)f.Hkv * f.D, f.D) > (int64_t)UINT32_MAX)
      return fail(BA_ERR_SHAPE, "one KV head of a page spans 4 GiB or more");
  } else {
    if (f.P > 0 && (!prefix_k || !prefix_v)) return fail(BA_ERR_NULL, "prefix k/v is NULL");
    if (f.S > 0 && (!suffix_k || !suffix_v)) return fail(BA_ERR_NULL, "suffix k/v is NULL");
    // One KV head of the prefix, and of one branch's suffix, is read through a
    // buffer resource with 32-bit byte offsets.
    if (head_extent_bf16(f.P, (int64_t)f.Hkv * f.D, f.D) > (int64_t)UINT32_MAX ||
        head_extent_bf16(f.S, (int64_t)f.Hkv * f.D, f.D) > (int64_t)UINT32_MAX)
      return fail(BA_ERR_SHAPE, "prefix or suffix: one KV head spans 4 GiB or more (32-bit offsets)");
  }
  const int D = f.D;
  const int64_t R = (int64_t)f.nb * f.T * f.Hq;
  const FanoutPlan fp = plan_fanout(f);
  const size_t need = partial_bytes(fp.slots, R, D);
  if (!workspace || workspace_bytes < need)
    return fail(BA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (((uintptr_t)workspace % 16) != 0) return fail(BA_ERR_WORKSPACE, "workspace not 16-byte aligned");
  float *wm, *wl, *wo;
  partial_ptrs(workspace, fp.slots, R, &wm, &wl, &wo);

  // The query rows of all branches as one block of nb * T tokens.
  ba_problem p;
  memset(&p, 0, sizeof(p));
  p.n_q_heads = f.Hq;
  p.n_kv_heads = f.Hkv;
  p.head_dim = D;
  p.q_len = f.nb * f.T;
  p.q_pos0 = 0;
  p.q_stride_token = (int64_t)f.Hq * D;
  p.q_stride_head = D;
  p.dtype = BA_BF16;
  p.scale = f.scale;
  p.causal = 0;
  const ba::QSide qs = make_qside(&p, q);

  ba::FanoutArgs a;
  memset(&a, 0, sizeof(a));
  a.qs = qs;
  ba_kv_block b = {};
  b.k = prefix_k;
  b.v = prefix_v;
  b.len = f.P;
  b.pos0 = 0;
  b.k_stride_token = b.v_stride_token = (int64_t)f.Hkv * D;
  b.k_stride_head = b.v_stride_head = D;
  a.prefix = make_seg(b, 1);
  a.row_tiles = fp.row_tiles;
  a.chunk_len = fp.chunk_len;
  a.n_chunks = fp.n_chunks;
  a.sk = suffix_k;
  a.sv = suffix_v;
  a.S = f.S;
  a.T = f.T;
  a.suffix_slot = fp.suffix_slot;
  a.srt = fp.srt;
  a.bpj = fp.bpj;
  a.wide = fp.wide ? 1 : 0;
  // Wide launches walk the prefix in 128-key tiles unless its pages split them.
  a.prefix_keys = fp.wide && (!pages || pages->page_len % 128 == 0) ? 128 : 64;
  if (pages) {
    // The kernel takes the paged path for a job kind when its table is set.
    a.sk = nullptr;
    a.sv = nullptr;
    a.prefix_pages = f.P > 0 ? pages->prefix_pages : nullptr;
    a.suffix_pages = f.S > 0 ? pages->suffix_pages : nullptr;
    a.page_len = pages->page_len;
    a.n_pool_pages = pages->n_pool_pages;
    a.suffix_pages_per_branch = (f.S + pages->page_len - 1) / pages->page_len;
  }
  a.ws_m = wm;
  a.ws_l = wl;
  a.ws_o = wo;
  a.R = R;
  hipError_t e = ba::launch_fanout_bf16(a, fp.n_jobs, D, stream);
  if (e != hipSuccess) return hip_status(e, "fanout attention launch");
  ba::MergeGroupArgs mg;
  memset(&mg, 0, sizeof(mg));
  mg.pm = wm;
  mg.pl = wl;
  mg.po = wo;
  mg.R = R;
  mg.n_groups = 1;
  mg.has_init = 0;
  mg.part_begin[0] = 0;
  mg.part_begin[1] = fp.slots;
  mg.fin_out = (uint16_t*)out;
  mg.fin_lse = lse;
  return hip_status(ba::launch_merge_groups(mg, D, stream), "fanout merge launch");
}

// Scratch of the allocation-free fan-out decode: one array per device, part of
// the library's code object, zero at load and held until the process ends.
// In host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kStaticScratchBytes = BLOCKATTN_STATIC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The scratch address on the current device (looked up on its first use).
ba_status static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(BA_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(BA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return BA_OK;
}

FanoutShape decode_shape(const ba_fanout* f) {
  FanoutShape s;
  s.nb = f->n_branches;
  s.T = 1;
  s.Hq = f->n_q_heads;
  s.Hkv = f->n_kv_heads;
  s.D = f->head_dim;
  s.P = f->prefix_len;
  s.S = f->suffix_len;
  s.scale = f->scale;
  return s;
}

ba_status prefill_shape(const ba_fanout_prefill* f, FanoutShape* s) {
  if (!f) return fail(BA_ERR_NULL, "fanout prefill descriptor is NULL");
  s->nb = f->n_branches;
  s->T = f->n_new;
  s->Hq = f->n_q_heads;
  s->Hkv = f->n_kv_heads;
  s->D = f->head_dim;
  s->P = f->prefix_len;
  s->S = f->suffix_len;
  s->scale = f->scale;
  if (f->n_new < 1 || f->n_new > f->suffix_len)
    return fail(BA_ERR_SHAPE, "n_new %d outside 1..suffix_len (%d)", f->n_new, f->suffix_len);
  return check_fanout_shape(*s);
}

}  // namespace

extern "C" {

size_t blockattn_workspace_bytes(const ba_problem* p, const ba_fanout* f) {
  size_t need = 0;
  if (p && check_problem(p, (const void*)256) == BA_OK && p->q_len > 0 && fwd_uses_split(p)) {
    // The split planner's chunks of a call: sum over visited blocks of
    // ceil(keys / chunk_len) <= total / chunk_len + n_visit, with chunk_len >=
    // total / want, so at most want + BLOCKATTN_MAX_VISITS slots.
    const SplitGeom geom = split_geom(p);
    const int tiles = geom.tiles;
    const int64_t want = std::max<int64_t>(1, (geom.target + tiles - 1) / (tiles > 0 ? tiles : 1));
    need = partial_bytes(want + BLOCKATTN_MAX_VISITS, state_rows(p), p->head_dim);
  }
  if (f && check_fanout(f) == BA_OK && f->n_branches > 0) need = std::max(need, fanout_bytes(decode_shape(f)));
  return need;
}

size_t fanout_workspace_bytes(const ba_fanout* f) {
  if (check_fanout(f) != BA_OK || f->n_branches == 0) return 0;
  return fanout_bytes(decode_shape(f));
}

ba_status fanout_prefix_decode(const ba_fanout* f, const void* q, const void* prefix_k, const void* prefix_v,
                               const void* suffix_k, const void* suffix_v, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  ba_status st = check_fanout(f);
  if (st) return st;
  return fanout_run(decode_shape(f), q, prefix_k, prefix_v, suffix_k, suffix_v, out, lse, workspace,
                    workspace_bytes, stream);
}

ba_status fanout_prefix_decode_noalloc(const ba_fanout* f, const void* q, const void* prefix_k,
                                       const void* prefix_v, const void* suffix_k, const void* suffix_v,
                                       void* out, float* lse, hipStream_t stream) {
  ba_status st = check_fanout(f);
  if (st) return st;
  if (f->n_branches == 0) return ok();
  const size_t need = fanout_bytes(decode_shape(f));
  if (need > kStaticScratchBytes)
    return fail(BA_ERR_WORKSPACE, "fan-out needs %zu bytes of scratch; the static scratch holds %zu", need,
                kStaticScratchBytes);
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st) return st;
  return fanout_run(decode_shape(f), q, prefix_k, prefix_v, suffix_k, suffix_v, out, lse, ws, kStaticScratchBytes,
                    stream);
}

size_t fanout_prefill_workspace_bytes(const ba_fanout_prefill* f) {
  FanoutShape s;
  if (prefill_shape(f, &s) != BA_OK || s.nb == 0) return 0;
  return fanout_bytes(s);
}

ba_status fanout_prefix_prefill(const ba_fanout_prefill* f, const void* q, const void* prefix_k,
                                const void* prefix_v, const void* suffix_k, const void* suffix_v, void* out,
                                float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  FanoutShape s;
  ba_status st = prefill_shape(f, &s);
  if (st) return st;
  return fanout_run(s, q, prefix_k, prefix_v, suffix_k, suffix_v, out, lse, workspace, workspace_bytes, stream);
}

ba_status fanout_prefix_decode_paged(const ba_fanout* f, const ba_kv_pages* pages, const void* q,
                                     const void* k_pool, const void* v_pool, void* out, float* lse,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ba_status st = check_fanout(f);
  if (st) return st;
  if (!pages) return fail(BA_ERR_NULL, "pages is NULL");
  return fanout_run(decode_shape(f), q, k_pool, v_pool, nullptr, nullptr, out, lse, workspace, workspace_bytes,
                    stream, pages);
}

ba_status fanout_prefix_prefill_paged(const ba_fanout_prefill* f, const ba_kv_pages* pages, const void* q,
                                      const void* k_pool, const void* v_pool, void* out, float* lse,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  FanoutShape s;
  ba_status st = prefill_shape(f, &s);
  if (st) return st;
  if (!pages) return fail(BA_ERR_NULL, "pages is NULL");
  return fanout_run(s, q, k_pool, v_pool, nullptr, nullptr, out, lse, workspace, workspace_bytes, stream, pages);
}

}  // extern "C"
