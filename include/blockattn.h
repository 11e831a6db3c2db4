/*
 * blockattn.h -- C ABI of the exact blockwise attention library (libblockattn.so).
 *
 * The library computes exact softmax attention for a stationary query block
 * by walking K/V blocks in a caller-given order while carrying the per-row
 * online-softmax state (running max m, denominator l, unnormalised output O);
 * it merges partial states of the same rows by log-sum-exp, finalises a state
 * into the attention output and its log-sum-exp, and runs shared-prefix
 * fan-out decode.  Sources (page title, section):
 *
 *   [RAC]  "RingAttention and Context Parallelism: Mathematical Foundations,
 *          Block-Wise Exact Attention Over Ring Topologies ..." (llms.blog):
 *          s.1 attention definition and causal mask; s.2 online-softmax
 *          recurrence and final normalisation; s.3 state initialisation and the
 *          ring schedule (device k holds block (k - t) mod N at step t);
 *          s.5 causal rule; s.7 log-sum-exp statistic L = m + ln l.
 *   [RAS]  "Ring Attention: Blockwise Transformers for Near-Infinite Context"
 *          (daily summary), "The mechanism": the order of the K/V walk for a
 *          fixed query block does not change the result.
 *   [AHBM] "AHBM Agentic Runtime Architecture": s.1.3 / s.3.2 query rows of
 *          several branches batched against one shared KV; s.3.3 per-shard row
 *          state; s.3.4 merge by matching row index only; s.3.5 hierarchical
 *          reduction with one merge primitive.
 *   [TEX]  "Supporting Agentic Workloads": Stationary-KV policy -- query rows
 *          logically replicated over a stationary, sequence-sharded KV.
 *
 * Conventions for every entry point
 *   - Every tensor pointer is a DEVICE pointer allocated and owned by the
 *     caller.  The library never allocates, frees or retains memory and never
 *     synchronises; all work is enqueued on `stream` (0 = the null stream) and
 *     runs asynchronously.  Argument arrays marked HOST are read before the
 *     call returns and may be freed afterwards.
 *   - All argument checks run on the host before anything is enqueued.  A
 *     failed check returns a non-zero ba_status, enqueues nothing, and leaves a
 *     message for blockattn_last_error().  A kernel launch failure returns
 *     BA_ERR_HIP; faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Strides are in elements.  The head_dim axis is always contiguous.
 *     bf16 tensors need 16-byte aligned base pointers and strides that are
 *     multiples of 8 elements; state `o` arrays need 16-byte alignment.
 *   - A "state" is three fp32 arrays indexed by row r = (b * q_len + token) *
 *     n_q_heads + q_head, b the sequence of a batched problem (0 without a
 *     batch): m[rows], l[rows], o[rows * head_dim] (row-major, o unnormalised).
 *     m is in natural-log units of the scaled logit.  The initial state of
 *     [RAC] s.3 is m = -inf, l = 0, o = 0; a row that has seen no key keeps it.
 *   - GQA: query head h reads KV head h / (n_q_heads / n_kv_heads).
 *   - Causal: a key at absolute position p_k is visible to a query at absolute
 *     position p_q iff p_k <= p_q ([RAC] s.5).  K/V blocks or chunks that no
 *     query of a tile can see are skipped.
 *   - Results are bitwise reproducible for identical inputs, arguments and
 *     device (no floating-point atomics).
 *   - Calls are thread-safe; calls that write the same buffers concurrently race.
 */
#ifndef BLOCKATTN_H
#define BLOCKATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BLOCKATTN_ABI_VERSION 2
#define BLOCKATTN_MAX_VISITS 32      /* max K/V blocks visited by one fwd call   */
#define BLOCKATTN_MAX_MERGE_PARTS 64 /* max partial states merged by one call    */

typedef enum {
  BA_OK = 0,
  BA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  BA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes or strides      */
  BA_ERR_UNSUPPORTED = 3, /* valid request this build does not implement        */
  BA_ERR_ORDER = 4,       /* visit order has a duplicate or out-of-range index  */
  BA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required         */
  BA_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed         */
} ba_status;

typedef enum { BA_F32 = 0, BA_BF16 = 1 } ba_dtype;

/* The stationary query block ([RAC] s.3: Q_k stays on its device).
 * q is [q_len, n_q_heads, head_dim] with the given token and head strides;
 * query row t sits at absolute position q_pos0 + t.
 *
 * batch > 1 runs that many independent sequences of the same shape, positions
 * and visit order in one call: q is [batch, q_len, n_q_heads, head_dim] with
 * q_stride_batch elements between sequences; every K/V block holds the keys of
 * all of them at its k/v_stride_batch (0: the sequences share the block's
 * keys); state, output and log-sum-exp rows number batch * q_len * n_q_heads.
 * batch 0 or 1 is one sequence (q_stride_batch is then not read). */
typedef struct {
  int32_t n_q_heads;      /* Hq, a multiple of n_kv_heads                      */
  int32_t n_kv_heads;     /* Hkv                                               */
  int32_t head_dim;       /* D: 64 or 128                                      */
  int32_t q_len;          /* query tokens (0 is a no-op)                       */
  int64_t q_pos0;         /* absolute position of query token 0                */
  int64_t q_stride_token; /* elements between consecutive tokens of q         */
  int64_t q_stride_head;  /* elements between consecutive heads of q          */
  int32_t dtype;          /* ba_dtype of Q, K and V                            */
  float scale;            /* logit scale; <= 0 selects 1/sqrt(head_dim)        */
  int32_t causal;         /* non-zero: apply the causal rule                   */
  int32_t split_mode;     /* 0: automatic; 1: never split the keys (one pass in
                             visit order); 2: always split.  Only
                             rounding differs between the modes.              */
  int32_t batch;          /* independent sequences (0 or 1: one)               */
  int64_t q_stride_batch; /* elements between consecutive sequences of q      */
} ba_problem;

/* One K/V block: k and v are [len, n_kv_heads, head_dim]; key i sits at
 * absolute position pos0 + i ([RAC] s.3, contiguous blocks of the sequence).
 * For a batched problem they are [batch, len, n_kv_heads, head_dim] with the
 * batch strides below (not read without a batch). */
typedef struct {
  const void* k;
  const void* v;
  int32_t len;
  int64_t pos0;
  int64_t k_stride_token, k_stride_head;
  int64_t v_stride_token, v_stride_head;
  int64_t k_stride_batch, v_stride_batch;  /* >= 0; 0 shares the keys */
} ba_kv_block;

/* fp32 online-softmax state; see the conventions above. */
typedef struct {
  float* m;
  float* l;
  float* o;
} ba_state;

/* Shared-prefix fan-out decode shapes ([AHBM] s.1.1, s.3.1-3.2). */
typedef struct {
  int32_t n_branches;  /* branches, one new query token each                   */
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;    /* 64 or 128                                             */
  int32_t prefix_len;  /* shared prefix keys (>= 0)                             */
  int32_t suffix_len;  /* private keys per branch, incl. the new token (>= 0)  */
  float scale;         /* <= 0 selects 1/sqrt(head_dim)                         */
} ba_fanout;

/* Walk K/V blocks for one stationary query block, updating `state` in place.
 *
 * Visits blocks[order[0]], blocks[order[1]], ..., blocks[order[n_visit-1]]
 * (order is a HOST array of distinct indices < n_blocks; NULL means
 * 0, 1, ..., n_visit-1) and applies the online-softmax step of [RAC] s.2 to
 * every query row: m_new = max(m_old, max_j s_j); P = exp(s - m_new);
 * l_new = exp(m_old - m_new) l_old + sum_j P_j; O_new = exp(m_old - m_new) O_old
 * + P V, with s = scale * q . k.  With reset_state != 0 the state is first
 * set to (-inf, 0, 0) ([RAC] s.3); otherwise the caller's state is continued,
 * so one call per ring step carries the state between steps.  The order only
 * affects rounding ([RAS]).  bf16 runs QK^T and PV on bf16 matrix cores with
 * fp32 accumulation and rounds P to bf16 (nearest-even) before PV; f32 runs
 * every step in fp32.
 *
 * When the query block has too few rows to fill the GPU the keys
 * are split into chunks computed in parallel and merged by log-sum-exp; that
 * needs `workspace` of blockattn_fwd_workspace_bytes() bytes (device memory,
 * 256-byte aligned).  Otherwise workspace may be NULL.
 *
 * Only keys [0, len) of a block are read: the bytes after a block's last key
 * are never touched, whatever they hold, and a key no query row of a tile of
 * the call can see under the causal rule is not read either.
 *
 * Errors: BA_ERR_NULL (p, q, blocks with n_visit > 0, a block's k/v with
 * len > 0, or a state array); BA_ERR_SHAPE (bad head counts, head_dim, negative
 * lengths or batch, non-positive token or head strides, with batch > 1 a
 * non-positive q_stride_batch or a negative k/v_stride_batch, more than 2^30
 * state rows, a bf16 block whose token stride is below head_dim, a bf16 block
 * one of whose KV heads spans 4 GiB or more in one sequence: the bf16 kernels
 * address it with 32-bit offsets); BA_ERR_ORDER (duplicate/out-of-range order
 * entry, n_visit > BLOCKATTN_MAX_VISITS or > n_blocks); BA_ERR_UNSUPPORTED
 * (dtype); BA_ERR_WORKSPACE. */
ba_status blockattn_fwd_block(const ba_problem* p, const void* q,
                              const ba_kv_block* blocks, int32_t n_blocks,
                              const int32_t* order, int32_t n_visit,
                              ba_state state, int32_t reset_state,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* The last visits of a query block and its finalisation in one call ([RAC]
 * s.2 and s.7): the result is that of blockattn_fwd_block with the same
 * arguments followed by blockattn_finalize(state, rows, head_dim, out,
 * out_dtype, out_row_stride, lse) with rows = batch * q_len * n_q_heads --
 * out [rows, state-row order] of A = O / l in out_dtype (BA_BF16,
 * rounded to nearest even, or BA_F32), lse (may be NULL) of m + ln l, and 0 /
 * -inf for rows that saw no key -- up to rounding: the bf16 walk writes A and
 * LSE from its registers instead of storing the state and reading it back.
 * With reset_state == 0 the caller's state is read first, as by
 * blockattn_fwd_block.  Afterwards the contents of state are unspecified (it
 * may or may not hold the updated state).  Same workspace as
 * blockattn_fwd_block (blockattn_fwd_workspace_bytes).  out and lse are
 * written by the device; the caller owns them.  Errors: as
 * blockattn_fwd_block, plus those of blockattn_finalize for out (BA_ERR_NULL,
 * BA_ERR_UNSUPPORTED out_dtype, BA_ERR_SHAPE out_row_stride < head_dim or not a
 * multiple of 4, out not 8-byte (bf16) or 16-byte (fp32) aligned), all checked
 * before anything is launched. */
ba_status blockattn_fwd_block_finalize(const ba_problem* p, const void* q,
                                       const ba_kv_block* blocks, int32_t n_blocks,
                                       const int32_t* order, int32_t n_visit,
                                       ba_state state, int32_t reset_state,
                                       void* out, int32_t out_dtype, int64_t out_row_stride,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* Bytes of workspace blockattn_fwd_block needs for these arguments (0 when
 * none).  Returns 0 as well for arguments blockattn_fwd_block would reject. */
size_t blockattn_fwd_workspace_bytes(const ba_problem* p, const ba_kv_block* blocks,
                                     int32_t n_blocks, const int32_t* order,
                                     int32_t n_visit);

/* Per-shard partial states ([AHBM] s.3.3; [TEX] Stationary-KV policy).
 *
 * For every block i < n_blocks, writes states_out[i] = the online-softmax
 * state of all query rows over block i alone (as if blockattn_fwd_block
 * visited only block i from the initial state).  states_out is a HOST array
 * of n_blocks states; they must not overlap.  bf16 or fp32.  Needs
 * blockattn_shard_workspace_bytes() bytes of workspace.  Errors as for
 * blockattn_fwd_block; n_blocks <= BLOCKATTN_MAX_VISITS. */
ba_status blockattn_shard_states(const ba_problem* p, const void* q,
                                 const ba_kv_block* blocks, int32_t n_blocks,
                                 const ba_state* states_out,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

size_t blockattn_shard_workspace_bytes(const ba_problem* p, const ba_kv_block* blocks,
                                       int32_t n_blocks);

/* Row-wise n-way log-sum-exp merge of partial states ([AHBM] s.3.4-3.5).
 *
 * parts is a HOST array of n_parts states over the same `rows` rows (each
 * computed over a disjoint key set).  For every row r:
 *   m* = max_s m_s[r];  w_s = exp(m_s[r] - m*) (0 when m_s[r] = -inf);
 *   l* = sum_s w_s l_s[r];  o*[r,:] = sum_s w_s o_s[r,:].
 * Parts whose m is -inf contribute nothing and their o is not read.  A part
 * whose m is +inf (the marker of rows whose keys could not be read, see
 * ba_kv_pages) is passed through: the row takes that part's l and o and
 * ignores the others.  Rows are never combined with other rows.  `out` may be one of the parts (in place);
 * it must not partially overlap any part.  1 <= n_parts <=
 * BLOCKATTN_MAX_MERGE_PARTS; merge more by merging merged states (the same
 * primitive at every level, [AHBM] s.3.5).  Errors: BA_ERR_NULL, BA_ERR_SHAPE. */
ba_status blockattn_merge_states(int32_t n_parts, const ba_state* parts,
                                 int64_t rows, int32_t head_dim,
                                 ba_state out, hipStream_t stream);

/* Final normalisation ([RAC] s.2: A = O / l) and log-sum-exp ([RAC] s.7).
 *
 * out[r * out_row_stride + d] = o[r, d] / l[r] stored as out_dtype (bf16
 * rounds to nearest even); lse[r] = m[r] + ln l[r] (lse may be NULL).  Rows
 * with l == 0 give out = 0 and lse = -inf.  Errors: BA_ERR_NULL, BA_ERR_SHAPE
 * (out_row_stride < head_dim), BA_ERR_UNSUPPORTED (out_dtype). */
ba_status blockattn_finalize(ba_state st, int64_t rows, int32_t head_dim,
                             void* out, int32_t out_dtype, int64_t out_row_stride,
                             float* lse, hipStream_t stream);

/* Shared-prefix fan-out decode ([AHBM] s.1.1-1.3, s.3.1-3.4; [TEX]).
 *
 * q [n_branches, n_q_heads, head_dim] bf16 holds one new query token per
 * branch; prefix_k/v [prefix_len, n_kv_heads, head_dim] bf16 is the shared
 * prefix, read once for all branches; suffix_k/v [n_branches, suffix_len,
 * n_kv_heads, head_dim] bf16 holds each branch's private keys (including the
 * new token's own K/V).  All contiguous.  Branch b attends, without a mask,
 * to the prefix followed by its own suffix.  The query rows of every branch
 * that share a KV head are batched into one matrix against each prefix chunk;
 * each branch's suffix gives its own partial; the partials of each row are
 * merged by log-sum-exp and finalised.  Writes out [n_branches, n_q_heads,
 * head_dim] bf16 and, if lse is not NULL, lse [n_branches, n_q_heads] fp32.
 * Needs fanout_workspace_bytes() bytes of workspace.  Errors: BA_ERR_NULL,
 * BA_ERR_SHAPE (no keys at all, bad heads or head_dim, one KV head of the
 * prefix or of a suffix spanning 4 GiB or more), BA_ERR_WORKSPACE. */
ba_status fanout_prefix_decode(const ba_fanout* f, const void* q,
                               const void* prefix_k, const void* prefix_v,
                               const void* suffix_k, const void* suffix_v,
                               void* out, float* lse,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

size_t fanout_workspace_bytes(const ba_fanout* f);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * fan-out decode as fanout_prefix_decode (same kernels, bit-identical
 * results) with no workspace argument.  Its partial states go to a scratch
 * array of BLOCKATTN_STATIC_SCRATCH_BYTES that the library holds on each
 * device it runs on, from the first call on that device (the calling thread's
 * current device, to which `stream` must belong) until the process ends.  The
 * call allocates nothing.  Every call on one device shares that device's
 * scratch, and it keeps the last call's contents: calls that overlap on one
 * device (on different streams, or from different threads without ordering)
 * race; calls on one stream are ordered and safe.  The caller owns q, the K/V
 * and out/lse as for fanout_prefix_decode.  Errors: as fanout_prefix_decode,
 * with BA_ERR_WORKSPACE when fanout_workspace_bytes(f) exceeds the scratch
 * (checked before anything is enqueued), BA_ERR_HIP when the scratch's
 * address cannot be obtained. */
#define BLOCKATTN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
ba_status fanout_prefix_decode_noalloc(const ba_fanout* f, const void* q,
                                       const void* prefix_k, const void* prefix_v,
                                       const void* suffix_k, const void* suffix_v,
                                       void* out, float* lse, hipStream_t stream);

/* Shared-prefix fan-out over several new tokens per branch: prefill of the
 * branches' private suffixes ([AHBM] s.2.5, s.3.1-3.2 and s.3.6: 8 sub-agents
 * x 20 new tokens give a combined query matrix of 160 rows per query head).
 *
 * q [n_branches, n_new, n_q_heads, head_dim] bf16 holds each branch's n_new
 * newest tokens; prefix_k/v [prefix_len, n_kv_heads, head_dim] bf16 is the
 * shared prefix, read once for all branches; suffix_k/v [n_branches,
 * suffix_len, n_kv_heads, head_dim] bf16 holds each branch's private tokens,
 * whose last n_new are the new ones (1 <= n_new <= suffix_len).  All
 * contiguous.  Branch b's context is the prefix then its own suffix, at
 * positions 0 .. prefix_len + suffix_len - 1; new token i sits at
 * prefix_len + suffix_len - n_new + i and sees every key up to and including
 * its own position (the causal rule of [RAC] s.5).  Every branch's rows that
 * share a KV head are batched against each prefix chunk; each branch's suffix
 * gives its own causal partial; partials merge by log-sum-exp per row.
 * Writes out [n_branches, n_new, n_q_heads, head_dim] bf16 and, if lse is not
 * NULL, lse [n_branches, n_new, n_q_heads] fp32.  With n_new = 1 this is
 * fanout_prefix_decode.  Needs fanout_prefill_workspace_bytes() bytes of
 * workspace (device memory, 16-byte aligned).  Errors: BA_ERR_NULL,
 * BA_ERR_SHAPE (bad head counts or head_dim, n_new outside 1..suffix_len,
 * negative lengths), BA_ERR_WORKSPACE. */
typedef struct {
  int32_t n_branches;  /* branches                                              */
  int32_t n_new;       /* new query tokens per branch (the suffix's last n_new) */
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;    /* 64 or 128                                             */
  int32_t prefix_len;  /* shared prefix keys (>= 0)                             */
  int32_t suffix_len;  /* private keys per branch, incl. the new tokens         */
  float scale;         /* <= 0 selects 1/sqrt(head_dim)                         */
} ba_fanout_prefill;

ba_status fanout_prefix_prefill(const ba_fanout_prefill* f, const void* q,
                                const void* prefix_k, const void* prefix_v,
                                const void* suffix_k, const void* suffix_v,
                                void* out, float* lse,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

size_t fanout_prefill_workspace_bytes(const ba_fanout_prefill* f);

/* Paged KV for the fan-out ([AHBM] s.3.1, s.5.12; [TEX] fork by page table):
 * a branch's context is a page table of the shared prefix pages followed by
 * its private pages, all in one pool, and the shared pages are referenced,
 * never copied.  Pools k_pool and v_pool are [n_pool_pages, page_len,
 * n_kv_heads, head_dim] bf16, contiguous, 16-byte aligned.  Prefix token t is
 * row t % page_len of pool page prefix_pages[t / page_len]; suffix token j of
 * branch b is row j % page_len of page
 * suffix_pages[b * ceil(suffix_len / page_len) + j / page_len].  Both tables
 * are DEVICE int32 arrays of at least ceil(prefix_len / page_len) and
 * n_branches * ceil(suffix_len / page_len) entries; the caller owns them and
 * must not change them until the call has run on its stream.  page_len is a
 * positive multiple of 64, so no 64-key tile straddles two pages.  The id -1
 * marks a hole: its tokens are left out and the other tokens keep their
 * positions.  Any other id outside [0, n_pool_pages) is a corrupt table, which
 * the host cannot see (the tables are device memory): no page is read through
 * it, and every row whose keys it would name -- a branch's rows for a corrupt
 * suffix id, every row for a corrupt prefix id -- comes out as NaN with LSE
 * +inf, so the error shows instead of a result over a wrong key set. */
typedef struct {
  const int32_t* prefix_pages;
  const int32_t* suffix_pages;
  int32_t page_len;
  int32_t n_pool_pages;
} ba_kv_pages;

/* fanout_prefix_decode and fanout_prefix_prefill over paged K/V: the same
 * attention, positions, outputs and workspace sizes (fanout_workspace_bytes,
 * fanout_prefill_workspace_bytes).  With every id valid the results equal the
 * contiguous entry points' bit for bit when page_len is a multiple of 128, or
 * when a KV head's query rows (n_branches * n_new * n_q_heads / n_kv_heads)
 * number at most 128; otherwise (pages of an odd multiple of 64 keys under a
 * launch that walks the prefix in 128-key tiles) they agree up to rounding.
 * Errors: as the contiguous entry
 * points, plus BA_ERR_NULL (pages, a needed page table, a pool) and
 * BA_ERR_SHAPE (page_len not a positive multiple of 64, n_pool_pages < 1,
 * misaligned pool). */
ba_status fanout_prefix_decode_paged(const ba_fanout* f, const ba_kv_pages* pages, const void* q,
                                     const void* k_pool, const void* v_pool, void* out, float* lse,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

ba_status fanout_prefix_prefill_paged(const ba_fanout_prefill* f, const ba_kv_pages* pages,
                                      const void* q, const void* k_pool, const void* v_pool,
                                      void* out, float* lse, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Workspace enough for every blockattn_fwd_block call on problem p whatever
 * its blocks and visit order (a bound: the split planner makes at most
 * ceil(W / (row tiles x KV heads)) + BLOCKATTN_MAX_VISITS key chunks, W being
 * 512 workgroups of 128-row tiles, or 256 of 256-row tiles when a KV head's
 * query rows fill two or more 128-row tiles), and
 * for fanout_prefix_decode with descriptor f; either may be NULL.  Lets a
 * caller size one workspace up front (blockattn_shard_states, which always
 * splits, has its own query above).  0 when nothing needs one or an argument
 * is invalid. */
size_t blockattn_workspace_bytes(const ba_problem* p_or_null, const ba_fanout* f_or_null);

/* Static description of a status code; never NULL. */
const char* blockattn_status_str(int32_t status);

/* Message of the last failed check on the calling thread ("" if none). */
const char* blockattn_last_error(void);

/* Backward pass, first step: delta[r] = sum_d dout[r, d] * out[r, d] (the row
 * term of the softmax Jacobian, [RAC] s.7 backward box with the chain rule of
 * s.1).  out is the forward's finalised output (bf16 or fp32 as out_dtype),
 * dout the gradient of the loss with respect to it (bf16); rows in state-row
 * order (token * n_q_heads + head), row strides in elements.  Errors:
 * BA_ERR_NULL, BA_ERR_SHAPE (head_dim, strides < head_dim or not multiples of
 * 8, misaligned), BA_ERR_UNSUPPORTED (out_dtype). */
ba_status blockattn_bwd_delta(int64_t rows, int32_t head_dim, const void* out, int32_t out_dtype,
                              int64_t out_row_stride, const void* dout, int64_t dout_row_stride,
                              float* delta, hipStream_t stream);

/* Backward pass over the K/V blocks one forward call visited ([RAC] s.7:
 * recompute each block's scores from the stored Q and log-sum-exp, accumulate
 * dQ for the stationary query block and dK, dV for the visiting block).
 *
 * p, q, blocks, n_blocks, order and n_visit are those of the forward; dout
 * ([batch,] q_len, n_q_heads, head_dim] bf16 with q's strides) is the gradient
 * of the loss with respect to the finalised output; lse [rows] is the
 * forward's final log-sum-exp (blockattn_finalize, natural log; -inf for a
 * row that saw no key) and delta the output of blockattn_bwd_delta, both in
 * state-row order.  With P = exp(scale q.k - lse) over the row's visible keys:
 *   dq[r, :] += scale * sum_j P_rj (dP_rj - delta_r) k_j,  dP_rj = dout_r . v_j;
 *   dk_b[j, g, :] += scale * sum_r P_rj (dP_rj - delta_r) q_r;
 *   dv_b[j, g, :] += sum_r P_rj dout_r,
 * summed over the query heads r of KV head g.  dq is fp32 [rows, head_dim]
 * (state-row order); dk and dv are HOST arrays of n_blocks device pointers,
 * entry b pointing at fp32 [blocks[b].len, n_kv_heads, head_dim] (contiguous)
 * for every visited block -- [batch, len, n_kv_heads, head_dim] for a batched
 * problem, one gradient per sequence also where the sequences share the
 * block's keys (their sum is the shared keys' gradient); rows = batch * q_len
 * * n_q_heads.  All accumulate (+=), so one call per
 * ring step (reverse order or any order) builds the full gradients; within a
 * call the blocks are processed in key-position order (order changes only
 * rounding).  Blocks no query of the block can see are skipped.  The dk/dv buffers of different
 * blocks of one call are updated concurrently and must not overlap; calls that
 * share buffers must be ordered (one stream).  The caller owns every buffer;
 * nothing is kept after the call returns.  Results do not depend on scheduling
 * (no atomics).  bf16 only; one sequence's q (and dout) rows, and the lse and
 * delta rows of all sequences, must each span less than 4 GiB.  Errors: as
 * blockattn_fwd_block, plus
 * BA_ERR_NULL (dout, lse, delta, dq, or a visited block's dk/dv) and
 * BA_ERR_UNSUPPORTED (fp32 problems). */
ba_status blockattn_bwd_block(const ba_problem* p, const void* q, const void* dout,
                              const float* lse, const float* delta,
                              const ba_kv_block* blocks, int32_t n_blocks,
                              const int32_t* order, int32_t n_visit,
                              float* dq, float* const* dk, float* const* dv,
                              hipStream_t stream);

/* BLOCKATTN_ABI_VERSION of the loaded library. */
int32_t blockattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKATTN_H */
