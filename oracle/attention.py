"""Exact attention and online-softmax state in NumPy float64 (test oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  No product code may
import this module.

Sources (cited by page title and section; the page text is the authority):

* [RAC] "RingAttention and Context Parallelism: Mathematical Foundations,
  Block-Wise Exact Attention Over Ring Topologies ..." (llms.blog)
  - section 1: the attention definition with an optional causal mask and the
    1/sqrt(d_k) scale;
  - section 2, "The Classical Online Softmax Formulation" and the "Online
    Softmax State Transition Step" box: running max m, denominator l,
    unnormalised accumulator O, the rescale factor exp(m_old - m_new), the
    final normalisation A = O / l, and the exactness identity;
  - section 3, "Initial Sequence Allocation" (state init m=-inf, l=0, O=0) and
    "The N-Step Ring Schedule" (device k holds block (k - t) mod N at step t);
  - section 5 (causal rule: token i attends to tokens j <= i);
  - section 7, backward box (log-sum-exp statistic L = m + ln l).
* [SIM] the systemcraft.online course page on agentic and multimodal
  distributed systems, section 8 (RingAttention simulator): the guard that
  turns the rescale factor into 0 while the running max is still -inf, and the
  ring rotation "send to the right neighbour".
* [AHBM] "AHBM Agentic Runtime Architecture", section 3.3 (per-shard row state
  m[row], l[row], o[row,:]), 3.4 (merge only the same row index across
  shards), 3.5 (hierarchical reduction with one merge primitive), 1.3 / 3.2
  (fan-out query rows batched against a shared prefix KV).
* [TEX] "Supporting Agentic Workloads" (06-agentic.tex), Stationary-KV
  execution policy: rows are independent, the reduction is by row index.

Readings taken where the pages are silent (each is also listed in the design
notes of the repository):

* GQA head mapping: query head h reads KV head h // (Hq / Hkv).
* Positions are absolute; with ``causal`` a key at position p_k is visible to
  a query at position p_q iff p_k <= p_q (diagonal included).
* A row that sees no key keeps the initial state (m=-inf, l=0, O=0); its
  finalised output is 0 and its LSE is -inf.
* The state's m is in natural-log units of the scaled logit.

Array conventions: q [T, Hq, D], k and v [L, Hkv, D]; per-row results are
indexed [T, Hq] (and [T, Hq, D] for vectors).  All arithmetic is float64.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf

# Rows of queries processed per NumPy matmul, to bound the [rows, keys] logit
# buffer.  Chunking the rows does not change any result: rows are independent.
_ROW_CHUNK = 256


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """GQA mapping (reading taken): contiguous groups of Hq/Hkv query heads."""
    assert n_q_heads % n_kv_heads == 0
    return h // (n_q_heads // n_kv_heads)


def scaled_logits(q_rows: np.ndarray, k_rows: np.ndarray, scale: float) -> np.ndarray:
    """z[i, j] = scale * sum_d q[i, d] k[j, d]   ([RAC] section 1 and 2, S = qK^T / sqrt(d_k))."""
    return scale * (q_rows @ k_rows.T)


def causal_visible(q_pos: np.ndarray, k_pos: np.ndarray) -> np.ndarray:
    """Boolean [rows, keys]: key j visible to query i iff k_pos[j] <= q_pos[i]  ([RAC] section 5)."""
    return k_pos[None, :] <= q_pos[:, None]


def softmax_state(z: np.ndarray, v_rows: np.ndarray):
    """Two-pass softmax statistics of one row chunk over its visible keys.

    z holds -inf for masked keys.  Returns (m, l, O) with
    m = max_j z_j, l = sum_j exp(z_j - m), O = sum_j exp(z_j - m) v_j
    -- the state the recurrence of [RAC] section 2 ends in, computed directly.
    Rows with no visible key get (-inf, 0, 0).
    """
    n_rows = z.shape[0]
    if z.shape[1] == 0:
        return (np.full(n_rows, NEG_INF), np.zeros(n_rows), np.zeros((n_rows, v_rows.shape[1])))
    m = z.max(axis=1)
    empty = np.isneginf(m)
    shift = np.where(empty, 0.0, m)
    w = np.exp(z - shift[:, None])          # exp(-inf) = 0 for masked keys
    l = w.sum(axis=1)
    o = w @ v_rows
    return m, l, o


def state(q, k, v, scale, q_pos=None, k_pos=None, causal=False, key_subset=None):
    """Partial online-softmax state over a key subset, for every (token, q-head) row.

    With ``key_subset`` None every key is used.  Returns m [T, Hq], l [T, Hq],
    O [T, Hq, D] (O unnormalised).  [AHBM] section 3.3 / [RAC] section 2.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, D = q.shape
    L, Hkv, Dk = k.shape
    assert Dk == D and v.shape[:2] == (L, Hkv)
    Dv = v.shape[2]
    if q_pos is None:
        q_pos = np.arange(T, dtype=np.int64)
    if k_pos is None:
        k_pos = np.arange(L, dtype=np.int64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    if key_subset is not None:
        key_subset = np.asarray(key_subset, dtype=np.int64)
        k = k[key_subset]
        v = v[key_subset]
        k_pos = k_pos[key_subset]
    m = np.empty((T, Hq))
    l = np.empty((T, Hq))
    o = np.empty((T, Hq, Dv))
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        for r0 in range(0, T, _ROW_CHUNK):
            r1 = min(T, r0 + _ROW_CHUNK)
            z = scaled_logits(q[r0:r1, h, :], k[:, g, :], scale)
            if causal:
                z = np.where(causal_visible(q_pos[r0:r1], k_pos), z, NEG_INF)
            mm, ll, oo = softmax_state(z, v[:, g, :])
            m[r0:r1, h] = mm
            l[r0:r1, h] = ll
            o[r0:r1, h, :] = oo
    return m, l, o


def finalize(m, l, o):
    """A = O / l and LSE = m + ln l  ([RAC] section 2 final normalisation; section 7 LSE).

    Rows with l == 0 (no visible key) give A = 0 and LSE = -inf (reading taken).
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    empty = l == 0.0
    safe_l = np.where(empty, 1.0, l)
    a = np.where(empty[..., None], 0.0, o / safe_l[..., None])
    with np.errstate(divide="ignore"):
        lse = np.where(empty, NEG_INF, m + np.log(safe_l))
    return a, lse


def attend(q, k, v, scale, q_pos=None, k_pos=None, causal=False):
    """Exact attention A = softmax(q k^T * scale + M) v  ([RAC] section 1).

    Returns (A [T, Hq, D], m [T, Hq], l [T, Hq], LSE [T, Hq]).
    """
    m, l, o = state(q, k, v, scale, q_pos, k_pos, causal)
    a, lse = finalize(m, l, o)
    return a, m, l, lse


def init_state(T, Hq, Dv):
    """m = -inf, l = 0, O = 0  ([RAC] section 3, "Initial Sequence Allocation")."""
    return np.full((T, Hq), NEG_INF), np.zeros((T, Hq)), np.zeros((T, Hq, Dv))


def online_step(st, q, k_blk, v_blk, scale, q_pos=None, k_pos_blk=None, causal=False):
    """One step of the online-softmax recurrence over one K/V block.

    In the order of [RAC] section 2's state-transition box:
      1. S = q K^T / sqrt(d_k)                       (block logits, masked)
      2. m_new = max(m_old, max_j S_j)
      3. P = exp(S - m_new)
      4. l_new = exp(m_old - m_new) l_old + sum_j P_j
      5. O_new = exp(m_old - m_new) O_old + P V
    with the [SIM] guard: the rescale factor is 0 while m_old = -inf, and a row
    whose running max is still -inf after the block adds nothing.
    """
    m_old, l_old, o_old = st
    q = np.asarray(q, dtype=np.float64)
    k_blk = np.asarray(k_blk, dtype=np.float64)
    v_blk = np.asarray(v_blk, dtype=np.float64)
    T, Hq, _ = q.shape
    Hkv = k_blk.shape[1]
    if q_pos is None:
        q_pos = np.arange(T, dtype=np.int64)
    if k_pos_blk is None:
        k_pos_blk = np.arange(k_blk.shape[0], dtype=np.int64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos_blk = np.asarray(k_pos_blk, dtype=np.int64)
    m_new = np.empty_like(m_old)
    l_new = np.empty_like(l_old)
    o_new = np.empty_like(o_old)
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        s = scaled_logits(q[:, h, :], k_blk[:, g, :], scale)
        if causal:
            s = np.where(causal_visible(q_pos, k_pos_blk), s, NEG_INF)
        blk_max = s.max(axis=1) if s.shape[1] else np.full(T, NEG_INF)
        mn = np.maximum(m_old[:, h], blk_max)
        still_empty = np.isneginf(mn)
        base = np.where(still_empty, 0.0, mn)
        p = np.exp(s - base[:, None])
        alpha = np.where(np.isneginf(m_old[:, h]), 0.0, np.exp(m_old[:, h] - base))
        m_new[:, h] = mn
        l_new[:, h] = alpha * l_old[:, h] + p.sum(axis=1)
        o_new[:, h, :] = alpha[:, None] * o_old[:, h, :] + p @ v_blk[:, g, :]
    return m_new, l_new, o_new


def walk_blocks(q, blocks, order, scale, q_pos=None, causal=False, st=None):
    """Visit ``blocks[order[0]], blocks[order[1]], ...`` carrying (m, l, O).

    ``blocks`` is a list of (k_blk, v_blk, k_pos_blk).  This is the outer loop
    of blockwise attention for one stationary query block ([RAC] section 3;
    the Ring Attention summary page, "The mechanism").  Returns the state.
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, _ = q.shape
    if st is None:
        st = init_state(T, Hq, np.asarray(blocks[0][1]).shape[2])
    for j in order:
        k_blk, v_blk, k_pos_blk = blocks[j]
        st = online_step(st, q, k_blk, v_blk, scale, q_pos, k_pos_blk, causal)
    return st


def merge(parts):
    """Log-sum-exp merge of partial states of the same rows ([AHBM] 3.4, [TEX]).

    parts: list of (m, l, O) over disjoint key sets, all indexed by the same
    rows.  m* = max_s m_s; w_s = exp(m_s - m*) (0 when m_s = -inf);
    l* = sum_s w_s l_s; O* = sum_s w_s O_s.  Rows never mix.
    """
    ms = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])
    ls = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])
    os_ = np.stack([np.asarray(p[2], dtype=np.float64) for p in parts])
    m_star = ms.max(axis=0)
    base = np.where(np.isneginf(m_star), 0.0, m_star)
    w = np.where(np.isneginf(ms), 0.0, np.exp(ms - base[None]))
    l_star = (w * ls).sum(axis=0)
    o_star = (w[..., None] * os_).sum(axis=0)
    return m_star, l_star, o_star


def merge_tree(parts, fan_in=8):
    """Hierarchical merge with the same primitive at every level ([AHBM] 3.5)."""
    level = list(parts)
    while len(level) > 1:
        level = [merge(level[i:i + fan_in]) for i in range(0, len(level), fan_in)]
    return level[0]


def ring_order(k: int, n: int):
    """Blocks device k visits: block (k - t) mod n at step t  ([RAC] section 3)."""
    return [(k - t) % n for t in range(n)]


def emulate_ring(q_blocks, kv_blocks, scale, causal=False, block_len=None):
    """N simulated devices; K/V blocks rotate one hop to the right per step.

    Device i keeps query block i and its own state.  At every step it updates
    its state with the K/V block it currently holds, then passes that block to
    device (i + 1) mod N ([SIM] section 8; [RAC] section 3).  Positions are
    contiguous: block b covers tokens [b*B, (b+1)*B).  Returns a list of the
    finalised (A, LSE) per device.
    """
    n = len(q_blocks)
    if block_len is None:
        block_len = np.asarray(q_blocks[0]).shape[0]
    states = []
    for i in range(n):
        T, Hq, _ = np.asarray(q_blocks[i]).shape
        states.append(init_state(T, Hq, np.asarray(kv_blocks[0][1]).shape[2]))
    held = list(range(n))            # device i holds block held[i]
    for _ in range(n):
        for i in range(n):
            b = held[i]
            k_blk, v_blk = kv_blocks[b]
            q_pos = i * block_len + np.arange(np.asarray(q_blocks[i]).shape[0])
            k_pos = b * block_len + np.arange(np.asarray(k_blk).shape[0])
            states[i] = online_step(states[i], q_blocks[i], k_blk, v_blk, scale,
                                    q_pos, k_pos, causal)
        rotated = [None] * n
        for i in range(n):
            rotated[(i + 1) % n] = held[i]
        held = rotated
    return [finalize(*s) for s in states]


# ---------------------------------------------------------------- backward pass
# [RAC] section 7, "Memory and Backward Pass Complexity": the forward keeps Q
# and the log-sum-exp L = m + ln l; the backward recomputes each block's
# scores from them, accumulates dQ locally and dK, dV per visiting block.
# The gradients themselves are those of the attention definition of section 1
# (A = softmax(scale * Q K^T + M) V), by the chain rule.

def attention_grads(q, k, v, d_out, scale, q_pos=None, k_pos=None, causal=False, key_subset=None):
    """Gradients of sum(A * d_out) with A the exact attention of ``attend``.

    With p = softmax(z) over row i's visible keys and z = scale * q . k:
      dV_j  = sum_i p_ij dO_i;   dp_ij = dO_i . V_j;
      dz_ij = p_ij (dp_ij - sum_j' p_ij' dp_ij');
      dQ_i  = scale * sum_j dz_ij K_j;   dK_j = scale * sum_i dz_ij Q_i,
    summed over the query heads that read a KV head.  With ``key_subset`` the
    probabilities are still those of the whole key set (the row's final
    softmax) and only the listed keys' terms are returned: dK and dV of the
    other keys are zero and dQ is the listed keys' share -- the contribution
    one visiting block makes in a blockwise backward.  Returns (dQ [T, Hq, D],
    dK [L, Hkv, D], dV [L, Hkv, Dv]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    T, Hq, D = q.shape
    L, Hkv, _ = k.shape
    q_pos = np.arange(T, dtype=np.int64) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    k_pos = np.arange(L, dtype=np.int64) if k_pos is None else np.asarray(k_pos, dtype=np.int64)
    keep = np.ones(L, dtype=bool)
    if key_subset is not None:
        keep[:] = False
        keep[np.asarray(key_subset, dtype=np.int64)] = True
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        z = scaled_logits(q[:, h, :], k[:, g, :], scale)
        vis = causal_visible(q_pos, k_pos) if causal else np.ones((T, L), dtype=bool)
        z = np.where(vis, z, NEG_INF)
        zmax = z.max(axis=1, keepdims=True)
        zmax = np.where(np.isneginf(zmax), 0.0, zmax)
        w = np.where(vis, np.exp(z - zmax), 0.0)
        den = w.sum(axis=1, keepdims=True)
        p = np.divide(w, den, out=np.zeros_like(w), where=den > 0)
        dp = d_out[:, h, :] @ v[:, g, :].T
        dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        pk = np.where(keep[None, :], p, 0.0)
        dzk = np.where(keep[None, :], dz, 0.0)
        dv[:, g, :] += pk.T @ d_out[:, h, :]
        dq[:, h, :] = scale * (dzk @ k[:, g, :])
        dk[:, g, :] += scale * (dzk.T @ q[:, h, :])
    return dq, dk, dv


def backward_ring(q_blocks, kv_blocks, d_out_blocks, scale, causal=False, block_len=None):
    """Blockwise backward over an emulated ring ([RAC] section 7): device i keeps
    Q_i, dO_i and its forward's log-sum-exp; the K/V blocks (with their dK, dV
    buffers) visit in reverse ring order; each visit adds the block's terms to
    the device's dQ and to the visiting block's dK and dV.  Returns
    (dQ per device, dK per block, dV per block)."""
    n = len(q_blocks)
    if block_len is None:
        block_len = np.asarray(q_blocks[0]).shape[0]
    k_all = np.concatenate([np.asarray(kv[0], dtype=np.float64) for kv in kv_blocks])
    v_all = np.concatenate([np.asarray(kv[1], dtype=np.float64) for kv in kv_blocks])
    k_pos = np.arange(k_all.shape[0])
    dqs = [np.zeros(np.asarray(qb).shape) for qb in q_blocks]
    dks = [np.zeros(np.asarray(kv[0]).shape) for kv in kv_blocks]
    dvs = [np.zeros(np.asarray(kv[1]).shape) for kv in kv_blocks]
    for i in range(n):
        q_pos = i * block_len + np.arange(np.asarray(q_blocks[i]).shape[0])
        for t in reversed(range(n)):       # the forward's visits, last first
            b = (i - t) % n
            sub = np.arange(b * block_len, (b + 1) * block_len)
            dq, dk, dv = attention_grads(q_blocks[i], k_all, v_all, d_out_blocks[i], scale, q_pos, k_pos,
                                         causal, key_subset=sub)
            dqs[i] += dq
            dks[b] += dk[sub]
            dvs[b] += dv[sub]
    return dqs, dks, dvs


# ---------------------------------------------------------------- load-balanced causal shares
# [RAC] section 5, "Causal Masking and Load Balancing: Striped vs. Zigzag Ring
# Attention": which tokens device k of n holds.  Each function returns the
# absolute token indices in the order the device stores them.

def contiguous_tokens(seq_len: int, n: int, k: int) -> np.ndarray:
    """Naive sequential partitioning: device k holds tokens [k*B, (k+1)*B), B = seq_len / n."""
    b = seq_len // n
    return np.arange(k * b, (k + 1) * b)


def striped_tokens(seq_len: int, n: int, k: int) -> np.ndarray:
    """Striped sharding: device k holds every token i with i mod n == k."""
    return np.array([i for i in range(seq_len) if i % n == k], dtype=np.int64)


def zigzag_tokens(seq_len: int, n: int, k: int) -> np.ndarray:
    """Zigzag sharding: the sequence is cut into 2n equal chunks c_0 .. c_{2n-1};
    device k holds c_k, then c_{2n-1-k}."""
    c = seq_len // (2 * n)
    first = k
    second = 2 * n - 1 - k
    return np.concatenate([np.arange(first * c, (first + 1) * c), np.arange(second * c, (second + 1) * c)])


def visible_pairs(q_pos, k_pos) -> int:
    """Number of (query, key) pairs the causal rule keeps: #{(i, j) : k_pos[j] <= q_pos[i]}."""
    return int(causal_visible(np.asarray(q_pos), np.asarray(k_pos)).sum())


def ring_step_pairs(owner, seq_len: int, n: int, k: int, t: int) -> int:
    """Causal pairs device k computes at ring step t: its query tokens against
    the K/V tokens of device (k - t) mod n, which it holds at that step
    ([RAC] section 3 ring schedule; section 5 causal rule)."""
    src = (k - t) % n
    return visible_pairs(owner(seq_len, n, k), owner(seq_len, n, src))


def fanout_decode(q, prefix_k, prefix_v, suffix_k, suffix_v, scale):
    """Shared-prefix fan-out decode, by definition.

    q [nb, Hq, D] holds one new query token per branch.  Branch b attends, with
    no mask, to the shared prefix keys followed by its own private suffix keys
    ([AHBM] 1.1 and 3.1: context = shared prefix + private suffix; 1.3: rows of
    several branches are independent).  suffix_k/v [nb, S, Hkv, D] include
    the new token's own K/V.  Returns (A [nb, Hq, D], LSE [nb, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    nb = q.shape[0]
    a = np.empty(q.shape)
    lse = np.empty(q.shape[:2])
    for b in range(nb):
        keys = np.concatenate([np.asarray(prefix_k, dtype=np.float64),
                               np.asarray(suffix_k[b], dtype=np.float64)], axis=0)
        vals = np.concatenate([np.asarray(prefix_v, dtype=np.float64),
                               np.asarray(suffix_v[b], dtype=np.float64)], axis=0)
        ab, _, _, lb = attend(q[b:b + 1], keys, vals, scale)
        a[b] = ab[0]
        lse[b] = lb[0]
    return a, lse


def fanout_prefill(q, prefix_k, prefix_v, suffix_k, suffix_v, scale):
    """Shared-prefix fan-out over several new tokens per branch, by definition.

    q [nb, T, Hq, D] holds the T newest tokens of each branch; suffix_k/v
    [nb, S, Hkv, D] are the branch's private tokens, whose last T are those new
    tokens ([AHBM] 3.1 context structure, 3.2 "20 new tokens per sub-agent",
    3.6 prefill of the private suffixes).  Branch b's context is the shared
    prefix followed by its own suffix; positions run 0 .. P + S - 1 in that
    order, the new token i of the branch sits at P + S - T + i, and the causal
    rule applies ([RAC] section 5).  Returns (A [nb, T, Hq, D], LSE [nb, T, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    nb, T = q.shape[:2]
    P = np.asarray(prefix_k).shape[0]
    S = np.asarray(suffix_k).shape[1]
    a = np.empty(q.shape)
    lse = np.empty(q.shape[:3])
    for b in range(nb):
        keys = np.concatenate([np.asarray(prefix_k, dtype=np.float64).reshape(P, *np.asarray(suffix_k).shape[2:]),
                               np.asarray(suffix_k[b], dtype=np.float64)], axis=0)
        vals = np.concatenate([np.asarray(prefix_v, dtype=np.float64).reshape(P, *np.asarray(suffix_v).shape[2:]),
                               np.asarray(suffix_v[b], dtype=np.float64)], axis=0)
        q_pos = P + S - T + np.arange(T)
        ab, _, _, lb = attend(q[b], keys, vals, scale, q_pos, np.arange(P + S), causal=True)
        a[b] = ab
        lse[b] = lb
    return a, lse


def page_gather(pool, pages, n, page_len, n_pool):
    """The tokens of a paged sequence ([AHBM] 3.1: a context is a page table
    over pages that are referenced, not copied).  Token t (0 <= t < n) is row
    t % page_len of pool page pages[t // page_len].  Readings taken (the pages
    say nothing about ids that name no page): the id -1 marks a hole, whose
    tokens are left out while every other token keeps its position; any other
    id outside [0, n_pool) is a corrupt table, an input error.  Returns
    (rows [m, ...], token indices [m]) in token order."""
    rows, idx = [], []
    for t in range(n):
        pid = int(pages[t // page_len])
        if pid == -1:
            continue
        if not 0 <= pid < n_pool:
            raise ValueError(f"page id {pid} names no page of a pool of {n_pool}")
        rows.append(np.asarray(pool[pid][t % page_len], dtype=np.float64))
        idx.append(t)
    shape = np.asarray(pool).shape[2:]
    return (np.stack(rows) if rows else np.zeros((0,) + tuple(shape))), np.asarray(idx, dtype=np.int64)


def fanout_paged(q, k_pool, v_pool, prefix_pages, suffix_pages, page_len, P, S, scale):
    """Fan-out over paged K/V, by definition: branch b's context is the shared
    prefix pages followed by its own suffix pages ([AHBM] 3.1), gathered by
    page_gather; prefix token t sits at position t, suffix token j at P + j,
    the branch's new token i at P + S - T + i, and the causal rule applies (as
    in fanout_prefill).  q [nb, T, Hq, D]; pools [n_pool, page_len, Hkv, D];
    suffix_pages [nb, ceil(S / page_len)].  Returns (A [nb, T, Hq, D], LSE [nb, T, Hq])."""
    q = np.asarray(q, dtype=np.float64)
    nb, T = q.shape[:2]
    n_pool = np.asarray(k_pool).shape[0]
    pk, pt = page_gather(k_pool, prefix_pages, P, page_len, n_pool)
    pv, _ = page_gather(v_pool, prefix_pages, P, page_len, n_pool)
    a = np.empty(q.shape)
    lse = np.empty(q.shape[:3])
    for b in range(nb):
        sk, st = page_gather(k_pool, suffix_pages[b], S, page_len, n_pool)
        sv, _ = page_gather(v_pool, suffix_pages[b], S, page_len, n_pool)
        keys = np.concatenate([pk, sk], axis=0)
        vals = np.concatenate([pv, sv], axis=0)
        k_pos = np.concatenate([pt, P + st])
        q_pos = P + S - T + np.arange(T)
        ab, _, _, lb = attend(q[b], keys, vals, scale, q_pos, k_pos, causal=True)
        a[b] = ab
        lse[b] = lb
    return a, lse


def fanout_state_rows(q, k, v, scale):
    """Partial state of fan-out rows against one KV range (no mask).

    q [nb, Hq, D]; k, v [L, Hkv, D].  Every branch's query row reads the same
    keys ([AHBM] 1.3, Q_combined x K_shared).  Returns m, l [nb, Hq] and
    O [nb, Hq, D].
    """
    return state(q, k, v, scale, causal=False)
