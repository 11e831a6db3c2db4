"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages or the mathematics fix.  ``test_oracle_pins.py`` runs them;
``test_oracle_mutations.py`` plants plausible mistakes in the oracle (on the
CPU) and checks that at least one pin catches each.

Citations name the page and section; see the oracle's module docstring for
the page list.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import scipy.special

from oracle import attention as ora
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(1000 + seed))


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    diff = np.where(both_inf, 0.0, np.abs(a - b))
    tol = atol + rtol * np.where(both_inf, 0.0, np.abs(b))
    bad = ~(diff <= tol)
    if bad.any():
        worst = np.where(bad, np.nan_to_num(diff, nan=np.inf), 0.0).max()
        raise AssertionError(f"{what}: max diff {worst} at {np.argwhere(bad)[:3].tolist()}")


# --- brute force on tiny inputs (llms.blog page, section 1 definition) -------

TINY_CASES = [
    # (T, L, Hq, Hkv, D, causal, q_pos0, k_pos0)
    (3, 5, 1, 1, 1, False, 0, 0),
    (4, 7, 2, 1, 2, True, 3, 0),
    (5, 9, 4, 2, 4, True, 2, 1),
    (2, 16, 2, 2, 8, False, 0, 0),
    (6, 11, 4, 1, 8, True, 5, 0),
    (3, 1, 2, 2, 4, True, 0, 0),
]


def pin_brute_force_tiny():
    """NumPy oracle == pure-Python fsum oracle within 1e-13 relative."""
    for idx, (T, L, Hq, Hkv, D, causal, qp0, kp0) in enumerate(TINY_CASES):
        g = _rng(idx)
        q = g.standard_normal((T, Hq, D))
        k = g.standard_normal((L, Hkv, D))
        v = g.standard_normal((L, Hkv, D))
        q_pos = qp0 + np.arange(T)
        k_pos = kp0 + np.arange(L)
        scale = 1.0 / math.sqrt(D)
        a, m, l, lse = ora.attend(q, k, v, scale, q_pos, k_pos, causal)
        A, M, Ls, LSE = brute.attend(q.tolist(), k.tolist(), v.tolist(), scale,
                                     q_pos.tolist(), k_pos.tolist(), causal)
        _close(a, A, 1e-13, 1e-14, f"A case {idx}")
        _close(m, M, 1e-13, 1e-14, f"m case {idx}")
        _close(l, Ls, 1e-13, 1e-14, f"l case {idx}")
        _close(lse, LSE, 1e-13, 1e-14, f"lse case {idx}")


# --- library routines: scipy softmax / logsumexp ----------------------------

def pin_scipy_softmax_logsumexp():
    """Per row, A == scipy softmax(z) @ v and LSE == scipy logsumexp(z)."""
    g = _rng(11)
    T, L, Hq, Hkv, D = 5, 13, 4, 2, 8
    q = g.standard_normal((T, Hq, D))
    k = g.standard_normal((L, Hkv, D))
    v = g.standard_normal((L, Hkv, D))
    scale = 0.37
    a, m, l, lse = ora.attend(q, k, v, scale)
    for t in range(T):
        for h in range(Hq):
            gg = h // (Hq // Hkv)
            z = np.array([scale * float(np.dot(q[t, h], k[j, gg])) for j in range(L)])
            _close(a[t, h], scipy.special.softmax(z) @ v[:, gg], 1e-13, 1e-14, "A vs scipy")
            _close(lse[t, h], scipy.special.logsumexp(z), 1e-13, 0, "lse vs scipy")
            _close(m[t, h], z.max(), 1e-13, 0, "m vs max")


# --- closed forms -----------------------------------------------------------

def pin_closed_forms():
    g = _rng(21)
    T, L, Hq, Hkv, D = 6, 10, 2, 1, 4
    q = g.standard_normal((T, Hq, D))
    k = g.standard_normal((L, Hkv, D))
    scale = 1.0 / math.sqrt(D)
    q_pos = 4 + np.arange(T)
    # (i) V all ones -> every output is 1 (softmax rows sum to 1), causal or not.
    for causal in (False, True):
        a, *_ = ora.attend(q, k, np.ones((L, Hkv, D)), scale, q_pos, None, causal)
        _close(a, np.ones_like(a), 0, 1e-15, "ones")
    # (ii) every V row equal to c -> A = c.
    c = g.standard_normal(D)
    a, *_ = ora.attend(q, k, np.broadcast_to(c, (L, Hkv, D)).copy(), scale)
    _close(a, np.broadcast_to(c, a.shape), 1e-14, 1e-15, "const rows")
    # (iii) K = 0 -> uniform weights: A = mean of the visible V rows.
    v = g.standard_normal((L, Hkv, D))
    a, m, l, lse = ora.attend(q, np.zeros((L, Hkv, D)), v, scale, q_pos, None, True)
    for t in range(T):
        n_vis = min(L, q_pos[t] + 1)
        _close(a[t, 0], v[:n_vis, 0].mean(axis=0), 1e-14, 1e-15, "K=0 mean")
        _close(l[t, 0], float(n_vis), 0, 0, "K=0 l counts keys")
        _close(m[t, 0], 0.0, 0, 0, "K=0 m")
    # (iv) D = 1, two keys: A = v1 sigmoid(z1 - z2) + v2 sigmoid(z2 - z1).
    qq = np.array([[[0.7]]])
    kk = np.array([[[1.3]], [[-0.4]]])
    vv = np.array([[[2.0]], [[-5.0]]])
    a, *_ = ora.attend(qq, kk, vv, 1.0)
    z1, z2 = 0.7 * 1.3, 0.7 * -0.4
    expect = 2.0 * scipy.special.expit(z1 - z2) + -5.0 * scipy.special.expit(z2 - z1)
    _close(a[0, 0, 0], expect, 1e-15, 0, "two-key sigmoid")
    # (v) causal query at position 0 sees only key 0 -> A = V[0] exactly.
    a, m, l, lse = ora.attend(q[:1], k, v, scale, np.array([0]), None, True)
    assert np.array_equal(a[0, 0], v[0, 0]), "causal position 0"
    assert l[0, 0] == 1.0
    # (vi) a query before every key sees nothing: A = 0, LSE = -inf.
    a, m, l, lse = ora.attend(q[:1], k, v, scale, np.array([-1]), None, True)
    assert np.all(a == 0) and np.all(np.isneginf(lse)) and np.all(l == 0) and np.all(np.isneginf(m))


def pin_shift_invariance():
    """K_j -> K_j + u: A unchanged, m shifts by scale q.u, l unchanged."""
    g = _rng(31)
    T, L, Hq, D = 4, 9, 2, 8
    q = g.standard_normal((T, Hq, D))
    k = g.standard_normal((L, 1, D))
    v = g.standard_normal((L, 1, D))
    u = g.standard_normal(D)
    s = 0.3
    a0, m0, l0, _ = ora.attend(q, k, v, s)
    a1, m1, l1, _ = ora.attend(q, k + u, v, s)
    _close(a1, a0, 1e-12, 1e-13, "shift A")
    _close(m1, m0 + s * (q @ u), 1e-12, 1e-13, "shift m")
    _close(l1, l0, 1e-12, 0, "shift l")


# --- order invariance and split/merge (Ring Attention summary; AHBM 3.4) -----

def _blocks(k, v, n_blk, blen, pos0=0):
    return [(k[b * blen:(b + 1) * blen], v[b * blen:(b + 1) * blen],
             pos0 + b * blen + np.arange(blen)) for b in range(n_blk)]


def pin_order_invariance():
    """The recurrence over every order of 4 blocks equals the definition."""
    g = _rng(41)
    T, blen, nb, Hq, Hkv, D = 5, 6, 4, 4, 2, 8
    q = g.standard_normal((T, Hq, D))
    k = g.standard_normal((nb * blen, Hkv, D)) * 2.0
    v = g.standard_normal((nb * blen, Hkv, D))
    s = 1.0 / math.sqrt(D)
    for causal, q_pos in ((False, np.arange(T)), (True, 11 + np.arange(T))):
        a_ref, m_ref, l_ref, lse_ref = ora.attend(q, k, v, s, q_pos, None, causal)
        blocks = _blocks(k, v, nb, blen)
        for order in itertools.permutations(range(nb)):
            st = ora.walk_blocks(q, blocks, order, s, q_pos, causal)
            a, lse = ora.finalize(*st)
            _close(a, a_ref, 1e-12, 1e-13, f"order {order}")
            _close(st[0], m_ref, 1e-12, 1e-13, "order m")
            _close(lse, lse_ref, 1e-12, 1e-13, "order lse")


def pin_split_merge():
    """Random key partitions (with empty shards, 32-way) merged == unsplit."""
    g = _rng(51)
    T, L, Hq, Hkv, D = 4, 40, 2, 1, 8
    q = g.standard_normal((T, Hq, D))
    k = g.standard_normal((L, Hkv, D)) * 3.0
    v = g.standard_normal((L, Hkv, D))
    s = 1.0 / math.sqrt(D)
    m_ref, l_ref, o_ref = ora.state(q, k, v, s)
    for n_parts in (2, 3, 7, 32):
        labels = g.integers(0, n_parts, size=L)
        labels[:1] = 0
        parts = [ora.state(q, k, v, s, key_subset=np.flatnonzero(labels == p)) for p in range(n_parts)]
        for merged in (ora.merge(parts), ora.merge_tree(parts, fan_in=3)):
            _close(merged[0], m_ref, 1e-13, 0, f"merge m n={n_parts}")
            _close(merged[1], l_ref, 1e-12, 0, f"merge l n={n_parts}")
            _close(merged[2], o_ref, 1e-12, 1e-13, f"merge O n={n_parts}")
    # an all-empty part is the identity
    empty = ora.init_state(T, Hq, D)
    merged = ora.merge([empty, (m_ref, l_ref, o_ref), empty])
    _close(merged[2], o_ref, 0, 0, "empty identity")


def pin_causal_future_keys():
    """Changing every future key and value leaves a row's output bitwise equal."""
    g = _rng(61)
    T, L, Hq, D = 6, 20, 2, 8
    q = g.standard_normal((T, Hq, D))
    k = g.standard_normal((L, 1, D))
    v = g.standard_normal((L, 1, D))
    q_pos = 7 + np.arange(T)
    s = 1.0 / math.sqrt(D)
    a0, *_ = ora.attend(q, k, v, s, q_pos, None, True)
    for t in range(T):
        k2, v2 = k.copy(), v.copy()
        fut = np.arange(L) > q_pos[t]
        k2[fut] = g.standard_normal((fut.sum(), 1, D)) * 10
        v2[fut] = g.standard_normal((fut.sum(), 1, D)) * 10
        a1, *_ = ora.attend(q, k2, v2, s, q_pos, None, True)
        assert np.array_equal(a1[t], a0[t]), f"future keys changed row {t}"


def pin_large_logits():
    """Logits of about +-1000: finite results, merge == unsplit, brute agrees."""
    g = _rng(71)
    T, L, D = 3, 12, 4
    q = g.standard_normal((T, 1, D)) * 30
    k = g.standard_normal((L, 1, D)) * 30
    v = g.standard_normal((L, 1, D))
    s = 1.0
    a, m, l, lse = ora.attend(q, k, v, s)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(lse))
    assert np.abs(m).max() > 300
    A, M, Ls, LSE = brute.attend(q.tolist(), k.tolist(), v.tolist(), s)
    _close(a, A, 1e-12, 1e-13, "large A")
    _close(lse, LSE, 1e-13, 0, "large lse")
    parts = [ora.state(q, k, v, s, key_subset=np.arange(i, L, 4)) for i in range(4)]
    mm, ll, oo = ora.merge(parts)
    a2, lse2 = ora.finalize(mm, ll, oo)
    _close(a2, a, 1e-12, 1e-13, "large merge")


# --- ring schedule and multi-device emulation --------------------------------

def pin_ring_schedule_printed():
    """The printed 4-GPU schedule (course page 3.1) and (k - t) mod N (llms.blog section 3)."""
    with open(os.path.join(GOLDEN, "ring_schedule_printed.json")) as f:
        gold = json.load(f)
    n = gold["n_devices"]
    for k_str, steps in gold["printed_steps"].items():
        assert ora.ring_order(int(k_str), n) == steps, (k_str, ora.ring_order(int(k_str), n), steps)


def pin_ring_simulator_worked_example():
    """The course page's 4-worker scalar simulator: ring emulation == definition == brute."""
    with open(os.path.join(GOLDEN, "ring_simulator_worked_example.json")) as f:
        gold = json.load(f)
    n = gold["n_devices"]
    q = np.array(gold["q"]).reshape(n, 1, 1)
    k = np.array(gold["k"]).reshape(n, 1, 1)
    v = np.array(gold["v"]).reshape(n, 1, 1)
    exp = gold["expected"]
    a, m, l, lse = ora.attend(q, k, v, gold["scale"])
    _close(a[:, 0, 0], exp["A"], 1e-14, 0, "worked A")
    _close(m[:, 0], exp["m"], 1e-15, 0, "worked m")
    _close(l[:, 0], exp["l"], 1e-14, 0, "worked l")
    _close(lse[:, 0], exp["lse"], 1e-14, 0, "worked lse")
    outs = ora.emulate_ring([q[i:i + 1] for i in range(n)], [(k[j:j + 1], v[j:j + 1]) for j in range(n)],
                            gold["scale"])
    _close([o[0][0, 0, 0] for o in outs], exp["A"], 1e-14, 0, "ring emulation A")


def pin_ring_emulation():
    """N devices rotating blocks == unsplit attention, causal and non-causal."""
    g = _rng(81)
    n, blen, Hq, Hkv, D = 4, 5, 4, 2, 8
    q = g.standard_normal((n * blen, Hq, D))
    k = g.standard_normal((n * blen, Hkv, D))
    v = g.standard_normal((n * blen, Hkv, D))
    s = 1.0 / math.sqrt(D)
    for causal in (False, True):
        a_ref, _, _, lse_ref = ora.attend(q, k, v, s, None, None, causal)
        outs = ora.emulate_ring([q[i * blen:(i + 1) * blen] for i in range(n)],
                                [(k[j * blen:(j + 1) * blen], v[j * blen:(j + 1) * blen]) for j in range(n)],
                                s, causal)
        for i, (a, lse) in enumerate(outs):
            _close(a, a_ref[i * blen:(i + 1) * blen], 1e-12, 1e-13, f"ring dev {i} causal={causal}")
            _close(lse, lse_ref[i * blen:(i + 1) * blen], 1e-12, 1e-13, "ring lse")


# --- fan-out decode (AHBM 1.1, 1.3, 3.4) ---------------------------------------

def pin_fanout_decode():
    """Fan-out decode == merge(prefix partial, own-suffix partial) == brute force."""
    g = _rng(91)
    nb, Hq, Hkv, D, P, S = 3, 4, 2, 8, 10, 4
    q = g.standard_normal((nb, Hq, D))
    pk = g.standard_normal((P, Hkv, D))
    pv = g.standard_normal((P, Hkv, D))
    sk = g.standard_normal((nb, S, Hkv, D))
    sv = g.standard_normal((nb, S, Hkv, D))
    s = 1.0 / math.sqrt(D)
    a, lse = ora.fanout_decode(q, pk, pv, sk, sv, s)
    pre = ora.fanout_state_rows(q, pk, pv, s)
    for b in range(nb):
        suf = ora.fanout_state_rows(q[b:b + 1], sk[b], sv[b], s)
        merged = ora.merge([tuple(x[b:b + 1] for x in pre), suf])
        a2, lse2 = ora.finalize(*merged)
        _close(a2[0], a[b], 1e-12, 1e-13, "fanout merge")
        _close(lse2[0], lse[b], 1e-12, 1e-13, "fanout lse")
        keys = np.concatenate([pk, sk[b]])
        vals = np.concatenate([pv, sv[b]])
        A, _, _, LSE = brute.attend(q[b:b + 1].tolist(), keys.tolist(), vals.tolist(), s)
        _close(a[b], A[0], 1e-13, 1e-14, "fanout brute")
        _close(lse[b], LSE[0], 1e-13, 0, "fanout brute lse")


def pin_fanout_prefill():
    """Fan-out prefill: T = 1 is the decode; each new token equals a one-token
    decode over the suffix cut just after it (pins the causal offset); brute force."""
    g = _rng(93)
    nb, T, Hq, Hkv, D, P, S = 2, 3, 4, 2, 8, 9, 5
    q = g.standard_normal((nb, T, Hq, D))
    pk = g.standard_normal((P, Hkv, D))
    pv = g.standard_normal((P, Hkv, D))
    sk = g.standard_normal((nb, S, Hkv, D))
    sv = g.standard_normal((nb, S, Hkv, D))
    s = 1.0 / math.sqrt(D)
    a, lse = ora.fanout_prefill(q, pk, pv, sk, sv, s)
    a1, lse1 = ora.fanout_prefill(q[:, -1:], pk, pv, sk, sv, s)
    ad, lsed = ora.fanout_decode(q[:, -1], pk, pv, sk, sv, s)
    _close(a1[:, 0], ad, 1e-13, 1e-14, "prefill T=1 vs decode")
    _close(lse1[:, 0], lsed, 1e-13, 0, "prefill T=1 vs decode lse")
    for i in range(T):
        cut = S - T + i + 1
        ai, lsei = ora.fanout_decode(q[:, i], pk, pv, sk[:, :cut], sv[:, :cut], s)
        _close(a[:, i], ai, 1e-13, 1e-14, f"prefill token {i}")
        _close(lse[:, i], lsei, 1e-13, 0, f"prefill token {i} lse")
    for b in range(nb):
        keys = np.concatenate([pk, sk[b]])
        vals = np.concatenate([pv, sv[b]])
        q_pos = [P + S - T + i for i in range(T)]
        A, _, _, LSE = brute.attend(q[b].tolist(), keys.tolist(), vals.tolist(), s, q_pos, list(range(P + S)), True)
        _close(a[b], A, 1e-13, 1e-14, "prefill brute")
        _close(lse[b], LSE, 1e-13, 0, "prefill brute lse")


def _pages_of(x, page_len):
    """Cut x [n, ...] into page_len-row pages (the last zero-padded)."""
    n = x.shape[0]
    out = []
    for p0 in range(0, n, page_len):
        page = np.zeros((page_len,) + x.shape[1:])
        page[:min(page_len, n - p0)] = x[p0:p0 + page_len]
        out.append(page)
    return out


def pin_fanout_paged():
    """Paged fan-out: pages scattered over a pool in a random order give the
    contiguous fan-out prefill exactly; a prefix page id of -1 (a hole) gives
    the prefill over the prefix with that page's tokens removed; any other id
    outside the pool is rejected as a corrupt table."""
    g = _rng(97)
    nb, T, Hq, Hkv, D, P, S, PL = 2, 3, 4, 2, 8, 10, 6, 4
    q = g.standard_normal((nb, T, Hq, D))
    pk, pv = g.standard_normal((P, Hkv, D)), g.standard_normal((P, Hkv, D))
    sk, sv = g.standard_normal((nb, S, Hkv, D)), g.standard_normal((nb, S, Hkv, D))
    s = 1.0 / math.sqrt(D)
    kp, vp = _pages_of(pk, PL), _pages_of(pv, PL)
    ks = [_pages_of(sk[b], PL) for b in range(nb)]
    vs = [_pages_of(sv[b], PL) for b in range(nb)]
    n_used = len(kp) + sum(len(x) for x in ks)
    n_pool = n_used + 2
    perm = g.permutation(n_pool)
    k_pool = g.standard_normal((n_pool, PL, Hkv, D))   # unused pool pages hold noise
    v_pool = g.standard_normal((n_pool, PL, Hkv, D))
    slots = iter(perm[:n_used])
    prefix_pages = []
    for kpg, vpg in zip(kp, vp):
        i = next(slots)
        k_pool[i], v_pool[i] = kpg, vpg
        prefix_pages.append(i)
    suffix_pages = []
    for b in range(nb):
        row = []
        for kpg, vpg in zip(ks[b], vs[b]):
            i = next(slots)
            k_pool[i], v_pool[i] = kpg, vpg
            row.append(i)
        suffix_pages.append(row)
    a, lse = ora.fanout_paged(q, k_pool, v_pool, prefix_pages, suffix_pages, PL, P, S, s)
    ra, rlse = ora.fanout_prefill(q, pk, pv, sk, sv, s)
    _close(a, ra, 1e-13, 1e-14, "paged vs contiguous")
    _close(lse, rlse, 1e-13, 0, "paged vs contiguous lse")
    hole = list(prefix_pages)
    hole[1] = -1
    a2, lse2 = ora.fanout_paged(q, k_pool, v_pool, hole, suffix_pages, PL, P, S, s)
    keep = np.r_[0:PL, 2 * PL:P]
    ra2, rlse2 = ora.fanout_prefill(q, pk[keep], pv[keep], sk, sv, s)
    _close(a2, ra2, 1e-13, 1e-14, "paged with a hole page")
    _close(lse2, rlse2, 1e-13, 0, "paged with a hole page lse")
    for bad_id in (n_pool, n_pool + 5, -2):
        bad = list(prefix_pages)
        bad[1] = bad_id
        try:
            ora.fanout_paged(q, k_pool, v_pool, bad, suffix_pages, PL, P, S, s)
        except ValueError:
            continue
        raise AssertionError(f"page id {bad_id} outside the pool was accepted")


def _loss_and_grads_fd(q, k, v, d_out, scale, q_pos, k_pos, causal, eps=1e-6):
    """Central finite differences of sum(A * d_out) -- independent of any gradient formula."""
    def loss(q_, k_, v_):
        a, _, _, _ = ora.attend(q_, k_, v_, scale, q_pos, k_pos, causal)
        return float((a * d_out).sum())
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        x = base[which]
        gx = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = loss(*base)
            x[idx] = old - eps
            lm = loss(*base)
            x[idx] = old
            gx[idx] = (lp - lm) / (2 * eps)
        grads.append(gx)
    return grads


def pin_attention_grads_finite_differences():
    """dQ, dK, dV against central finite differences of the forward, GQA, causal and not."""
    g = _rng(95)
    T, L, Hq, Hkv, D = 4, 5, 4, 2, 3
    q = g.standard_normal((T, Hq, D))
    k = g.standard_normal((L, Hkv, D))
    v = g.standard_normal((L, Hkv, D))
    d_out = g.standard_normal((T, Hq, D))
    s = 0.7
    for causal in (False, True):
        q_pos = np.arange(T) + 1
        k_pos = np.arange(L)
        dq, dk, dv = ora.attention_grads(q, k, v, d_out, s, q_pos, k_pos, causal)
        fq, fk, fv = _loss_and_grads_fd(q, k, v, d_out, s, q_pos, k_pos, causal)
        _close(dq, fq, 1e-6, 1e-8, "dQ vs finite differences")
        _close(dk, fk, 1e-6, 1e-8, "dK vs finite differences")
        _close(dv, fv, 1e-6, 1e-8, "dV vs finite differences")


def pin_attention_grads_autograd():
    """dQ, dK, dV against torch autograd (float64, CPU) of a plain masked softmax attention."""
    import torch
    g = _rng(96)
    T, L, Hq, Hkv, D = 6, 9, 4, 2, 5
    q = g.standard_normal((T, Hq, D))
    k = g.standard_normal((L, Hkv, D))
    v = g.standard_normal((L, Hkv, D))
    d_out = g.standard_normal((T, Hq, D))
    s = 1.0 / math.sqrt(D)
    q_pos = np.arange(T) + 3
    k_pos = np.arange(L)
    dq, dk, dv = ora.attention_grads(q, k, v, d_out, s, q_pos, k_pos, True)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    G = Hq // Hkv
    kk = tk.repeat_interleave(G, dim=1)
    vv = tv.repeat_interleave(G, dim=1)
    z = torch.einsum("thd,lhd->htl", tq, kk) * s
    mask = torch.tensor(k_pos[None, :] <= q_pos[:, None])
    z = z.masked_fill(~mask[None], float("-inf"))
    a = torch.einsum("htl,lhd->thd", torch.softmax(z, dim=-1), vv)
    (a * torch.tensor(d_out)).sum().backward()
    _close(dq, tq.grad.numpy(), 1e-12, 1e-13, "dQ vs autograd")
    _close(dk, tk.grad.numpy(), 1e-12, 1e-13, "dK vs autograd")
    _close(dv, tv.grad.numpy(), 1e-12, 1e-13, "dV vs autograd")


def pin_backward_ring_is_full_gradient():
    """Reverse-ring blockwise backward (per-block terms with the row's final
    softmax) sums to the gradient of plain causal attention."""
    g = _rng(97)
    n, B, Hq, Hkv, D = 3, 4, 4, 2, 6
    S = n * B
    q = g.standard_normal((S, Hq, D))
    k = g.standard_normal((S, Hkv, D))
    v = g.standard_normal((S, Hkv, D))
    d_out = g.standard_normal((S, Hq, D))
    s = 1.0 / math.sqrt(D)
    dq, dk, dv = ora.attention_grads(q, k, v, d_out, s, np.arange(S), np.arange(S), True)
    blocks = [slice(i * B, (i + 1) * B) for i in range(n)]
    dqs, dks, dvs = ora.backward_ring([q[b] for b in blocks], [(k[b], v[b]) for b in blocks],
                                      [d_out[b] for b in blocks], s, causal=True, block_len=B)
    _close(np.concatenate(dqs), dq, 1e-12, 1e-13, "ring dQ")
    _close(np.concatenate(dks), dk, 1e-12, 1e-13, "ring dK")
    _close(np.concatenate(dvs), dv, 1e-12, 1e-13, "ring dV")


def pin_finalize_empty():
    a, lse = ora.finalize(np.array([-np.inf, 0.5]), np.array([0.0, 2.0]), np.array([[0.0, 0.0], [1.0, -3.0]]))
    assert np.all(a[0] == 0) and np.isneginf(lse[0])
    _close(a[1], [0.5, -1.5], 0, 0, "finalize")
    _close(lse[1], 0.5 + math.log(2.0), 1e-15, 0, "finalize lse")


# ---------------------------------------------------------------- load-balanced causal shares
# [RAC] section 5 (Striped vs. Zigzag Ring Attention).

def pin_zigzag_printed_allocation():
    """Zigzag ownership equals the page's printed 4-GPU allocation (GPU k holds c_k and c_{2N-1-k})."""
    g = json.load(open(os.path.join(GOLDEN, "zigzag_allocation_printed.json")))
    n, c = g["n_devices"], 5
    S = 2 * n * c
    for k, chunks in g["chunks_per_device"].items():
        want = np.concatenate([np.arange(ci * c, (ci + 1) * c) for ci in chunks])
        got = ora.zigzag_tokens(S, n, int(k))
        assert np.array_equal(got, want), ("zigzag", k, got, want)


def pin_layouts_partition():
    """Every layout hands each token to exactly one device, S / n tokens each."""
    for owner in (ora.contiguous_tokens, ora.striped_tokens, ora.zigzag_tokens):
        for n in (1, 2, 4, 8):
            S = 16 * n
            parts = [np.asarray(owner(S, n, k)) for k in range(n)]
            assert all(len(p) == S // n for p in parts), owner.__name__
            assert np.array_equal(np.sort(np.concatenate(parts)), np.arange(S)), owner.__name__


def pin_layout_pair_counts():
    """Closed forms of the causal pairs per device and ring step, from the layouts' definitions:
    contiguous B^2 / B(B+1)/2 / 0 for a block before / at / after the device's own; zigzag
    2C^2 + C at step 0 and 2C^2 after (equal on every device); striped B(B+1)/2 when the
    source device index is <= k, else B(B-1)/2.  The totals are the causal triangle S(S+1)/2."""
    for n in (2, 4, 8):
        B = 12
        S, C = n * B, B // 2
        tot = {}
        for k in range(n):
            for t in range(n):
                src = (k - t) % n
                cont = ora.ring_step_pairs(ora.contiguous_tokens, S, n, k, t)
                assert cont == (B * B if src < k else B * (B + 1) // 2 if src == k else 0), ("cont", n, k, t)
                zz = ora.ring_step_pairs(ora.zigzag_tokens, S, n, k, t)
                assert zz == (2 * C * C + C if t == 0 else 2 * C * C), ("zigzag", n, k, t)
                st = ora.ring_step_pairs(ora.striped_tokens, S, n, k, t)
                assert st == (B * (B + 1) // 2 if src <= k else B * (B - 1) // 2), ("striped", n, k, t)
                for name, v in (("c", cont), ("z", zz), ("s", st)):
                    tot[name] = tot.get(name, 0) + v
        assert all(v == S * (S + 1) // 2 for v in tot.values()), tot


def pin_zigzag_ring_exact():
    """Walking the zigzag ring with the recurrence reproduces plain causal attention
    (the page's exact causal equivalence)."""
    rng = _rng(31)
    n, c, Hq, Hkv, D = 3, 7, 4, 2, 8
    S = 2 * n * c
    q = rng.standard_normal((S, Hq, D))
    k = rng.standard_normal((S, Hkv, D))
    v = rng.standard_normal((S, Hkv, D))
    scale = 1.0 / math.sqrt(D)
    a_ref, _, _, lse_ref = brute_free_attend(q, k, v, scale)
    for dev in range(n):
        mine = ora.zigzag_tokens(S, n, dev)
        st = ora.init_state(len(mine), Hq, D)
        for t in range(n):
            src = ora.zigzag_tokens(S, n, (dev - t) % n)
            st = ora.online_step(st, q[mine], k[src], v[src], scale, mine, src, causal=True)
        a, lse = ora.finalize(*st)
        _close(a, a_ref[mine], 0, 1e-12, "zigzag A")
        _close(lse, lse_ref[mine], 0, 1e-12, "zigzag lse")


def brute_free_attend(q, k, v, scale):
    """Causal attention written out with scipy's softmax (not the oracle's own state code)."""
    S, Hq, D = q.shape
    G = Hq // k.shape[1]
    a = np.zeros_like(q)
    lse = np.zeros((S, Hq))
    for h in range(Hq):
        g = h // G
        z = scale * (q[:, h, :] @ k[:, g, :].T)
        z = np.where(np.tril(np.ones((S, S), dtype=bool)), z, -np.inf)
        a[:, h, :] = scipy.special.softmax(z, axis=1) @ v[:, g, :]
        lse[:, h] = scipy.special.logsumexp(z, axis=1)
    return a, None, None, lse


ALL_PINS = [
    pin_brute_force_tiny,
    pin_scipy_softmax_logsumexp,
    pin_closed_forms,
    pin_shift_invariance,
    pin_order_invariance,
    pin_split_merge,
    pin_causal_future_keys,
    pin_large_logits,
    pin_ring_schedule_printed,
    pin_ring_simulator_worked_example,
    pin_ring_emulation,
    pin_fanout_decode,
    pin_fanout_prefill,
    pin_fanout_paged,
    pin_attention_grads_finite_differences,
    pin_attention_grads_autograd,
    pin_backward_ring_is_full_gradient,
    pin_finalize_empty,
    pin_zigzag_printed_allocation,
    pin_layouts_partition,
    pin_layout_pair_counts,
    pin_zigzag_ring_exact,
]
