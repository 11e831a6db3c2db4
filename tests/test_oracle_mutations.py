"""Plant plausible mistakes in the oracle (CPU only) and check a pin catches each.

A pin set that a dropped term, a wrong sign or index, or a transposed operand
slips through would not be pinning anything.
"""

import numpy as np
import pytest

from oracle import attention as ora
from tests import oracle_pins

_orig_state_fn = ora.softmax_state
_orig_merge = ora.merge
_orig_online_step = ora.online_step
_orig_finalize = ora.finalize


def _no_scale(q_rows, k_rows, scale):
    return q_rows @ k_rows.T


def _strict_causal(q_pos, k_pos):
    return k_pos[None, :] < q_pos[:, None]


def _reversed_causal(q_pos, k_pos):
    return k_pos[None, :] >= q_pos[:, None]


def _modulo_gqa(h, n_q_heads, n_kv_heads):
    return h % n_kv_heads


def _unshifted_softmax(z, v_rows):
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.exp(z)
        m = z.max(axis=1) if z.shape[1] else np.full(z.shape[0], -np.inf)
        l = w.sum(axis=1) * np.exp(-m)
        o = (w @ v_rows) * np.exp(-m)[:, None]
    return m, l, o


def _v_is_k(z, v_rows):
    m, l, o = _orig_state_fn(z, v_rows)
    return m, l, o[:, ::-1].copy()


def _dropped_l_term(z, v_rows):
    m, l, o = _orig_state_fn(z, v_rows)
    return m, np.ones_like(l), o


def _merge_no_weights(parts):
    ms = np.stack([p[0] for p in parts])
    return ms.max(axis=0), sum(p[1] for p in parts), sum(p[2] for p in parts)


def _merge_min(parts):
    ms = np.stack([np.asarray(p[0]) for p in parts])
    m_star = np.where(np.isneginf(ms), np.inf, ms).min(axis=0)
    m_star = np.where(np.isinf(m_star), -np.inf, m_star)
    base = np.where(np.isneginf(m_star), 0.0, m_star)
    w = np.where(np.isneginf(ms), 0.0, np.exp(ms - base[None]))
    return m_star, (w * np.stack([p[1] for p in parts])).sum(0), (w[..., None] * np.stack([p[2] for p in parts])).sum(0)


def _online_no_alpha_on_o(st, q, k_blk, v_blk, scale, q_pos=None, k_pos_blk=None, causal=False):
    m_old, l_old, o_old = st
    m_new, l_new, o_new = _orig_online_step(st, q, k_blk, v_blk, scale, q_pos, k_pos_blk, causal)
    fresh = _orig_online_step(ora.init_state(*o_old.shape), q, k_blk, v_blk, scale, q_pos, k_pos_blk, causal)
    # O_new = O_old + P V (rescale of the old accumulator dropped)
    base = np.where(np.isneginf(m_new), 0.0, m_new)
    fb = np.where(np.isneginf(fresh[0]), 0.0, fresh[0])
    pv = fresh[2] * np.exp(fb - base)[..., None]
    return m_new, l_new, o_old + pv


def _finalize_no_log(m, l, o):
    a, lse = _orig_finalize(m, l, o)
    return a, np.where(np.isneginf(lse), lse, m + l)


def _ring_wrong_direction(k, n):
    return [(k + t) % n for t in range(n)]


def _zigzag_mirror_off_by_one(seq_len, n, k):
    c = seq_len // (2 * n)
    second = (2 * n - k) % (2 * n)
    return np.concatenate([np.arange(k * c, (k + 1) * c), np.arange(second * c, (second + 1) * c)])


def _striped_shifted(seq_len, n, k):
    return np.array([i for i in range(seq_len) if i % n == (k + 1) % n], dtype=np.int64)


def _pairs_strict(q_pos, k_pos):
    return int((np.asarray(k_pos)[None, :] < np.asarray(q_pos)[:, None]).sum())


_orig_fanout_prefill = ora.fanout_prefill


def _prefill_offset_by_one(q, prefix_k, prefix_v, suffix_k, suffix_v, scale):
    # the new tokens placed one position early: each misses its own key
    q = np.asarray(q, dtype=np.float64)
    nb, T = q.shape[:2]
    P = np.asarray(prefix_k).shape[0]
    S = np.asarray(suffix_k).shape[1]
    a = np.empty(q.shape)
    lse = np.empty(q.shape[:3])
    for b in range(nb):
        keys = np.concatenate([prefix_k, suffix_k[b]])
        vals = np.concatenate([prefix_v, suffix_v[b]])
        ab, _, _, lb = ora.attend(q[b], keys, vals, scale, P + S - T - 1 + np.arange(T), np.arange(P + S), True)
        a[b], lse[b] = ab, lb
    return a, lse


_orig_grads = ora.attention_grads


def _grads_without_delta(q, k, v, d_out, scale, q_pos=None, k_pos=None, causal=False, key_subset=None):
    # dz = p * dp: the row term sum_j p_ij dp_ij of the softmax Jacobian dropped
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    T, Hq, D = q.shape
    L, Hkv, _ = k.shape
    q_pos = np.arange(T) if q_pos is None else np.asarray(q_pos)
    k_pos = np.arange(L) if k_pos is None else np.asarray(k_pos)
    keep = np.ones(L, dtype=bool)
    if key_subset is not None:
        keep[:] = False
        keep[np.asarray(key_subset)] = True
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        z = scale * (q[:, h] @ k[:, g].T)
        vis = (k_pos[None, :] <= q_pos[:, None]) if causal else np.ones((T, L), dtype=bool)
        z = np.where(vis, z, -np.inf)
        w = np.where(vis, np.exp(z - z.max(axis=1, keepdims=True)), 0.0)
        p = w / w.sum(axis=1, keepdims=True)
        dz = p * (d_out[:, h] @ v[:, g].T)
        pk, dzk = np.where(keep[None], p, 0.0), np.where(keep[None], dz, 0.0)
        dv[:, g] += pk.T @ d_out[:, h]
        dq[:, h] = scale * (dzk @ k[:, g])
        dk[:, g] += scale * (dzk.T @ q[:, h])
    return dq, dk, dv


def _grads_dk_unscaled(q, k, v, d_out, scale, q_pos=None, k_pos=None, causal=False, key_subset=None):
    dq, dk, dv = _orig_grads(q, k, v, d_out, scale, q_pos, k_pos, causal, key_subset)
    return dq, dk / scale, dv


_orig_page_gather = ora.page_gather


def _page_row_shifted(pool, pages, n, page_len, n_pool):
    shifted = [np.roll(np.asarray(x), 1, axis=0) for x in pool]
    return _orig_page_gather(np.stack(shifted), pages, n, page_len, n_pool)


MUTATIONS = {
    "page row offset by one": ("page_gather", _page_row_shifted),
    "softmax Jacobian row term dropped": ("attention_grads", _grads_without_delta),
    "dK missing the scale": ("attention_grads", _grads_dk_unscaled),
    "prefill new tokens one position early": ("fanout_prefill", _prefill_offset_by_one),
    "zigzag mirror chunk off by one": ("zigzag_tokens", _zigzag_mirror_off_by_one),
    "striped residue shifted": ("striped_tokens", _striped_shifted),
    "pair count excludes the diagonal": ("visible_pairs", _pairs_strict),
    "dropped scale": ("scaled_logits", _no_scale),
    "diagonal excluded from causal mask": ("causal_visible", _strict_causal),
    "causal mask reversed": ("causal_visible", _reversed_causal),
    "GQA head mapping h % Hkv": ("kv_head_of", _modulo_gqa),
    "softmax without max shift": ("softmax_state", _unshifted_softmax),
    "output accumulates a permuted V": ("softmax_state", _v_is_k),
    "denominator term dropped": ("softmax_state", _dropped_l_term),
    "merge without exp(m_s - m*) weights": ("merge", _merge_no_weights),
    "merge takes the min": ("merge", _merge_min),
    "recurrence drops the O rescale": ("online_step", _online_no_alpha_on_o),
    "LSE without the log": ("finalize", _finalize_no_log),
    "ring rotates the wrong way": ("ring_order", _ring_wrong_direction),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ora, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake: {name}"
