"""A batch of independent sequences in one call (ba_problem.batch).

q is [batch, q_len, Hq, D] and every K/V block [batch, len, Hkv, D] (or a
[len, Hkv, D] block shared by all sequences); state, output and LSE rows are
(b * q_len + t) * Hq + h.  A sequence's rows take the same tiles, visits and
instructions as they would in a call of their own, so on the walk (and the
fp32 and backward kernels) a batched call equals one call per sequence bit for
bit; the split path plans its key chunks for the whole batch, so there the
comparison is against the oracle.  Every case prints its shape and seed before
it touches the GPU.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_blockwise_long_amd import blockattn as ba
from exact_blockwise_long_amd import synth
from oracle import attention as ora
from tests import helpers as H

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ba.load()
    yield
    torch.cuda.synchronize()


def make_batch(seed, B, T, Hq, Hkv, D, L, dtype="bf16", shared_kv=False):
    g = synth.rng(seed)
    q = synth.normal(g, (B, T, Hq, D), 0.5, dtype)
    kv_shape = (L, Hkv, D) if shared_kv else (B, L, Hkv, D)
    k = synth.normal(g, kv_shape, 0.5, dtype)
    v = synth.normal(g, kv_shape, 0.5, dtype)
    return q, k, v


def blocks_of(kd, vd, lens, pos0=0, b=None):
    """Blocks over the key axis of [.., L, Hkv, D] tensors (the sequence b's own when given)."""
    out, off = [], 0
    for n in lens:
        if b is None:
            out.append((kd[..., off:off + n, :, :], vd[..., off:off + n, :, :], pos0 + off))
        else:
            out.append((kd[b, off:off + n], vd[b, off:off + n], pos0 + off))
        off += n
    return out


def per_sequence(qd, kd, vd, lens, order, b, shared, **kw):
    blocks = blocks_of(kd, vd, lens) if shared else blocks_of(kd, vd, lens, b=b)
    T, Hq, D = qd.shape[1:]
    st = ba.new_state(T * Hq, D)
    return ba.fwd_block_finalize(qd[b], blocks, order, st, reset=True, **kw)


def oracle_seq(q, k, v, b, T, q_pos0, causal, scale, shared):
    kk = k.f64() if shared else k.f64()[b]
    vv = v.f64() if shared else v.f64()[b]
    a, _, _, lse = ora.attend(q.f64()[b], kk, vv, scale, q_pos0 + np.arange(T), None, causal)
    return a, lse


WALK_CASES = [
    # (seed, B, T, Hq, Hkv, D, lens, order, q_pos0, causal, shared_kv)
    (101, 3, 300, 8, 2, 128, [200, 77, 129, 64], [2, 0, 3, 1], 350, True, False),
    (102, 2, 130, 4, 4, 64, [65, 128, 31], [1, 2, 0], 150, True, False),
    (103, 4, 97, 16, 2, 128, [160, 96], [1, 0], 0, False, True),
]


@pytest.mark.parametrize("case", WALK_CASES, ids=lambda c: f"seed{c[0]}")
def test_batch_walk_equals_one_call_per_sequence(case):
    seed, B, T, Hq, Hkv, D, lens, order, q_pos0, causal, shared = case
    announce(f"batch walk seed {seed} B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} order={order} "
             f"q_pos0={q_pos0} causal={causal} shared_kv={shared}")
    q, k, v = make_batch(seed, B, T, Hq, Hkv, D, sum(lens), shared_kv=shared)
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    kw = dict(n_kv_heads=Hkv, q_pos0=q_pos0, causal=causal, split_mode=1)
    st = ba.new_state(B * T * Hq, D)
    out, lse = ba.fwd_block_finalize(qd, blocks_of(kd, vd, lens), order, st, reset=True, **kw)
    # the same visits one call at a time, state carried between calls, then finalised
    st2 = ba.new_state(B * T * Hq, D)
    for i, j in enumerate(order):
        ba.fwd_block(qd, blocks_of(kd, vd, lens), [j], st2, reset=(i == 0), **kw)
    out2, lse2 = ba.finalize(st2)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    R = T * Hq
    scale = 1.0 / np.sqrt(D)
    for b in range(B):
        o1, l1 = per_sequence(qd, kd, vd, lens, order, b, shared, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out[b * R:(b + 1) * R], o1) and torch.equal(lse[b * R:(b + 1) * R], l1), \
            f"sequence {b} differs from its own call"
        a_ref, lse_ref = oracle_seq(q, k, v, b, T, q_pos0, causal, scale, shared)
        H.assert_bf16_out(H.host(out2[b * R:(b + 1) * R]).reshape(T, Hq, D), a_ref, f"seq {b} (per visit)")
        H.assert_close(H.host(lse2[b * R:(b + 1) * R]).reshape(T, Hq), lse_ref, H.BF16_LSE, f"seq {b} lse")


@pytest.mark.parametrize("seed", range(7000, 7024))
def test_batch_random(seed):
    """Seeded random batched problems: batch 2-5, group sizes 1-8, ragged and
    empty blocks, causal or not, shared or per-sequence keys, every split mode.
    Without a key split each sequence must equal its own call bit for bit; every
    sequence must match the oracle."""
    g = np.random.Generator(np.random.PCG64(seed))
    B = int(g.choice([2, 3, 5]))
    D = int(g.choice([64, 128]))
    Hkv = int(g.choice([1, 2, 8]))
    Hq = Hkv * int(g.choice([1, 4, 8]))
    n_blocks = int(g.integers(1, 5))
    lens = [int(x) for x in g.choice([0, 1, 63, 64, 65, 129, 300], size=n_blocks)]
    if sum(lens) == 0:
        lens[0] = 40
    L = sum(lens)
    T = int(g.choice([1, 17, 65, 200]))
    causal = bool(g.integers(0, 2))
    q_pos0 = max(int(g.integers(-T // 2, L + 20)), 0) if causal else 0
    shared = bool(g.integers(0, 2))
    mode = int(g.integers(0, 3))
    order = g.permutation(n_blocks).tolist()
    announce(f"batch random seed {seed}: B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} order={order} "
             f"q_pos0={q_pos0} causal={causal} shared_kv={shared} split_mode={mode}")
    q, k, v = make_batch(seed, B, T, Hq, Hkv, D, L, shared_kv=shared)
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    kw = dict(n_kv_heads=Hkv, q_pos0=q_pos0, causal=causal, split_mode=mode)
    st = ba.new_state(B * T * Hq, D)
    out, lse = ba.fwd_block_finalize(qd, blocks_of(kd, vd, lens), order, st, reset=True, **kw)
    torch.cuda.synchronize()
    R = T * Hq
    for b in range(B):
        if mode == 1:
            o1, l1 = per_sequence(qd, kd, vd, lens, order, b, shared, **kw)
            torch.cuda.synchronize()
            assert torch.equal(out[b * R:(b + 1) * R], o1) and torch.equal(lse[b * R:(b + 1) * R], l1), \
                f"sequence {b} differs from its own call"
        a_ref, lse_ref = oracle_seq(q, k, v, b, T, q_pos0, causal, 1.0 / np.sqrt(D), shared)
        H.assert_bf16_out(H.host(out[b * R:(b + 1) * R]).reshape(T, Hq, D), a_ref, f"seq {b}")
        H.assert_close(H.host(lse[b * R:(b + 1) * R]).reshape(T, Hq), lse_ref, H.BF16_LSE, f"seq {b} lse")


def test_batch_split_against_oracle():
    seed, B, T, Hq, Hkv, D, lens, order = 104, 3, 40, 8, 2, 128, [700, 333], [1, 0]
    announce(f"batch split seed {seed} B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} causal")
    q, k, v = make_batch(seed, B, T, Hq, Hkv, D, sum(lens))
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    kw = dict(n_kv_heads=Hkv, q_pos0=1000, causal=True, split_mode=2)
    assert ba.fwd_workspace_bytes(qd, blocks_of(kd, vd, lens), order, **kw) > 0
    st = ba.new_state(B * T * Hq, D)
    out, lse = ba.fwd_block_finalize(qd, blocks_of(kd, vd, lens), order, st, reset=True, **kw)
    torch.cuda.synchronize()
    R = T * Hq
    for b in range(B):
        a_ref, lse_ref = oracle_seq(q, k, v, b, T, 1000, True, 1.0 / np.sqrt(D), False)
        H.assert_bf16_out(H.host(out[b * R:(b + 1) * R]).reshape(T, Hq, D), a_ref, f"split seq {b}")
        H.assert_close(H.host(lse[b * R:(b + 1) * R]).reshape(T, Hq), lse_ref, H.BF16_LSE, f"split seq {b} lse")


def test_batch_shard_states_and_merge():
    seed, B, T, Hq, Hkv, D, lens = 105, 2, 24, 8, 1, 128, [512, 300, 260]
    announce(f"batch shard states seed {seed} B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens}")
    q, k, v = make_batch(seed, B, T, Hq, Hkv, D, sum(lens))
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    states = [ba.new_state(B * T * Hq, D) for _ in lens]
    ba.shard_states(qd, blocks_of(kd, vd, lens), states, n_kv_heads=Hkv)
    merged = ba.new_state(B * T * Hq, D)
    ba.merge_states(states, merged)
    out, lse = ba.finalize(merged)
    torch.cuda.synchronize()
    R = T * Hq
    for b in range(B):
        a_ref, lse_ref = oracle_seq(q, k, v, b, T, 0, False, 1.0 / np.sqrt(D), False)
        H.assert_bf16_out(H.host(out[b * R:(b + 1) * R]).reshape(T, Hq, D), a_ref, f"shard seq {b}")
        H.assert_close(H.host(lse[b * R:(b + 1) * R]).reshape(T, Hq), lse_ref, H.BF16_LSE, f"shard seq {b} lse")


def test_batch_f32_equals_one_call_per_sequence():
    seed, B, T, Hq, Hkv, D, lens, order = 106, 2, 70, 4, 2, 64, [50, 45], [1, 0]
    announce(f"batch f32 seed {seed} B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} causal")
    q, k, v = make_batch(seed, B, T, Hq, Hkv, D, sum(lens), dtype="f32")
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    kw = dict(n_kv_heads=Hkv, q_pos0=40, causal=True, split_mode=1)
    st = ba.new_state(B * T * Hq, D)
    out, lse = ba.fwd_block_finalize(qd, blocks_of(kd, vd, lens), order, st, reset=True, out_dtype=torch.float32,
                                     **kw)
    torch.cuda.synchronize()
    R = T * Hq
    for b in range(B):
        o1, l1 = per_sequence(qd, kd, vd, lens, order, b, False, out_dtype=torch.float32, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out[b * R:(b + 1) * R], o1) and torch.equal(lse[b * R:(b + 1) * R], l1)
        a_ref, lse_ref = oracle_seq(q, k, v, b, T, 40, True, 1.0 / np.sqrt(D), False)
        H.assert_close(H.host(out[b * R:(b + 1) * R]).reshape(T, Hq, D), a_ref, H.F32_TOL, f"f32 seq {b}")
    # the key split (chunks planned for the whole batch) against the oracle
    kw["split_mode"] = 2
    st = ba.new_state(B * T * Hq, D)
    out, lse = ba.fwd_block_finalize(qd, blocks_of(kd, vd, lens), order, st, reset=True, out_dtype=torch.float32,
                                     **kw)
    torch.cuda.synchronize()
    for b in range(B):
        a_ref, lse_ref = oracle_seq(q, k, v, b, T, 40, True, 1.0 / np.sqrt(D), False)
        H.assert_close(H.host(out[b * R:(b + 1) * R]).reshape(T, Hq, D), a_ref, H.F32_TOL, f"f32 split seq {b}")
        H.assert_close(H.host(lse[b * R:(b + 1) * R]).reshape(T, Hq), lse_ref, H.F32_TOL, f"f32 split seq {b} lse")


def test_batch_strided_query_view():
    """q as a view with a padded batch stride (and K/V with padded sequences)."""
    seed, B, T, Hq, Hkv, D, lens = 107, 3, 50, 8, 2, 128, [96, 64]
    announce(f"batch strided views seed {seed} B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens}")
    q, k, v = make_batch(seed, B, T + 7, Hq, Hkv, D, sum(lens) + 33)
    qd, kd, vd = H.to_device(q)[:, :T], H.to_device(k)[:, :sum(lens)], H.to_device(v)[:, :sum(lens)]
    assert not qd.is_contiguous()
    kw = dict(n_kv_heads=Hkv, q_pos0=80, causal=True, split_mode=1)
    st = ba.new_state(B * T * Hq, D)
    out, lse = ba.fwd_block_finalize(qd, blocks_of(kd, vd, lens), None, st, reset=True, **kw)
    torch.cuda.synchronize()
    R = T * Hq
    for b in range(B):
        o1, l1 = per_sequence(qd.contiguous(), kd.contiguous(), vd.contiguous(), lens, None, b, False, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out[b * R:(b + 1) * R], o1) and torch.equal(lse[b * R:(b + 1) * R], l1)


def test_batch_backward_equals_one_call_per_sequence():
    seed, B, T, Hq, Hkv, D, lens, order, q_pos0 = 108, 2, 300, 8, 2, 128, [200, 77, 129, 64], [2, 0, 3, 1], 350
    announce(f"batch backward seed {seed} B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} causal")
    g = synth.rng(seed)
    q = synth.normal(g, (B, T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (B, sum(lens), Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (B, sum(lens), Hkv, D), 0.5, "bf16")
    do = synth.normal(g, (B, T, Hq, D), 0.5, "bf16")
    qd, kd, vd, dod = (H.to_device(x) for x in (q, k, v, do))
    kw = dict(n_kv_heads=Hkv, q_pos0=q_pos0, causal=True)

    def grads(qx, dox, blocks):
        Bx = qx.shape[0] if qx.dim() == 4 else 1
        rows = Bx * T * Hq
        st = ba.new_state(rows, D)
        ba.fwd_block(qx, blocks, order, st, reset=True, split_mode=1, **kw)
        out, lse = ba.finalize(st)
        delta = ba.bwd_delta(out, dox)
        dq = torch.zeros(rows, D, dtype=torch.float32, device="cuda")
        shape = (lambda n: (Bx, n, Hkv, D)) if qx.dim() == 4 else (lambda n: (n, Hkv, D))
        dkv = [(torch.zeros(shape(n), dtype=torch.float32, device="cuda"),
                torch.zeros(shape(n), dtype=torch.float32, device="cuda")) for n in lens]
        ba.bwd_block(qx, dox, lse, delta, blocks, order, dq, dkv, **kw)
        return dq, dkv

    dq, dkv = grads(qd, dod, blocks_of(kd, vd, lens))
    torch.cuda.synchronize()
    R = T * Hq
    for b in range(B):
        dq1, dkv1 = grads(qd[b], dod[b], blocks_of(kd, vd, lens, b=b))
        torch.cuda.synchronize()
        assert torch.equal(dq[b * R:(b + 1) * R], dq1), f"dq of sequence {b}"
        for i, ((dk, dv), (dk1, dv1)) in enumerate(zip(dkv, dkv1)):
            assert torch.equal(dk[b], dk1) and torch.equal(dv[b], dv1), f"dk/dv of block {i}, sequence {b}"
    # and sequence 1 against the oracle's gradients
    kpos = np.arange(sum(lens))
    rq, rk, rv = ora.attention_grads(q.f64()[1], k.f64()[1], v.f64()[1], do.f64()[1], 1.0 / np.sqrt(D),
                                     q_pos0 + np.arange(T), kpos, True)
    got_dq = H.host(dq[R:2 * R]).reshape(T, Hq, D)
    got_dk = np.concatenate([H.host(x[0][1]) for x in dkv])
    got_dv = np.concatenate([H.host(x[1][1]) for x in dkv])
    for got, ref, name in ((got_dq, rq, "dQ"), (got_dk, rk, "dK"), (got_dv, rv, "dV")):
        err = np.abs(got - ref)
        assert np.all(np.isfinite(got)), name
        # the backward tests' bounds: max error / max |ref| <= 2e-2, mean error / mean |ref| <= 5e-3
        assert err.max() / np.abs(ref).max() <= 2e-2 and err.mean() / np.abs(ref).mean() <= 5e-3, name


def test_batch_backward_shared_keys_one_gradient_per_sequence():
    """Blocks shared by all sequences (3-D K/V under a batched q): each
    sequence gets its own dK/dV, equal to its own call's bit for bit."""
    seed, B, T, Hq, Hkv, D, lens, order, q_pos0 = 109, 3, 90, 8, 2, 64, [100, 60], [1, 0], 120
    announce(f"batch backward, shared keys, seed {seed} B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} causal")
    g = synth.rng(seed)
    q = synth.normal(g, (B, T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (sum(lens), Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (sum(lens), Hkv, D), 0.5, "bf16")
    do = synth.normal(g, (B, T, Hq, D), 0.5, "bf16")
    qd, kd, vd, dod = (H.to_device(x) for x in (q, k, v, do))
    blocks = blocks_of(kd, vd, lens)
    kw = dict(n_kv_heads=Hkv, q_pos0=q_pos0, causal=True)

    def grads(qx, dox, batched):
        rows = (B if batched else 1) * T * Hq
        st = ba.new_state(rows, D)
        ba.fwd_block(qx, blocks, order, st, reset=True, split_mode=1, **kw)
        out, lse = ba.finalize(st)
        delta = ba.bwd_delta(out, dox)
        dq = torch.zeros(rows, D, dtype=torch.float32, device="cuda")
        shape = (lambda n: (B, n, Hkv, D)) if batched else (lambda n: (n, Hkv, D))
        dkv = [(torch.zeros(shape(n), dtype=torch.float32, device="cuda"),
                torch.zeros(shape(n), dtype=torch.float32, device="cuda")) for n in lens]
        ba.bwd_block(qx, dox, lse, delta, blocks, order, dq, dkv, **kw)
        return dq, dkv

    dq, dkv = grads(qd, dod, True)
    torch.cuda.synchronize()
    R = T * Hq
    for b in range(B):
        dq1, dkv1 = grads(qd[b], dod[b], False)
        torch.cuda.synchronize()
        assert torch.equal(dq[b * R:(b + 1) * R], dq1), f"dq of sequence {b}"
        for i, ((dk, dv), (dk1, dv1)) in enumerate(zip(dkv, dkv1)):
            assert torch.equal(dk[b], dk1) and torch.equal(dv[b], dv1), f"dk/dv of block {i}, sequence {b}"
