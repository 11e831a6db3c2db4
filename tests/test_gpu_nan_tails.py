"""Keys past a K/V range are never read, and never reach a result (GPU,
through the C ABI).

Every block, prefix and suffix here sits at the start of a larger allocation
whose following rows hold bf16 NaN, +inf and -inf (inside the allocation, so
every address is mapped).  The ranges are ragged against every key tile the
kernels use (64 and 128 keys) and longer than one tile.  A tile that loaded
the rows after its range would multiply them by a zero weight, and 0 * inf
and 0 * NaN are NaN.  Each case is compared with the oracle element by element
and bit for bit with the same call on a twin allocation whose trailing rows
are finite.  The causal rule must drop future keys whatever they hold ("RingAttention
and Context Parallelism", section 2 box: a masked key's weight is exactly 0),
and a paged context's partial last page ends its keys ("AHBM Agentic Runtime
Architecture", section 3.1).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_blockwise_long_amd import blockattn as ba
from exact_blockwise_long_amd import synth
from exact_blockwise_long_amd import workloads as wl
from oracle import attention as ora
from tests import helpers as H

pytestmark = pytest.mark.gpu

GAP = 160            # trailing rows after each range: more than one 128-key tile
FINITE = 0x4040      # bf16 3.0, the twin allocation's trailing rows
LENS = [200, 333, 129, 71]   # ragged for 64- and 128-key tiles, three longer than a tile


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ba.load()
    yield
    torch.cuda.synchronize()


def with_tails(t: synth.Tensor, lens, poison: bool):
    """The rows of ``t`` [sum(lens), H, D] split into ranges of ``lens``, each
    followed by GAP trailing rows, as one device allocation.  Returns the
    device views of the ranges."""
    rows = t.storage
    tail_shape = (GAP,) + rows.shape[1:]
    if t.dtype == "bf16":
        tail = wl.poison_rows(tail_shape) if poison else np.full(tail_shape, FINITE, np.uint16)
    else:
        pat = np.array([np.nan, np.inf, -np.inf], dtype=np.float32)
        tail = np.resize(pat, tail_shape).astype(np.float32) if poison else np.full(tail_shape, 3.0, np.float32)
    parts, offs, off = [], [], 0
    for n in lens:
        parts += [rows[off:off + n], tail]
        offs.append(sum(p.shape[0] for p in parts[:-2]))
        off += n
    buf = H.to_device(synth.Tensor(np.ascontiguousarray(np.concatenate(parts, axis=0)), t.dtype))
    return [buf[o:o + n] for o, n in zip(offs, lens)]


def blocks_of(k, v, lens, poison):
    ks = with_tails(k, lens, poison)
    vs = with_tails(v, lens, poison)
    pos = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    return [(kb, vb, int(p)) for kb, vb, p in zip(ks, vs, pos)]


def check_vs_oracle(out, lse, q, k, v, q_pos0, causal, bf16, what):
    T, Hq, D = q.shape
    a_ref, _, _, lse_ref = ora.attend(q.f64(), k.f64(), v.f64(), 1.0 / np.sqrt(D), q_pos0 + np.arange(T), None,
                                      causal)
    got = H.host(out).reshape(T, Hq, D)
    if bf16:
        mx, mn = H.assert_bf16_out(got, a_ref, what)
        H.assert_close(H.host(lse).reshape(T, Hq), lse_ref, H.BF16_LSE, what + " lse")
    else:
        H.assert_close(got, a_ref, H.F32_TOL, what)
        H.assert_close(H.host(lse).reshape(T, Hq), lse_ref, H.F32_TOL, what + " lse")
        mx, mn = H.err_stats(got, a_ref)
    print(f"    {what}: max/mean abs err {mx:.2e}/{mn:.2e}", flush=True)


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("split_mode", [1, 2])
def test_fwd_ignores_trailing_rows(split_mode, causal, D):
    T, Hq, Hkv, q_pos0, seed = 300, 16, 2, 600, 501
    announce(f"fwd with NaN/inf after every block: split_mode {split_mode} causal {causal} D {D} T {T} "
             f"lens {LENS} seed {seed}")
    g = synth.rng(seed)
    q = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (sum(LENS), Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (sum(LENS), Hkv, D), 0.5, "bf16")
    qd = H.to_device(q)
    order = [2, 0, 3, 1]
    kw = dict(n_kv_heads=Hkv, q_pos0=q_pos0, causal=causal, split_mode=split_mode)
    res = {}
    for poison in (True, False):
        blocks = blocks_of(k, v, LENS, poison)
        st = ba.new_state(T * Hq, D)
        out, lse = ba.fwd_block_finalize(qd, blocks, order, st, reset=True, **kw)
        # one call per visit, then finalize
        st2 = ba.new_state(T * Hq, D)
        for i, j in enumerate(order):
            ba.fwd_block(qd, blocks, [j], st2, reset=(i == 0), **kw)
        out2, lse2 = ba.finalize(st2)
        torch.cuda.synchronize()
        res[poison] = (out, lse, out2, lse2)
    check_vs_oracle(res[True][0], res[True][1], q, k, v, q_pos0, causal, True, "one call")
    check_vs_oracle(res[True][2], res[True][3], q, k, v, q_pos0, causal, True, "call per visit")
    for a, b in zip(res[True], res[False]):
        assert torch.equal(a, b), "trailing NaN/inf rows changed the result"


def test_f32_ignores_trailing_rows():
    T, Hq, Hkv, D, q_pos0, seed = 90, 4, 2, 64, 300, 502
    lens = [70, 133, 65]
    announce(f"f32 fwd with NaN/inf after every block: T {T} lens {lens} seed {seed}")
    g = synth.rng(seed)
    q = synth.normal(g, (T, Hq, D), 1.0, "f32")
    k = synth.normal(g, (sum(lens), Hkv, D), 1.0, "f32")
    v = synth.normal(g, (sum(lens), Hkv, D), 1.0, "f32")
    blocks = blocks_of(k, v, lens, True)
    st = ba.new_state(T * Hq, D)
    ba.fwd_block(H.to_device(q), blocks, [1, 2, 0], st, reset=True, n_kv_heads=Hkv, q_pos0=q_pos0, causal=True)
    out, lse = ba.finalize(st, torch.float32)
    torch.cuda.synchronize()
    check_vs_oracle(out, lse, q, k, v, q_pos0, True, False, "f32 walk")


def test_shard_states_ignore_trailing_rows():
    T, Hq, Hkv, D, seed = 24, 16, 2, 128, 503
    announce(f"shard_states with NaN/inf after every block: T {T} lens {LENS} seed {seed}")
    g = synth.rng(seed)
    q = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (sum(LENS), Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (sum(LENS), Hkv, D), 0.5, "bf16")
    qd = H.to_device(q)
    res = {}
    for poison in (True, False):
        blocks = blocks_of(k, v, LENS, poison)
        states = [ba.new_state(T * Hq, D) for _ in LENS]
        ba.shard_states(qd, blocks, states, n_kv_heads=Hkv)
        merged = ba.new_state(T * Hq, D)
        ba.merge_states(states, merged)
        res[poison] = ba.finalize(merged)
        torch.cuda.synchronize()
    check_vs_oracle(res[True][0], res[True][1], q, k, v, 0, False, True, "shards + merge")
    assert torch.equal(res[True][0], res[False][0]) and torch.equal(res[True][1], res[False][1])


def test_backward_ignores_trailing_rows():
    T, Hq, Hkv, D, q_pos0, seed = 200, 8, 2, 128, 550, 504
    announce(f"backward with NaN/inf after every block: T {T} lens {LENS} causal seed {seed}")
    g = synth.rng(seed)
    q = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (sum(LENS), Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (sum(LENS), Hkv, D), 0.5, "bf16")
    do = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    qd, dod = H.to_device(q), H.to_device(do)
    order = [3, 2, 1, 0]
    kw = dict(n_kv_heads=Hkv, q_pos0=q_pos0, causal=True)
    res = {}
    for poison in (True, False):
        blocks = blocks_of(k, v, LENS, poison)
        st = ba.new_state(T * Hq, D)
        ba.fwd_block(qd, blocks, order, st, reset=True, split_mode=1, **kw)
        out, lse = ba.finalize(st)
        delta = ba.bwd_delta(out, dod)
        dq = torch.zeros(T * Hq, D, dtype=torch.float32, device="cuda")
        dkv = [(torch.zeros(n, Hkv, D, dtype=torch.float32, device="cuda"),
                torch.zeros(n, Hkv, D, dtype=torch.float32, device="cuda")) for n in LENS]
        ba.bwd_block(qd, dod, lse, delta, blocks, order, dq, dkv, **kw)
        torch.cuda.synchronize()
        res[poison] = [dq] + [t for pair in dkv for t in pair]
    for t in res[True]:
        assert bool(torch.isfinite(t).all()), "non-finite gradient"
    for a, b in zip(res[True], res[False]):
        assert torch.equal(a, b), "trailing NaN/inf rows changed a gradient"
    # and the gradients are the oracle's
    dq_ref, dk_ref, dv_ref = ora.attention_grads(q.f64(), k.f64(), v.f64(), do.f64(), 1.0 / np.sqrt(D),
                                                 q_pos0 + np.arange(T), None, True)
    got_dq = H.host(res[True][0]).reshape(T, Hq, D)
    err = np.abs(got_dq - dq_ref).max() / np.abs(dq_ref).max()
    got_dk = np.concatenate([H.host(res[True][1 + 2 * i]) for i in range(len(LENS))], axis=0)
    got_dv = np.concatenate([H.host(res[True][2 + 2 * i]) for i in range(len(LENS))], axis=0)
    err_k = np.abs(got_dk - dk_ref).max() / np.abs(dk_ref).max()
    err_v = np.abs(got_dv - dv_ref).max() / np.abs(dv_ref).max()
    print(f"    dq {err:.2e} dk {err_k:.2e} dv {err_v:.2e} (max err / max |ref|)", flush=True)
    assert max(err, err_k, err_v) <= 2e-2


@pytest.mark.parametrize("T", [1, 5])
def test_fanout_ignores_trailing_rows(T):
    nb, Hq, Hkv, D, P, S, seed = 3, 16, 2, 128, 1000, 100, 505
    announce(f"fan-out with NaN/inf after the prefix and the suffixes: T {T} nb {nb} P {P} S {S} seed {seed}")
    g = synth.rng(seed)
    q = synth.normal(g, (nb, T, Hq, D), 0.5, "bf16")
    pk = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    pv = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    sk = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    sv = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    qd = H.to_device(q)
    res = {}
    for poison in (True, False):
        pkd, = with_tails(pk, [P], poison)
        pvd, = with_tails(pv, [P], poison)
        flat = lambda t: synth.Tensor(t.storage.reshape((nb * S,) + t.shape[2:]), t.dtype)
        skd, = with_tails(flat(sk), [nb * S], poison)
        svd, = with_tails(flat(sv), [nb * S], poison)
        skd, svd = skd.view(nb, S, Hkv, D), svd.view(nb, S, Hkv, D)
        if T == 1:
            out, lse = ba.fanout_prefix_decode(qd[:, 0].contiguous(), pkd, pvd, skd, svd)
        else:
            out, lse = ba.fanout_prefix_prefill(qd, pkd, pvd, skd, svd)
        torch.cuda.synchronize()
        res[poison] = (out.reshape(nb, T, Hq, D), lse.reshape(nb, T, Hq))
    a_ref, lse_ref = ora.fanout_prefill(q.f64(), pk.f64(), pv.f64(), sk.f64(), sv.f64(), 1.0 / np.sqrt(D))
    H.assert_bf16_out(H.host(res[True][0]), a_ref, "fan-out")
    H.assert_close(H.host(res[True][1]), lse_ref, H.BF16_LSE, "fan-out lse")
    assert torch.equal(res[True][0], res[False][0]) and torch.equal(res[True][1], res[False][1])
