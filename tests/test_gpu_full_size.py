"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, checked on sampled rows the oracle computes one by one (and
on every row where the oracle is cheap enough)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_blockwise_long_amd import blockattn as ba
from exact_blockwise_long_amd import workloads as wl
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
    torch.cuda.empty_cache()


def sample_tokens(T, block_len, seed, n_random):
    g = np.random.Generator(np.random.PCG64(seed))
    fixed = [0, 1, 63, 64, 127, 128, block_len // 2, T - 129, T - 128, T - 2, T - 1]
    rnd = g.choice(T, size=n_random, replace=False).tolist()
    return np.array(sorted(set(t for t in fixed + rnd if 0 <= t < T)))


def blockwise_device(w):
    q, k, v = w.make_inputs()
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    blocks = [(kd[b * w.block_len:(b + 1) * w.block_len], vd[b * w.block_len:(b + 1) * w.block_len],
               b * w.block_len) for b in range(w.n_blocks)]
    return q, k, v, qd, blocks


def check_sampled(w, q, k, v, out, lse, tokens):
    q_rows = q.storage[tokens]
    from exact_blockwise_long_amd import synth
    q64 = synth.Tensor(q_rows, q.dtype).f64()
    visible_end = min(w.kv_len, w.q_pos0 + w.q_len)  # keys past the block's last query never matter
    k64 = synth.Tensor(k.storage[:visible_end], k.dtype).f64()
    v64 = synth.Tensor(v.storage[:visible_end], v.dtype).f64()
    a_ref, m_ref, l_ref, lse_ref = ora.attend(q64, k64, v64, w.scale, w.q_pos0 + tokens, None, w.causal)
    got = H.host(out).reshape(w.q_len, w.n_q_heads, w.head_dim)[tokens]
    stats = H.assert_bf16_out(got, a_ref, w.name)
    H.assert_close(H.host(lse).reshape(w.q_len, w.n_q_heads)[tokens], lse_ref, H.BF16_LSE, "lse")
    print(f"    sampled {len(tokens)} tokens x {w.n_q_heads} heads: max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}",
          flush=True)


def test_causal_prefill_full_size():
    w = wl.CAUSAL_PREFILL
    announce(w.name)
    q, k, v, qd, blocks = blockwise_device(w)
    st = ba.new_state(w.rows, w.head_dim)
    ba.fwd_block(qd, blocks, w.order, st, reset=True, n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0,
                 causal=w.causal)
    out, lse = ba.finalize(st)
    torch.cuda.synchronize()
    check_sampled(w, q, k, v, out, lse, sample_tokens(w.q_len, w.block_len, 2, 21))


def test_ring_share_full_size_one_call_per_visit():
    w = wl.RING_SHARE
    announce(w.name)
    q, k, v, qd, blocks = blockwise_device(w)
    st = ba.new_state(w.rows, w.head_dim)
    for i, j in enumerate(w.order):
        ba.fwd_block(qd, blocks, [j], st, reset=(i == 0), n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0,
                     causal=w.causal)
    out, lse = ba.finalize(st)
    torch.cuda.synchronize()
    del blocks, qd
    check_sampled(w, q, k, v, out, lse, sample_tokens(w.q_len, w.block_len, 3, 9))


def test_fanout_decode_full_size_all_rows():
    w = wl.FANOUT_DECODE
    announce(w.name)
    ins = w.make_inputs()
    dev = [H.to_device(t) for t in ins]
    out, lse = ba.fanout_prefix_decode(*dev)
    torch.cuda.synchronize()
    a_ref, lse_ref = ora.fanout_decode(*[t.f64() for t in ins], w.scale)
    stats = H.assert_bf16_out(H.host(out), a_ref, w.name)
    H.assert_close(H.host(lse), lse_ref, H.BF16_LSE, "fanout lse")
    print(f"    all {w.rows} rows: max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}", flush=True)


def test_shard_merge_full_size_all_rows():
    w = wl.SHARD_MERGE
    announce(w.name)
    q, k, v = w.make_inputs()
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    sl = w.shard_len
    blocks = [(kd[i * sl:(i + 1) * sl], vd[i * sl:(i + 1) * sl], i * sl) for i in range(w.n_shards)]
    states = [ba.new_state(w.rows, w.head_dim) for _ in range(w.n_shards)]
    ba.shard_states(qd, blocks, states, n_kv_heads=1)
    merged = ba.new_state(w.rows, w.head_dim)
    ba.merge_states(states, merged)
    out, lse = ba.finalize(merged)
    torch.cuda.synchronize()
    a_ref, m_ref, l_ref, lse_ref = ora.attend(q.f64(), k.f64(), v.f64(), w.scale)
    logits_span = float(np.abs(m_ref).max())
    stats = H.assert_bf16_out(H.host(out).reshape(a_ref.shape), a_ref, w.name)
    H.assert_close(H.host(lse).reshape(lse_ref.shape), lse_ref, H.BF16_LSE, "shard lse")
    H.assert_close(H.host(merged[0]).reshape(m_ref.shape), m_ref, H.BF16_M * max(1.0, logits_span / 4), "shard m")
    print(f"    all {w.rows} rows, max |m| {logits_span:.1f}: max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}",
          flush=True)


def test_fanout_prefill_full_size_all_rows():
    w = wl.FANOUT_PREFILL
    announce(w.name)
    ins = w.make_inputs()
    dev = [H.to_device(t) for t in ins]
    out, lse = ba.fanout_prefix_prefill(*dev)
    torch.cuda.synchronize()
    a_ref, lse_ref = ora.fanout_prefill(*[t.f64() for t in ins], 1.0 / np.sqrt(w.head_dim))
    stats = H.assert_bf16_out(H.host(out), a_ref, w.name)
    H.assert_close(H.host(lse), lse_ref, H.BF16_LSE, "fanout prefill lse")
    print(f"    all {w.n_branches * w.n_new * w.n_q_heads} rows: max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}",
          flush=True)
