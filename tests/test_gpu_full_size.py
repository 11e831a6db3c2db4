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


def check_grad(got, ref, what):
    """Gradient error judged against the gradient's own scale, as in the
    small-size backward tests: max error <= 2e-2 of max |ref|, mean error <=
    5e-3 of mean |ref| (bf16 rounding of P, dS and A gives about 2e-3)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    mx = float(err.max()) / max(float(np.abs(ref).max()), 1e-30)
    mn = float(err.mean()) / max(float(np.abs(ref).mean()), 1e-30)
    print(f"    {what}: max err / max|ref| {mx:.2e}, mean err / mean|ref| {mn:.2e}", flush=True)
    assert mx <= 2e-2 and mn <= 5e-3, f"{what}: {mx:.3e} / {mn:.3e}"


def blockwise_device(w):
    q, k, v = w.make_inputs()
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    blocks = [(kd[b * w.block_len:(b + 1) * w.block_len], vd[b * w.block_len:(b + 1) * w.block_len],
               b * w.block_len) for b in range(w.n_blocks)]
    return q, k, v, qd, blocks


def oracle_rows(w, q, k, v, tokens):
    """The oracle's output and LSE for every query head of ``tokens``."""
    from exact_blockwise_long_amd import synth
    q64 = synth.Tensor(q.storage[tokens], q.dtype).f64()
    visible_end = min(w.kv_len, w.q_pos0 + w.q_len) if w.causal else w.kv_len  # later keys are never visible
    k64 = synth.Tensor(k.storage[:visible_end], k.dtype).f64()
    v64 = synth.Tensor(v.storage[:visible_end], v.dtype).f64()
    a_ref, _, _, lse_ref = ora.attend(q64, k64, v64, w.scale, w.q_pos0 + tokens, None, w.causal)
    return a_ref, lse_ref


class PrefillRun:
    """The 32K causal prefill in the benchmark's configuration, run once: the
    output and LSE of every row on the host."""
    out = lse = None


@pytest.fixture(scope="module")
def prefill_run():
    w = wl.CAUSAL_PREFILL
    announce(f"{w.name}: one fwd_block_finalize call over every visit (the benchmark's step)")
    q, k, v, qd, blocks = blockwise_device(w)
    st = ba.new_state(w.rows, w.head_dim)
    out, lse = ba.fwd_block_finalize(qd, blocks, w.order, st, reset=True, n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0,
                                     causal=w.causal)
    torch.cuda.synchronize()
    r = PrefillRun()
    r.q, r.k, r.v = q, k, v
    r.out = H.host(out).reshape(w.q_len, w.n_q_heads, w.head_dim)
    r.lse = H.host(lse).reshape(w.q_len, w.n_q_heads)
    del qd, blocks, st, out, lse
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(r.out)) and np.all(np.isfinite(r.lse)), "non-finite output or LSE"
    return r


@pytest.mark.parametrize("part", range(8))
def test_causal_prefill_full_size_every_row(prefill_run, part):
    """Every row of the 32K causal prefill against the oracle, an eighth of the
    query tokens (all 64 heads) per case so each stays well inside its time limit."""
    w = wl.CAUSAL_PREFILL
    n = w.q_len // 8
    tokens = np.arange(part * n, (part + 1) * n)
    announce(f"{w.name}: every head of tokens {tokens[0]}..{tokens[-1]} against the oracle")
    a_ref, lse_ref = oracle_rows(w, prefill_run.q, prefill_run.k, prefill_run.v, tokens)
    stats = H.assert_bf16_out(prefill_run.out[tokens], a_ref, w.name)
    H.assert_close(prefill_run.lse[tokens], lse_ref, H.BF16_LSE, "lse")
    print(f"    {len(tokens)} tokens x {w.n_q_heads} heads: max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}",
          flush=True)


def test_causal_prefill_fwd_block_then_finalize_full_size():
    """The same visits through fwd_block (fp32 state in HBM) and then finalize,
    on sampled tokens."""
    w = wl.CAUSAL_PREFILL
    announce(f"{w.name}: fwd_block then finalize")
    q, k, v, qd, blocks = blockwise_device(w)
    st = ba.new_state(w.rows, w.head_dim)
    ba.fwd_block(qd, blocks, w.order, st, reset=True, n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0, causal=w.causal)
    out, lse = ba.finalize(st)
    torch.cuda.synchronize()
    tokens = sample_tokens(w.q_len, w.block_len, 2, 21)
    a_ref, lse_ref = oracle_rows(w, q, k, v, tokens)
    got = H.host(out).reshape(w.q_len, w.n_q_heads, w.head_dim)
    assert np.all(np.isfinite(got)), "non-finite output"
    stats = H.assert_bf16_out(got[tokens], a_ref, w.name)
    H.assert_close(H.host(lse).reshape(w.q_len, w.n_q_heads)[tokens], lse_ref, H.BF16_LSE, "lse")
    print(f"    sampled {len(tokens)} tokens: max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}", flush=True)


def ring_share_tokens(w, seed, n_total=32):
    """Query tokens of the 256K ring share checked against the oracle, every
    query head of each (so every head is covered): the first and last token,
    the edges of the walk's 256-row tiles (32 tokens each), and the tokens
    where the diagonal block's 128-key tiles begin and end, then seeded random
    tokens up to n_total."""
    fixed = [0, 31, 32, 127, 128, 255, 256, w.q_len // 2 - 1, w.q_len // 2, w.q_len - 129, w.q_len - 128,
             w.q_len - 33, w.q_len - 32, w.q_len - 1]
    g = np.random.Generator(np.random.PCG64(seed))
    rest = [t for t in g.permutation(w.q_len).tolist() if t not in fixed]
    return np.array(sorted(fixed + rest[:n_total - len(fixed)]))


def test_ring_share_full_size_one_call_per_visit():
    """As the benchmark runs it: one call per visit of a block with visible
    keys, the last of them finalising (blocks 13-15 lie in the causal future
    and get no call).  2048 (token, head) rows are checked against the oracle:
    32 tokens x all 64 heads, including the first and last token and the tile
    edges (sampled parity); every row's output and LSE must be finite."""
    w = wl.RING_SHARE
    announce(w.name)
    q, k, v, qd, blocks = blockwise_device(w)
    st = ba.new_state(w.rows, w.head_dim)
    vis = w.visited_nonempty()
    for i, j in enumerate(vis):
        kw = dict(reset=(i == 0), n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0, causal=w.causal)
        if i < len(vis) - 1:
            ba.fwd_block(qd, blocks, [j], st, **kw)
        else:
            out, lse = ba.fwd_block_finalize(qd, blocks, [j], st, **kw)
    torch.cuda.synchronize()
    del blocks, qd, st
    got = H.host(out).reshape(w.q_len, w.n_q_heads, w.head_dim)
    got_lse = H.host(lse).reshape(w.q_len, w.n_q_heads)
    del out, lse
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got_lse)), "non-finite output or LSE"
    tokens = ring_share_tokens(w, 3)
    assert len(tokens) * w.n_q_heads == 2048
    a_ref, lse_ref = oracle_rows(w, q, k, v, tokens)
    stats = H.assert_bf16_out(got[tokens], a_ref, w.name)
    H.assert_close(got_lse[tokens], lse_ref, H.BF16_LSE, "lse")
    print(f"    {len(tokens)} tokens x {w.n_q_heads} heads = 2048 rows: max/mean abs err "
          f"{stats[0]:.2e}/{stats[1]:.2e}", flush=True)


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


def test_fanout_decode_paged_full_size():
    """The 64K fan-out decode with its prefix and private suffixes scattered
    over a page pool (256-token pages, seeded random order): bit for bit the
    contiguous entry point's result (checked on every row above), and two
    branches against the paged definition directly."""
    w = wl.FANOUT_DECODE
    PL = 256
    announce(f"{w.name}, paged: page_len {PL}, pages in random pool order (seed {w.seed + 500})")
    q, pk, pv, sk, sv = w.make_inputs()
    g = np.random.Generator(np.random.PCG64(w.seed + 500))
    n_pool, pp, sp = wl.paged_layout(g, w.n_branches, w.prefix_len, w.suffix_len, PL)
    k_pool = wl.scatter_pages(g, pk, sk, n_pool, pp, sp, PL)
    v_pool = wl.scatter_pages(g, pv, sv, n_pool, pp, sp, PL)
    qd = H.to_device(q)
    out, lse = ba.fanout_prefix_decode_paged(qd, H.to_device(k_pool), H.to_device(v_pool),
                                             torch.from_numpy(pp).cuda(), torch.from_numpy(sp).cuda(),
                                             w.prefix_len, w.suffix_len)
    o2, l2 = ba.fanout_prefix_decode(qd, *[H.to_device(t) for t in (pk, pv, sk, sv)])
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2), "paged differs from contiguous"
    b = [0, w.n_branches - 1]
    a_ref, lse_ref = ora.fanout_paged(q.f64()[b][:, None], k_pool.f64(), v_pool.f64(), pp, sp[b], PL,
                                      w.prefix_len, w.suffix_len, w.scale)
    stats = H.assert_bf16_out(H.host(out)[b], a_ref[:, 0], "paged fanout")
    H.assert_close(H.host(lse)[b], lse_ref[:, 0], H.BF16_LSE, "paged fanout lse")
    print(f"    branches {b}: max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}; all rows equal the contiguous call",
          flush=True)


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
    # The same 1,048,576 keys as ONE block of one call (the split planner cuts
    # it into key chunks), finalised in the same call.
    st = ba.new_state(w.rows, w.head_dim)
    out1, lse1 = ba.fwd_block_finalize(qd, [(kd, vd, 0)], [0], st, reset=True, n_kv_heads=1)
    torch.cuda.synchronize()
    stats = H.assert_bf16_out(H.host(out1).reshape(a_ref.shape), a_ref, w.name + " one block")
    H.assert_close(H.host(lse1).reshape(lse_ref.shape), lse_ref, H.BF16_LSE, "one-block lse")
    print(f"    one 1M-key block, fused finalisation: max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}", flush=True)


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


def test_backward_full_size_sampled():
    """The backward of the causal prefill workload in the configuration the
    benchmark times (one bwd_block call over the forward's visits).  Checked:
    dQ on sampled tokens; dK and dV of the last keys, which only the last few
    tokens see, so the oracle can take every row that reaches them; and two
    identities over all 32768 keys of each KV head: sum_j dV_j = sum_i dO_i
    (each softmax row sums to 1) and sum_j dK_j = 0 (each row of dS sums to
    0, as sum_j P_ij dP_ij = D_i)."""
    w = wl.CAUSAL_PREFILL
    announce(f"backward full size: {w.name}, seed {w.seed} (dO seed {w.seed + 1000})")
    q, k, v, qd, blocks = blockwise_device(w)
    do = w.make_dout()
    dod = H.to_device(do)
    st = ba.new_state(w.rows, w.head_dim)
    ba.fwd_block(qd, blocks, w.order, st, reset=True, n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0, causal=w.causal)
    out, lse = ba.finalize(st)
    del st
    delta = ba.bwd_delta(out, dod)
    L = w.block_len
    dq = torch.zeros(w.rows, w.head_dim, dtype=torch.float32, device="cuda")
    dkv = [(torch.zeros(L, w.n_kv_heads, w.head_dim, dtype=torch.float32, device="cuda"),
            torch.zeros(L, w.n_kv_heads, w.head_dim, dtype=torch.float32, device="cuda")) for _ in blocks]
    ba.bwd_block(qd, dod, lse, delta, blocks, w.order, dq, dkv, n_kv_heads=w.n_kv_heads, q_pos0=w.q_pos0,
                 causal=w.causal)
    torch.cuda.synchronize()
    dq_g = H.host(dq).reshape(w.q_len, w.n_q_heads, w.head_dim)
    dk_g = np.concatenate([H.host(a) for a, _ in dkv])
    dv_g = np.concatenate([H.host(b) for _, b in dkv])
    del dq, dkv
    assert np.all(np.isfinite(dq_g)) and np.all(np.isfinite(dk_g)) and np.all(np.isfinite(dv_g))
    q64, k64, v64, do64 = q.f64(), k.f64(), v.f64(), do.f64()

    tokens = sample_tokens(w.q_len, w.block_len, 51, 6)
    rq, _, _ = ora.attention_grads(q64[tokens], k64, v64, do64[tokens], w.scale, w.q_pos0 + tokens, None, True)
    check_grad(dq_g[tokens], rq, f"dQ on {len(tokens)} sampled tokens")

    last = w.q_pos0 + w.q_len - 1
    keys = np.array([last - 20, last - 7, last - 1, last])
    sub = np.arange(keys.min() - w.q_pos0, w.q_len)
    _, rk, rv = ora.attention_grads(q64[sub], k64, v64, do64[sub], w.scale, w.q_pos0 + sub, None, True,
                                    key_subset=keys)
    check_grad(dk_g[keys], rk[keys], f"dK of keys {keys.tolist()}")
    check_grad(dv_g[keys], rv[keys], f"dV of keys {keys.tolist()}")

    G = w.n_q_heads // w.n_kv_heads
    do_g = do64.reshape(w.q_len, w.n_kv_heads, G, w.head_dim)
    want = do_g.sum(axis=(0, 2))
    got = dv_g.sum(axis=0)
    tol = 1e-2 * np.sqrt((do_g ** 2).sum(axis=(0, 2)))
    print(f"    sum_j dV_j vs sum_i dO_i: worst {np.max(np.abs(got - want) / tol):.3f} of the tolerance", flush=True)
    assert np.all(np.abs(got - want) <= tol)
    # sum_j dK_j cancels to zero exactly, so what is left is the rounding of
    # dS to bf16 (the MFMA operand), summed over 32768 keys: a CPU emulation of
    # the kernels' rounding points puts it at up to about 1 % of the norm of
    # the keys' dK at this size.  5 % still fails a missing or doubled block
    # (a block carries about a third of the norm).  The norm is that of the
    # output, whose magnitudes the sampled keys above pin.
    ksum = dk_g.sum(axis=0)
    tol_k = 5e-2 * np.sqrt((dk_g ** 2).sum(axis=0))
    print(f"    sum_j dK_j vs 0: worst {np.max(np.abs(ksum) / tol_k):.3f} of the tolerance", flush=True)
    assert np.all(np.abs(ksum) <= tol_k)
