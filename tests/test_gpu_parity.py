"""GPU parity of the HIP path (through the C ABI) against the CPU fp64 oracle.

Sizes here finish in seconds on the oracle while spanning several 128-row
tiles, several 64-key tiles and ragged tails.  Full-size workloads are in
test_gpu_full_size.py.  Every case prints its name, shape and seed before it
touches the GPU.
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


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ba.load()
    yield
    torch.cuda.synchronize()


def make_case(seed, T, Hq, Hkv, D, lens, dtype="bf16", kscale=0.5, qscale=0.5, vscale=0.5):
    g = synth.rng(seed)
    L = sum(lens)
    q = synth.normal(g, (T, Hq, D), qscale, dtype)
    k = synth.normal(g, (L, Hkv, D), kscale, dtype)
    v = synth.normal(g, (L, Hkv, D), vscale, dtype)
    return q, k, v


def device_blocks(k, v, lens, pos0=0):
    kd, vd = H.to_device(k), H.to_device(v)
    blocks, off = [], 0
    for n in lens:
        blocks.append((kd[off:off + n], vd[off:off + n], pos0 + off))
        off += n
    return blocks


def oracle_final(q, k, v, q_pos0, causal, scale, lens_visited_mask=None):
    T = q.shape[0]
    q_pos = q_pos0 + np.arange(T)
    a, m, l, lse = ora.attend(q.f64(), k.f64(), v.f64(), scale, q_pos, None, causal)
    return a, m, l, lse


def run_fwd(q, k, v, lens, order, *, Hkv, q_pos0, causal, split_mode, per_visit=False, reset_first=True):
    qd = H.to_device(q)
    blocks = device_blocks(k, v, lens)
    T, Hq, D = q.shape
    st = ba.new_state(T * Hq, D)
    if per_visit:
        for i, j in enumerate(order):
            ba.fwd_block(qd, blocks, [j], st, reset=(i == 0 and reset_first), n_kv_heads=Hkv, q_pos0=q_pos0,
                         causal=causal, split_mode=split_mode)
    else:
        ba.fwd_block(qd, blocks, order, st, reset=True, n_kv_heads=Hkv, q_pos0=q_pos0, causal=causal,
                     split_mode=split_mode)
    return st


def check_state_vs_oracle(st, q, k, v, q_pos0, causal, bf16=True, what=""):
    T, Hq, D = q.shape
    scale = 1.0 / np.sqrt(D)
    a_ref, m_ref, l_ref, lse_ref = oracle_final(q, k, v, q_pos0, causal, scale)
    out, lse = ba.finalize(st, torch.bfloat16 if bf16 else torch.float32)
    torch.cuda.synchronize()
    got = H.host(out).reshape(T, Hq, D)
    m = H.host(st[0]).reshape(T, Hq)
    l = H.host(st[1]).reshape(T, Hq)
    lse_g = H.host(lse).reshape(T, Hq)
    if bf16:
        stats = H.assert_bf16_out(got, a_ref, what)
        H.assert_close(m, m_ref, H.BF16_M, what + " m")
        H.assert_close(lse_g, lse_ref, H.BF16_LSE, what + " lse")
        H.assert_close(l, l_ref, H.BF16_LREL, what + " l", rel=True)
    else:
        H.assert_close(got, a_ref, H.F32_TOL, what + " out")
        H.assert_close(m, m_ref, H.F32_TOL, what + " m")
        H.assert_close(lse_g, lse_ref, H.F32_TOL, what + " lse")
        H.assert_close(l, l_ref, H.F32_TOL, what + " l", rel=True)
        stats = H.err_stats(got, a_ref)
    print(f"    {what}: max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}", flush=True)


# ---------------------------------------------------------------- fp32 path

def test_f32_tiny_exact_workload():
    w = wl.TINY_EXACT
    announce(f"f32 {w.name}")
    q, k, v = w.make_inputs()
    lens = [w.block_len] * w.n_blocks
    st = run_fwd(q, k, v, lens, w.order, Hkv=1, q_pos0=w.q_pos0, causal=False, split_mode=0)
    check_state_vs_oracle(st, q, k, v, w.q_pos0, False, bf16=False, what="tiny_exact f32")


@pytest.mark.parametrize("causal", [False, True])
def test_f32_gqa_ragged(causal):
    announce(f"f32 GQA 4/2 D128 T=70 lens 33,64,50 causal={causal} seed 11")
    lens = [33, 64, 50]
    q, k, v = make_case(11, 70, 4, 2, 128, lens, dtype="f32", qscale=1.0, kscale=1.0, vscale=1.0)
    st = run_fwd(q, k, v, lens, [2, 0, 1], Hkv=2, q_pos0=60, causal=causal, split_mode=0)
    check_state_vs_oracle(st, q, k, v, 60, causal, bf16=False, what="f32 gqa")


@pytest.mark.parametrize("causal", [False, True])
def test_f32_key_split_matches_walk_and_oracle(causal):
    """The fp32 key split (chunks walked in parallel, partial states merged)
    against the fp32 walk and the oracle, with a caller state carried in."""
    lens = [200, 77, 129]
    announce(f"f32 key split GQA 8/2 D64 T=90 lens {lens} causal={causal} seed 12")
    q, k, v = make_case(12, 90, 8, 2, 64, lens, dtype="f32", qscale=1.0, kscale=1.0, vscale=1.0)
    qd = H.to_device(q)
    blocks = device_blocks(k, v, lens)
    kw = dict(n_kv_heads=2, q_pos0=300, causal=causal)
    assert ba.fwd_workspace_bytes(qd, blocks, None, split_mode=0, **kw) > 0   # small: splits by itself
    outs = {}
    for mode in (1, 2):
        st = ba.new_state(90 * 8, 64)
        ba.fwd_block(qd, blocks, [2], st, reset=True, split_mode=mode, **kw)      # one visit, then the rest
        ba.fwd_block(qd, blocks, [0, 1], st, reset=False, split_mode=mode, **kw)
        torch.cuda.synchronize()
        check_state_vs_oracle(st, q, k, v, 300, causal, bf16=False, what=f"f32 split_mode {mode}")
        outs[mode] = ba.finalize(st, torch.float32)
    torch.cuda.synchronize()
    H.assert_close(H.host(outs[2][0]), H.host(outs[1][0]), 1e-6, "split vs walk output")
    H.assert_close(H.host(outs[2][1]), H.host(outs[1][1]), 1e-6, "split vs walk lse")


def test_f32_shard_states_and_merge():
    lens = [96, 130, 64]
    announce(f"f32 shard states D128 T=40 Hq 4 Hkv 1 lens {lens} seed 13")
    q, k, v = make_case(13, 40, 4, 1, 128, lens, dtype="f32", qscale=1.0, kscale=1.0, vscale=1.0)
    qd = H.to_device(q)
    blocks = device_blocks(k, v, lens)
    states = [ba.new_state(40 * 4, 128) for _ in lens]
    ba.shard_states(qd, blocks, states, n_kv_heads=1)
    merged = ba.new_state(40 * 4, 128)
    ba.merge_states(states, merged)
    torch.cuda.synchronize()
    check_state_vs_oracle(merged, q, k, v, 0, False, bf16=False, what="f32 shards merged")


# ---------------------------------------------------------------- bf16 path

BF16_CASES = [
    # (seed, T, Hq, Hkv, D, lens, order, q_pos0, causal)
    (21, 300, 8, 2, 128, [200, 77, 129, 64], [2, 0, 3, 1], 350, True),
    (22, 300, 8, 2, 128, [200, 77, 129, 64], [3, 2, 1, 0], 0, False),
    (23, 130, 4, 4, 64, [65, 128, 31], [1, 2, 0], 150, True),
    (24, 17, 16, 1, 128, [513, 1000], [1, 0], 1400, True),
]


@pytest.mark.parametrize("split_mode", [1, 2])
@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: f"seed{c[0]}")
def test_bf16_walk_and_split(case, split_mode):
    seed, T, Hq, Hkv, D, lens, order, q_pos0, causal = case
    announce(f"bf16 seed {seed} T={T} Hq={Hq} Hkv={Hkv} D={D} lens={lens} order={order} causal={causal} "
             f"split_mode={split_mode}")
    q, k, v = make_case(seed, T, Hq, Hkv, D, lens)
    st = run_fwd(q, k, v, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=causal, split_mode=split_mode)
    check_state_vs_oracle(st, q, k, v, q_pos0, causal, what=f"bf16 seed{seed} mode{split_mode}")


def test_bf16_one_call_per_visit_and_checkpoint():
    """One call per ring step == one call for the walk; a state round trip through host memory is bitwise."""
    seed, T, Hq, Hkv, D, lens, order, q_pos0, causal = BF16_CASES[0]
    announce(f"bf16 per-visit seed {seed} order={order}")
    q, k, v = make_case(seed, T, Hq, Hkv, D, lens)
    st = run_fwd(q, k, v, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=causal, split_mode=1, per_visit=True)
    check_state_vs_oracle(st, q, k, v, q_pos0, causal, what="per-visit")
    # interrupted walk: 2 visits, copy the state to the host and back, then the rest
    qd = H.to_device(q)
    blocks = device_blocks(k, v, lens)
    st2 = ba.new_state(T * Hq, D)
    for i, j in enumerate(order[:2]):
        ba.fwd_block(qd, blocks, [j], st2, reset=(i == 0), n_kv_heads=Hkv, q_pos0=q_pos0, causal=causal,
                     split_mode=1)
    saved = [x.cpu().numpy().copy() for x in st2]
    st3 = tuple(torch.from_numpy(x).cuda() for x in saved)
    for j in order[2:]:
        ba.fwd_block(qd, blocks, [j], st3, reset=False, n_kv_heads=Hkv, q_pos0=q_pos0, causal=causal,
                     split_mode=1)
    torch.cuda.synchronize()
    for a, b in zip(st, st3):
        assert torch.equal(a, b), "resumed walk differs from the uninterrupted one"


def test_bf16_order_invariance():
    seed, T, Hq, Hkv, D, lens, _, q_pos0, causal = BF16_CASES[1]
    announce(f"bf16 order invariance seed {seed}")
    q, k, v = make_case(seed, T, Hq, Hkv, D, lens)
    outs = []
    for order in ([0, 1, 2, 3], [3, 2, 1, 0], [1, 3, 0, 2]):
        st = run_fwd(q, k, v, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=causal, split_mode=1)
        check_state_vs_oracle(st, q, k, v, q_pos0, causal, what=f"order {order}")
        outs.append(H.host(ba.finalize(st)[0]))
    for o in outs[1:]:
        mx, _ = H.err_stats(o, outs[0])
        assert mx <= H.BF16_MAX


def test_bf16_deterministic():
    seed, T, Hq, Hkv, D, lens, order, q_pos0, causal = BF16_CASES[0]
    announce(f"bf16 determinism seed {seed}")
    q, k, v = make_case(seed, T, Hq, Hkv, D, lens)
    for mode in (1, 2):
        a = run_fwd(q, k, v, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=causal, split_mode=mode)
        b = run_fwd(q, k, v, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=causal, split_mode=mode)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_bf16_causal_future_keys_ignored():
    """Changing every key/value no query can see leaves the state bitwise unchanged."""
    seed, T, Hq, Hkv, D = 31, 100, 8, 2, 128
    lens = [128, 128]
    announce(f"bf16 causal future perturbation seed {seed}")
    q, k, v = make_case(seed, T, Hq, Hkv, D, lens)
    q_pos0 = 120  # queries at 120..219: keys 220..255 are in everyone's future
    st_a = run_fwd(q, k, v, lens, [1, 0], Hkv=Hkv, q_pos0=q_pos0, causal=True, split_mode=1)
    k2 = synth.Tensor(k.storage.copy(), "bf16")
    v2 = synth.Tensor(v.storage.copy(), "bf16")
    g = synth.rng(99)
    k2.storage[220:] = synth.normal(g, k2.storage[220:].shape, 5.0, "bf16").storage
    v2.storage[220:] = synth.normal(g, v2.storage[220:].shape, 5.0, "bf16").storage
    st_b = run_fwd(q, k2, v2, lens, [1, 0], Hkv=Hkv, q_pos0=q_pos0, causal=True, split_mode=1)
    torch.cuda.synchronize()
    for x, y in zip(st_a, st_b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("split_mode", [1, 2])
@pytest.mark.parametrize("D", [64, 128])
def test_bf16_row_without_keys_in_first_tile(split_mode, D):
    """The first visited block is wholly in the future for the first rows of a
    row tile and visible to the tile's later rows: the first rows' reference
    max stays -inf through a tile in which other rows of the wave move theirs
    (regression: their rescale factor was exp2(-inf - -inf) = NaN)."""
    seed, T, Hq, Hkv, lens, order, q_pos0 = 84, 70, 8, 2, [100, 37], [1, 0], 67
    announce(f"bf16 first tile masked for some rows: D={D} lens={lens} order={order} q_pos0={q_pos0} "
             f"split_mode={split_mode} seed {seed}")
    q, k, v = make_case(seed, T, Hq, Hkv, D, lens)
    st = run_fwd(q, k, v, lens, order, Hkv=Hkv, q_pos0=q_pos0, causal=True, split_mode=split_mode)
    check_state_vs_oracle(st, q, k, v, q_pos0, True, what=f"first tile masked D{D} mode{split_mode}")


def test_empty_and_degenerate():
    announce("degenerate: q_len 0, no visits with reset, all keys in the future")
    q, k, v = make_case(41, 40, 8, 2, 128, [64])
    qd = H.to_device(q)
    blocks = device_blocks(k, v, [64], pos0=1000)
    st = ba.new_state(40 * 8, 128)
    # reset with zero visits -> initial state
    ba.fwd_block(qd, blocks, [], st, reset=True, n_kv_heads=2, causal=True, split_mode=1)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(st[0])) and torch.all(st[1] == 0) and torch.all(st[2] == 0)
    # every key after every query -> the state stays initial, finalize gives 0 and -inf
    for mode in (1, 2):
        ba.fwd_block(qd, blocks, [0], st, reset=True, n_kv_heads=2, q_pos0=0, causal=True, split_mode=mode)
        out, lse = ba.finalize(st)
        torch.cuda.synchronize()
        assert torch.all(torch.isneginf(st[0])) and torch.all(st[1] == 0)
        assert torch.all(out.float() == 0) and torch.all(torch.isneginf(lse))
    # q_len 0 is a no-op
    ba.fwd_block(qd[:0], blocks, [0], st, reset=True, n_kv_heads=2, split_mode=1)


# ---------------------------------------------------------------- merge and finalize

def test_merge_of_oracle_partials_f32():
    """GPU merge of fp32 oracle partials == oracle merge (fp32 rounding only)."""
    announce("merge of oracle partials, 5 parts incl. an empty one, logits ~ +-30")
    g = np.random.Generator(np.random.PCG64(51))
    T, Hq, D, L = 50, 4, 128, 400
    q = g.standard_normal((T, Hq, D))
    k = g.standard_normal((L, 1, D)) * 6.0
    v = g.standard_normal((L, 1, D))
    s = 1.0 / np.sqrt(D)
    labels = g.integers(0, 4, size=L)
    parts = [ora.state(q, k, v, s, key_subset=np.flatnonzero(labels == p)) for p in range(4)]
    parts.append(ora.init_state(T, Hq, D))
    mr, lr, orr = ora.merge(parts)
    dev = [tuple(torch.from_numpy(np.ascontiguousarray(x.reshape(-1, D) if x.ndim == 3 else x.reshape(-1),
                                                       dtype=np.float32)).cuda() for x in p) for p in parts]
    out = ba.new_state(T * Hq, D)
    ba.merge_states(dev, out)
    torch.cuda.synchronize()
    H.assert_close(H.host(out[0]), mr.reshape(-1), 1e-5, "merge m")
    H.assert_close(H.host(out[1]), lr.reshape(-1), 1e-5, "merge l", rel=True)
    H.assert_close(H.host(out[2]) / H.host(out[1])[:, None], (orr / lr[..., None]).reshape(-1, D), 1e-5,
                   "merge O/l")
    # in place into part 0
    ba.merge_states(dev, dev[0])
    torch.cuda.synchronize()
    for x, y in zip(dev[0], out):
        assert torch.equal(x, y)


def test_finalize_values():
    announce("finalize: empty rows and fp32/bf16 outputs")
    m = torch.tensor([-float("inf"), 0.5, 3.0], device="cuda")
    l = torch.tensor([0.0, 2.0, 0.25], device="cuda")
    o = torch.arange(3 * 64, dtype=torch.float32, device="cuda").reshape(3, 64) / 7.0
    o[0] = 0
    out32, lse = ba.finalize((m, l, o), torch.float32)
    out16, _ = ba.finalize((m, l, o), torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.all(out32[0] == 0) and torch.isneginf(lse[0])
    H.assert_close(H.host(out32[1:]), H.host(o[1:]) / H.host(l[1:])[:, None], 1e-6, "finalize", rel=True)
    H.assert_close(H.host(lse[1:]), [0.5 + np.log(2.0), 3.0 + np.log(0.25)], 1e-6, "lse")
    assert torch.equal(out16, out32.to(torch.bfloat16))


# ---------------------------------------------------------------- shards + merge (sharded sequence)

def test_shard_states_then_merge():
    announce("shard_states: 8 branches x 8 heads, 4 shards x 1500 keys, K x12 (logits ~ +-30)")
    nb, G, D, n_sh, sl = 8, 8, 128, 4, 1500
    g = synth.rng(61)
    q = synth.normal(g, (nb, G, D), 0.5, "bf16")
    k = synth.normal(g, (n_sh * sl, 1, D), 12.0, "bf16")
    v = synth.normal(g, (n_sh * sl, 1, D), 0.5, "bf16")
    qd = H.to_device(q)
    blocks = device_blocks(k, v, [sl] * n_sh)
    states = [ba.new_state(nb * G, D) for _ in range(n_sh)]
    ba.shard_states(qd, blocks, states, n_kv_heads=1)
    s = 1.0 / np.sqrt(D)
    # each shard against the oracle
    for i in range(n_sh):
        mi, li, oi = ora.state(q.f64(), k.f64()[i * sl:(i + 1) * sl], v.f64()[i * sl:(i + 1) * sl], s)
        torch.cuda.synchronize()
        H.assert_close(H.host(states[i][0]), mi.reshape(-1), H.BF16_M, f"shard {i} m")
        H.assert_bf16_out(H.host(states[i][2]) / H.host(states[i][1])[:, None], (oi / li[..., None]).reshape(-1, D),
                          f"shard {i} O/l")
    out = ba.new_state(nb * G, D)
    ba.merge_states(states, out)
    a, lse = ba.finalize(out)
    torch.cuda.synchronize()
    a_ref, _, _, lse_ref = ora.attend(q.f64(), k.f64(), v.f64(), s)
    H.assert_bf16_out(H.host(a).reshape(nb, G, D), a_ref, "sharded merge")
    H.assert_close(H.host(lse).reshape(nb, G), lse_ref, H.BF16_LSE, "sharded lse")


# ---------------------------------------------------------------- fan-out decode

# The last case plans two branches per suffix job with a ragged last group
# (131 branches) and two row tiles per KV head (G = 1).
@pytest.mark.parametrize("nb,Hq,Hkv,D,P,S", [(3, 8, 2, 128, 1000, 37), (3, 8, 2, 128, 0, 70), (3, 8, 2, 128, 333, 0),
                                             (3, 8, 2, 128, 4096, 512), (131, 8, 8, 64, 100, 40)])
def test_fanout_small(nb, Hq, Hkv, D, P, S):
    announce(f"fanout nb={nb} Hq={Hq} Hkv={Hkv} D={D} P={P} S={S} seed 71")
    g = synth.rng(71)
    q = synth.normal(g, (nb, Hq, D), 0.5, "bf16")
    pk = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    pv = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    sk = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    sv = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    dev = [H.to_device(t) if t.storage.size else None for t in (q, pk, pv, sk, sv)]
    out, lse = ba.fanout_prefix_decode(*dev)
    torch.cuda.synchronize()
    a_ref, lse_ref = ora.fanout_decode(q.f64(), pk.f64(), pv.f64(), sk.f64(), sv.f64(), 1.0 / np.sqrt(D))
    H.assert_bf16_out(H.host(out), a_ref, "fanout")
    H.assert_close(H.host(lse), lse_ref, H.BF16_LSE, "fanout lse")


# ---------------------------------------------------------------- fan-out prefill

# (nb, T, Hq, Hkv, D, P, S): several new tokens per branch, causal in the suffix.
# 2 x 20 x 8 rows: 160 rows per branch and KV head (one 256-row tile of the
# wide launch, whose tiles span branches for the prefix); T = S: no
# older private tokens; P = 0: no prefix; the fifth case groups branches per
# job; the last is one branch (one 256-row tile per KV head, each K/V byte read
# by one workgroup).
@pytest.mark.parametrize("nb,T,Hq,Hkv,D,P,S", [(3, 5, 8, 2, 128, 1000, 37), (2, 20, 64, 8, 128, 700, 90),
                                               (4, 7, 8, 2, 64, 300, 7), (3, 9, 8, 2, 128, 0, 70),
                                               (42, 2, 4, 4, 64, 2000, 3), (1, 20, 64, 8, 128, 700, 90)])
def test_fanout_prefill(nb, T, Hq, Hkv, D, P, S):
    announce(f"fanout prefill nb={nb} T={T} Hq={Hq} Hkv={Hkv} D={D} P={P} S={S} seed 72")
    g = synth.rng(72)
    q = synth.normal(g, (nb, T, Hq, D), 0.5, "bf16")
    pk = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    pv = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    sk = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    sv = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    dev = [H.to_device(t) if t.storage.size else None for t in (q, pk, pv, sk, sv)]
    out, lse = ba.fanout_prefix_prefill(*dev)
    torch.cuda.synchronize()
    a_ref, lse_ref = ora.fanout_prefill(q.f64(), pk.f64(), pv.f64(), sk.f64(), sv.f64(), 1.0 / np.sqrt(D))
    H.assert_bf16_out(H.host(out), a_ref, "fanout prefill")
    H.assert_close(H.host(lse), lse_ref, H.BF16_LSE, "fanout prefill lse")


# ---------------------------------------------------------------- paged fan-out

# (seed, nb, T, Hq, Hkv, D, P, S, page_len, holes): T = 1 goes through the
# decode entry point, T > 1 through the prefill one.  Pages sit at random pool
# pages among poisoned pages; the last prefix page and suffix pages are
# partial.  holes lists (table, index) entries set to the hole marker -1.
PAGED_CASES = [
    (61, 3, 1, 8, 2, 128, 1000, 37, 64, []),
    (62, 2, 20, 64, 8, 128, 700, 90, 128, []),
    (63, 4, 7, 8, 2, 64, 300, 70, 256, [("prefix", 1), ("suffix", (2, 0))]),
    (64, 16, 1, 64, 8, 128, 4096, 512, 256, []),
    (65, 5, 3, 8, 2, 128, 0, 200, 64, []),
    # more than 128 rows per KV head (a wide launch) over 64-key pages: the prefix
    # jobs keep 64-key tiles there, while the contiguous call takes 128
    (66, 2, 20, 64, 8, 128, 700, 90, 64, []),
]


def paged_inputs(seed, nb, T, Hq, Hkv, D, P, S, PL):
    g = synth.rng(seed)
    q = synth.normal(g, (nb, T, Hq, D), 0.5, "bf16")
    pk = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    pv = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    sk = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    sv = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    n_pool, pp, sp = wl.paged_layout(g, nb, P, S, PL)
    k_pool = wl.scatter_pages(g, pk, sk, n_pool, pp, sp, PL)
    v_pool = wl.scatter_pages(g, pv, sv, n_pool, pp, sp, PL)
    return q, pk, pv, sk, sv, n_pool, pp, sp, k_pool, v_pool


@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: f"seed{c[0]}")
def test_fanout_paged(case):
    seed, nb, T, Hq, Hkv, D, P, S, PL, bad = case
    announce(f"paged fanout nb={nb} T={T} Hq={Hq} Hkv={Hkv} D={D} P={P} S={S} page_len={PL} holes={bad} "
             f"seed {seed}")
    q, pk, pv, sk, sv, n_pool, pp, sp, k_pool, v_pool = paged_inputs(seed, nb, T, Hq, Hkv, D, P, S, PL)
    for table, i in bad:
        if table == "prefix":
            pp[i] = -1
        else:
            sp[i] = -1
    kd, vd = H.to_device(k_pool), H.to_device(v_pool)
    ppd = torch.from_numpy(pp).cuda() if P else None
    spd = torch.from_numpy(sp).cuda() if S else None
    if T == 1:
        qd = H.to_device(q)[:, 0].contiguous()
        out, lse = ba.fanout_prefix_decode_paged(qd, kd, vd, ppd, spd, P, S)
        out, lse = out[:, None], lse[:, None]
    else:
        qd = H.to_device(q)
        out, lse = ba.fanout_prefix_prefill_paged(qd, kd, vd, ppd, spd, P, S)
    torch.cuda.synchronize()
    a_ref, lse_ref = ora.fanout_paged(q.f64(), k_pool.f64(), v_pool.f64(), pp, sp, PL, P, S, 1.0 / np.sqrt(D))
    H.assert_bf16_out(H.host(out), a_ref, "paged fanout")
    H.assert_close(H.host(lse), lse_ref, H.BF16_LSE, "paged fanout lse")
    wide = nb * T * (Hq // Hkv) > 128      # launches of more than one 128-row tile per KV head
    if not bad and (not wide or PL % 128 == 0):
        # the same tiles in the same order as the contiguous entry points: bit for bit
        dev = [H.to_device(t) if t.storage.size else None for t in (pk, pv, sk, sv)]
        if T == 1:
            o2, l2 = ba.fanout_prefix_decode(qd, *dev)
            o2, l2 = o2[:, None], l2[:, None]
        else:
            o2, l2 = ba.fanout_prefix_prefill(qd, *dev)
        torch.cuda.synchronize()
        assert torch.equal(out, o2) and torch.equal(lse, l2), "paged differs from contiguous"


@pytest.mark.parametrize("T", [1, 4])
def test_fanout_paged_corrupt_page_ids_give_nan_rows(T):
    """A page id that is neither a pool page nor the hole marker -1 cannot be
    checked on the host (the tables are device memory).  The rows whose keys
    it would name come out as NaN with LSE +inf -- a corrupt suffix page only
    its branch's rows, a corrupt prefix page every row -- and every other row
    is the oracle's."""
    seed, nb, Hq, Hkv, D, P, S, PL = 66, 4, 16, 2, 128, 700, 150, 64
    announce(f"paged fanout with corrupt page ids: nb={nb} T={T} P={P} S={S} page_len={PL} seed {seed}")
    q, pk, pv, sk, sv, n_pool, pp, sp, k_pool, v_pool = paged_inputs(seed, nb, T, Hq, Hkv, D, P, S, PL)
    kd, vd = H.to_device(k_pool), H.to_device(v_pool)
    qd = H.to_device(q)

    def run(ppt, spt):
        ppd, spd = torch.from_numpy(ppt).cuda(), torch.from_numpy(spt).cuda()
        if T == 1:
            o, l = ba.fanout_prefix_decode_paged(qd[:, 0].contiguous(), kd, vd, ppd, spd, P, S)
            o, l = o[:, None], l[:, None]
        else:
            o, l = ba.fanout_prefix_prefill_paged(qd, kd, vd, ppd, spd, P, S)
        torch.cuda.synchronize()
        return H.host(o), H.host(l)

    a_ref, lse_ref = ora.fanout_paged(q.f64(), k_pool.f64(), v_pool.f64(), pp, sp, PL, P, S, 1.0 / np.sqrt(D))
    # a corrupt suffix page of branch 2 (an id past the pool)
    sp_bad = sp.copy()
    sp_bad[2, 1] = n_pool + 3
    out, lse = run(pp, sp_bad)
    assert np.isnan(out[2]).all() and np.isposinf(lse[2]).all(), "branch 2's rows are not marked"
    others = [b for b in range(nb) if b != 2]
    H.assert_bf16_out(out[others], a_ref[others], "other branches")
    H.assert_close(lse[others], lse_ref[others], H.BF16_LSE, "other branches lse")
    # a corrupt prefix page (a negative id other than -1): every row
    pp_bad = pp.copy()
    pp_bad[3] = -7
    out, lse = run(pp_bad, sp)
    assert np.isnan(out).all() and np.isposinf(lse).all(), "rows of a corrupt prefix are not marked"


def test_fanout_prefill_one_token_is_the_decode():
    nb, Hq, Hkv, D, P, S = 5, 8, 2, 128, 900, 33
    announce(f"fanout prefill T=1 vs decode nb={nb} P={P} S={S} seed 74")
    g = synth.rng(74)
    q = synth.normal(g, (nb, 1, Hq, D), 0.5, "bf16")
    pk = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    pv = synth.normal(g, (P, Hkv, D), 0.5, "bf16")
    sk = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    sv = synth.normal(g, (nb, S, Hkv, D), 0.5, "bf16")
    qd, pkd, pvd, skd, svd = [H.to_device(t) for t in (q, pk, pv, sk, sv)]
    o1, l1 = ba.fanout_prefix_prefill(qd, pkd, pvd, skd, svd)
    o2, l2 = ba.fanout_prefix_decode(qd[:, 0].contiguous(), pkd, pvd, skd, svd)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 0], o2) and torch.equal(l1[:, 0], l2)
