"""Seeded random configurations against the CPU fp64 oracle: block counts,
lengths (empty and one-key blocks included), visit orders, query positions
(rows before every key, rows past every key), causal or not, group sizes,
head dims and split modes, for the forward walk (also ending in the fused
forward-and-finalise call), the backward and the fan-out.  Each configuration is drawn from its own seed, printed before it
touches the GPU, and small enough for the oracle to finish in a second."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_blockwise_long_amd import blockattn as ba
from exact_blockwise_long_amd import synth
from exact_blockwise_long_amd import workloads as wl
from oracle import attention as ora
from tests import helpers as H
from tests.test_gpu_parity import check_state_vs_oracle, make_case, run_fwd

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


def draw(seed):
    g = np.random.Generator(np.random.PCG64(seed))
    D = int(g.choice([64, 128]))
    Hkv = int(g.choice([1, 2, 4, 8]))
    G = int(g.choice([1, 2, 4, 8, 16]))
    while Hkv * G > 64:
        G //= 2
    n_blocks = int(g.integers(1, 7))
    lens = [int(x) for x in g.choice([0, 1, 2, 31, 63, 64, 65, 100, 128, 129, 200, 257], size=n_blocks)]
    if sum(lens) == 0:
        lens[0] = 17
    L = sum(lens)
    T = int(g.choice([1, 2, 17, 64, 65, 130, 300]))
    causal = bool(g.integers(0, 2))
    q_pos0 = int(g.integers(-T // 2, L + 40)) if causal else 0
    q_pos0 = max(q_pos0, 0)
    order = g.permutation(n_blocks).tolist()
    split_mode = int(g.integers(0, 3))
    per_visit = bool(g.integers(0, 2))
    return dict(D=D, Hkv=Hkv, Hq=Hkv * G, lens=lens, T=T, causal=causal, q_pos0=q_pos0, order=order,
                split_mode=split_mode, per_visit=per_visit)


@pytest.mark.parametrize("seed", range(1000, 1064))
def test_random_forward(seed):
    c = draw(seed)
    announce(f"random forward seed {seed}: {c}")
    q, k, v = make_case(seed, c["T"], c["Hq"], c["Hkv"], c["D"], c["lens"])
    st = run_fwd(q, k, v, c["lens"], c["order"], Hkv=c["Hkv"], q_pos0=c["q_pos0"], causal=c["causal"],
                 split_mode=c["split_mode"], per_visit=c["per_visit"])
    check_state_vs_oracle(st, q, k, v, c["q_pos0"], c["causal"], what=f"random seed {seed}")


def draw_long(seed):
    """Longer draws than draw(): query blocks of 257-1024 tokens against blocks
    of up to 1000 keys (several row and key tiles, the wide workgroups, key
    splits across many chunks), every fifth seed on the fp32 path at sizes its
    vector-ALU kernels finish quickly."""
    g = np.random.Generator(np.random.PCG64(seed))
    D = int(g.choice([64, 128]))
    Hkv = int(g.choice([1, 2, 4, 8]))
    G = int(g.choice([1, 2, 4, 8, 16]))
    while Hkv * G > 64:
        G //= 2
    f32 = seed % 5 == 0
    n_blocks = int(g.integers(1, 7))
    pool = [0, 1, 31, 127, 128, 129, 255, 256, 300] if f32 else [0, 1, 127, 128, 255, 256, 300, 511, 513, 1000]
    lens = [int(x) for x in g.choice(pool, size=n_blocks)]
    if sum(lens) == 0:
        lens[0] = 33
    L = sum(lens)
    T = int(g.choice([17, 65, 130] if f32 else [257, 511, 700, 1024]))
    causal = bool(g.integers(0, 2))
    q_pos0 = max(int(g.integers(-T // 2, L + 40)), 0) if causal else 0
    return dict(D=D, Hkv=Hkv, Hq=Hkv * G, lens=lens, T=T, causal=causal, q_pos0=q_pos0,
                order=g.permutation(n_blocks).tolist(), split_mode=int(g.integers(0, 3)),
                per_visit=bool(g.integers(0, 2)), f32=f32)


@pytest.mark.parametrize("seed", range(6000, 6048))
def test_random_forward_long(seed):
    c = draw_long(seed)
    announce(f"random long forward seed {seed}: {c}")
    q, k, v = make_case(seed, c["T"], c["Hq"], c["Hkv"], c["D"], c["lens"], dtype="f32" if c["f32"] else "bf16")
    st = run_fwd(q, k, v, c["lens"], c["order"], Hkv=c["Hkv"], q_pos0=c["q_pos0"], causal=c["causal"],
                 split_mode=c["split_mode"], per_visit=c["per_visit"])
    check_state_vs_oracle(st, q, k, v, c["q_pos0"], c["causal"], bf16=not c["f32"], what=f"random long seed {seed}")


@pytest.mark.parametrize("seed", range(2000, 2032))
def test_random_backward(seed):
    c = draw(seed)
    announce(f"random backward seed {seed}: {c}")
    T, Hq, Hkv, D, lens = c["T"], c["Hq"], c["Hkv"], c["D"], c["lens"]
    g = synth.rng(seed)
    L = sum(lens)
    q = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    k = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    v = synth.normal(g, (L, Hkv, D), 0.5, "bf16")
    do = synth.normal(g, (T, Hq, D), 0.5, "bf16")
    qd, kd, vd, dod = (H.to_device(x) for x in (q, k, v, do))
    blocks, off = [], 0
    for n in lens:
        blocks.append((kd[off:off + n], vd[off:off + n], off))
        off += n
    st = ba.new_state(T * Hq, D)
    ba.fwd_block(qd, blocks, c["order"], st, reset=True, n_kv_heads=Hkv, q_pos0=c["q_pos0"], causal=c["causal"],
                 split_mode=c["split_mode"])
    out, lse = ba.finalize(st)
    delta = ba.bwd_delta(out, dod.reshape(T * Hq, D))
    dq = torch.zeros(T * Hq, D, dtype=torch.float32, device="cuda")
    dkv = [(torch.zeros(n, Hkv, D, dtype=torch.float32, device="cuda"),
            torch.zeros(n, Hkv, D, dtype=torch.float32, device="cuda")) for n in lens]
    visits = [[j] for j in reversed(c["order"])] if c["per_visit"] else [c["order"]]
    for vis in visits:
        ba.bwd_block(qd, dod, lse, delta, blocks, vis, dq, dkv, n_kv_heads=Hkv, q_pos0=c["q_pos0"],
                     causal=c["causal"])
    torch.cuda.synchronize()
    rq, rk, rv = ora.attention_grads(q.f64(), k.f64(), v.f64(), do.f64(), 1.0 / np.sqrt(D),
                                     c["q_pos0"] + np.arange(T), None, c["causal"])
    got = (H.host(dq).reshape(T, Hq, D), np.concatenate([H.host(a) for a, _ in dkv]),
           np.concatenate([H.host(b) for _, b in dkv]))
    # When every row sees a single key, P = 1 and dS = dP - D cancels to zero
    # exactly; the kernels form dP and D in different fp32 orders, so what is
    # left is rounding of terms of size |dO| |V| sqrt(D) (times scale |K| or
    # |Q| for dK, dQ).  A zero reference is judged against that size.
    s = 1.0 / np.sqrt(D)
    term = np.abs(do.f64()).max() * np.abs(v.f64()).max() * np.sqrt(D) * s * max(np.abs(k.f64()).max(),
                                                                                 np.abs(q.f64()).max())
    for x, ref, name in zip(got, (rq, rk, rv), ("dQ", "dK", "dV")):
        assert np.all(np.isfinite(x)), f"{name} not finite"
        scale_max = np.abs(ref).max()
        if scale_max == 0:
            assert np.abs(x).max() <= 1e-5 * term, f"{name} should cancel to zero: {np.abs(x).max():.3e}"
            continue
        err = np.abs(x - ref)
        mx, mn = err.max() / scale_max, err.mean() / max(np.abs(ref).mean(), 1e-30)
        print(f"    {name}: {mx:.2e} / {mn:.2e}", flush=True)
        assert mx <= 2e-2 and mn <= 5e-3, f"random backward seed {seed} {name}: {mx:.3e} / {mn:.3e}"


@pytest.mark.parametrize("seed", range(3000, 3024))
def test_random_fanout(seed):
    g = np.random.Generator(np.random.PCG64(seed))
    D = int(g.choice([64, 128]))
    Hkv = int(g.choice([1, 2, 8]))
    Hq = Hkv * int(g.choice([1, 4, 8]))
    nb = int(g.choice([1, 3, 16, 40]))
    T = int(g.choice([1, 1, 5, 20]))
    S = int(g.choice([T, T + 3, 100, 512])) if T > 1 else int(g.choice([1, 40, 512]))
    P = int(g.choice([0, 64, 1000, 5000]))
    announce(f"random fanout seed {seed}: nb={nb} T={T} Hq={Hq} Hkv={Hkv} D={D} P={P} S={S}")
    gs = synth.rng(seed)
    q = synth.normal(gs, (nb, T, Hq, D), 0.5, "bf16")
    pk = synth.normal(gs, (P, Hkv, D), 0.5, "bf16")
    pv = synth.normal(gs, (P, Hkv, D), 0.5, "bf16")
    sk = synth.normal(gs, (nb, S, Hkv, D), 0.5, "bf16")
    sv = synth.normal(gs, (nb, S, Hkv, D), 0.5, "bf16")
    dev = [H.to_device(t) if t.storage.size else None for t in (pk, pv, sk, sv)]
    qd = H.to_device(q)
    if T == 1:
        out, lse = ba.fanout_prefix_decode(qd[:, 0].contiguous(), *dev)
        out, lse = out[:, None], lse[:, None]
    else:
        out, lse = ba.fanout_prefix_prefill(qd, *dev)
    torch.cuda.synchronize()
    a_ref, lse_ref = ora.fanout_prefill(q.f64(), pk.f64(), pv.f64(), sk.f64(), sv.f64(), 1.0 / np.sqrt(D))
    stats = H.assert_bf16_out(H.host(out), a_ref, f"random fanout seed {seed}")
    H.assert_close(H.host(lse), lse_ref, H.BF16_LSE, "lse")
    print(f"    max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}", flush=True)
    # the same inputs through a page pool: bit for bit the contiguous result
    PL = int(g.choice([64, 128, 256]))
    n_pool, pp, sp = wl.paged_layout(g, nb, P, S, PL)
    kd = H.to_device(wl.scatter_pages(g, pk, sk, n_pool, pp, sp, PL))
    vd = H.to_device(wl.scatter_pages(g, pv, sv, n_pool, pp, sp, PL))
    ppd = torch.from_numpy(pp).cuda() if P else None
    spd = torch.from_numpy(sp).cuda()
    if T == 1:
        o2, l2 = ba.fanout_prefix_decode_paged(qd[:, 0].contiguous(), kd, vd, ppd, spd, P, S)
        o2, l2 = o2[:, None], l2[:, None]
    else:
        o2, l2 = ba.fanout_prefix_prefill_paged(qd, kd, vd, ppd, spd, P, S)
    torch.cuda.synchronize()
    if nb * T * (Hq // Hkv) <= 128 or PL % 128 == 0:
        # the same key tiles as the contiguous call (wide launches take 128-key
        # prefix tiles, which 64-key pages would split): bit for bit
        assert torch.equal(out, o2) and torch.equal(lse, l2), f"paged (page_len {PL}) differs from contiguous"
    else:
        H.assert_bf16_out(H.host(o2), a_ref, f"random fanout seed {seed}, paged (page_len {PL})")
        H.assert_close(H.host(l2), lse_ref, H.BF16_LSE, "paged lse")


@pytest.mark.parametrize("seed", range(4000, 4016))
def test_random_shards_then_merge(seed):
    """One partial state per block (shard_states), the n-way merge, finalize:
    equal to attention over all the blocks' keys."""
    c = draw(seed)
    announce(f"random shards seed {seed}: {c}")
    T, Hq, Hkv, D, lens = c["T"], c["Hq"], c["Hkv"], c["D"], c["lens"]
    q, k, v = make_case(seed, T, Hq, Hkv, D, lens)
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    blocks, off = [], 0
    for n in lens:
        blocks.append((kd[off:off + n], vd[off:off + n], off))
        off += n
    states = [ba.new_state(T * Hq, D) for _ in lens]
    ba.shard_states(qd, blocks, states, n_kv_heads=Hkv, q_pos0=c["q_pos0"], causal=c["causal"])
    merged = ba.new_state(T * Hq, D)
    ba.merge_states(states, merged)
    check_state_vs_oracle(merged, q, k, v, c["q_pos0"], c["causal"], what=f"random shards seed {seed}")


@pytest.mark.parametrize("seed", range(5000, 5032))
def test_random_fused_finalize(seed):
    """The visits of a random configuration ending in blockattn_fwd_block_finalize:
    all in one call, or (per_visit) one fwd_block call per visit with the last
    visit's call finalising; output in bf16 or fp32."""
    c = draw(seed)
    out_dtype = torch.float32 if seed % 3 == 0 else torch.bfloat16
    announce(f"random fused finalize seed {seed}: {c} out {out_dtype}")
    T, Hq, Hkv, D = c["T"], c["Hq"], c["Hkv"], c["D"]
    q, k, v = make_case(seed, T, Hq, Hkv, D, c["lens"])
    qd, kd, vd = H.to_device(q), H.to_device(k), H.to_device(v)
    blocks, off = [], 0
    for n in c["lens"]:
        blocks.append((kd[off:off + n], vd[off:off + n], off))
        off += n
    kw = dict(n_kv_heads=Hkv, q_pos0=c["q_pos0"], causal=c["causal"], split_mode=c["split_mode"])
    st = ba.new_state(T * Hq, D)
    order = c["order"]
    if c["per_visit"]:
        for i, j in enumerate(order[:-1]):
            ba.fwd_block(qd, blocks, [j], st, reset=(i == 0), **kw)
        out, lse = ba.fwd_block_finalize(qd, blocks, order[-1:], st, reset=(len(order) == 1), out_dtype=out_dtype,
                                         **kw)
    else:
        out, lse = ba.fwd_block_finalize(qd, blocks, order, st, reset=True, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    a_ref, _, _, lse_ref = ora.attend(q.f64(), k.f64(), v.f64(), 1.0 / np.sqrt(D), c["q_pos0"] + np.arange(T),
                                      None, c["causal"])
    got = H.host(out).reshape(T, Hq, D)
    stats = H.assert_bf16_out(got, a_ref, f"random fused seed {seed}")
    H.assert_close(H.host(lse).reshape(T, Hq), lse_ref, H.BF16_LSE, f"random fused seed {seed} lse")
    print(f"    max/mean abs err {stats[0]:.2e}/{stats[1]:.2e}", flush=True)
